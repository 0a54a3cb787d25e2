// Gradients of the block-sparse prefill attention with the kept blocks fixed
// (block selection is a top-k and has no gradient), bf16 inputs, float32
// accumulation, on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16); float32
// inputs take a vector-ALU kernel (bwd_f32_kernel, at the end).
// Sources: "MiniCPM 4.0" blog (shadowrocket9.top), InfLLM v2 section (the
// sparse attention is trainable: the model is trained with it); "MiniCPM4:
// running LLMs on phones and PCs" (xugj520.cn), section 1.1 (attention over
// the selected blocks only).  For one (query row, head) with weights
// p = softmax(scale * K q) over its kept keys and output o = p V, given the
// upstream gradient do:
//   dV_j += p_j do                  dP_j = do . v_j
//   dS_j  = p_j (dP_j - do . o)     dq = scale * sum_j dS_j k_j
//   dK_j += scale * dS_j q
// The backward recomputes p from the forward's log-sum-exp, so nothing of
// size keys x rows is stored.
//
// Kernels (in launch order):
//   bwd_dsum    per (row, head): lse * log2(e) and dsum = do . o (float32)
//   bwd_mark    bitmap[g][b] bit i set when row i kept block b for KV head g
//               (sparse chunks only): one workgroup per 32-row word column,
//               built in LDS and written whole; above 16384 blocks a fill
//               kernel clears the bitmap and global atomics set the bits
//   bwd_count   per (g, block): segments of at most kSegPairs (row, head)
//               pairs, so that block 0, which every row keeps, is spread over
//               many workgroups
//   bwd_plan    scans the segment counts into a list of work items (KV
//               head, 64-key chunk, segment), 1024 units per workgroup
//   bwd_dkdv    key-major: a workgroup of four waves owns one item; each wave
//               holds 16 keys of K and V as MFMA operands and their dK^T, dV^T
//               accumulators in registers (two waves per SIMD), and walks the
//               segment's rows 32 (row, head) pairs at a time through a
//               four-slot LDS ring filled by direct global->LDS copies:
//                 S = Q K^T, dP = dO V^T            (pairs x keys)
//                 P = exp(scale S - lse), dS = P (dP - dsum)
//                 dV^T += dO^T P, dK^T += Q^T dS    (reduction over pairs)
//               The two products over pairs take P and dS straight from the
//               accumulator registers (element e of the B operand is pair
//               4h+e or 16+4h+e-4, the order of lane h's accumulator rows;
//               the A operands dO^T and Q^T are read in the same order with
//               transposing LDS reads).  Results are added to float32 dK, dV
//               with atomics, since several segments may share a chunk.
//   bwd_dq      query-major, like the forward kernel: a workgroup owns the
//               (row, head) pairs of a tile of tokens and one KV head, walks
//               the union of the tokens' kept blocks (K and V tiles staged in
//               LDS by direct loads), and per 64-key chunk computes
//               S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
// float32 inputs: bwd_dsum, then bwd_f32 (one wave per (row, head)).
#include "lds_tiles.h"

namespace infllmv2 {

// Element pointers hold bfloat16 bits; the float32 kernels reinterpret them
// as float.
struct BwdArgs {
  const uint16_t* q;          // [n_q][h_q][D]
  const uint16_t* k;          // [h_kv][cap][D]
  const uint16_t* v;
  const int32_t* block_idx;   // [n_q][h_kv][topk], NULL when dense
  const uint16_t* out;        // forward output [n_q][h_q][D]
  const float* lse;           // forward log-sum-exp [n_q][h_q] (natural log)
  const uint16_t* d_out;      // upstream gradient [n_q][h_q][D]
  uint16_t* dq;               // [n_q][h_q][D]
  float* dk;                  // [h_kv][cap][D], accumulated
  float* dv;
  float* meta;                // workspace [n_q][h_q][2]: lse * log2(e), do . o
  uint32_t* bitmap;           // workspace [h_kv][n_b][nw]
  int32_t* nseg;              // workspace [h_kv][n_b]
  int2* items;                // workspace [max_items]: (g * n_chunks + chunk, segment)
  int32_t* n_items;           // workspace [1]
  int64_t cap, n_k;
  int n_q, h_q, h_kv, topk, B, n_b, nw, n_chunks, seg_rows, max_items, n_tiles;
  int dense;
  float scale, scale_log2;
};

// (row, head) pairs per dK/dV work item: bounds a workgroup's work.  Each
// item adds its partial dK/dV with float32 atomics, whose write traffic grows
// with the item count; smaller items balance better.  Measured on the 128K
// chunk (MI355X), first kernel: dK/dV 2.49 / 2.17 / 2.40 / 2.55 ms at 2048 /
// 4096 / 8192 / 16384 pairs; current kernel (rocprofv3 means, one box): 1.79 /
// 1.69 / 1.71 / 1.76 ms at 4096 / 5120 / 6144 / 7168 pairs; with whole-line
// atomics, 3072 / 4096 / 6144 pairs stayed within the run-to-run spread of
// 5120 (backward call 2.54-2.86 ms on one box).  Rows per item are capped so
// the row list stays at 8 KB of LDS.
constexpr int kSegPairs = 5120;
constexpr int kMaxSegRows = 2048;
__host__ __device__ constexpr int seg_rows_for(int G) {
  return kSegPairs / G < kMaxSegRows ? (kSegPairs / G > 0 ? kSegPairs / G : 1) : kMaxSegRows;
}
constexpr int kPlanThreads1 = 1024;

// ---------------------------------------------------------------------------
// meta[row][h] = (lse * log2 e, sum_d do[row][h][d] * o[row][h][d]); D/8
// lanes per pair.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BwdArgs a) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int L = D / E;
  const T* dO = reinterpret_cast<const T*>(a.d_out);
  const T* O = reinterpret_cast<const T*>(a.out);
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gid / L;
  const int part = (int)(gid % L);
  const int64_t n_pairs = (int64_t)a.n_q * a.h_q;
  float acc = 0.0f;
  if (pair < n_pairs) {
    float x[E], y[E];
    Elem<T>::unpack(ldg16(dO + pair * D + E * part), x);
    Elem<T>::unpack(ldg16(O + pair * D + E * part), y);
#pragma unroll
    for (int i = 0; i < E; ++i) acc = __builtin_fmaf(x[i], y[i], acc);
  }
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (pair < n_pairs && part == 0)
    *reinterpret_cast<float2*>(a.meta + 2 * pair) = make_float2(a.lse[pair] * kLog2e, acc);
}

__global__ __launch_bounds__(256) void bwd_fill_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// bit (row % 32) of bitmap[g][b][row / 32] <- row kept block b for KV head g
__global__ __launch_bounds__(256) void bwd_mark_kernel(BwdArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.n_q * a.h_kv * a.topk;
  if (gid >= total) return;
  const int row = (int)(gid / ((int64_t)a.h_kv * a.topk));
  const int g = (int)((gid / a.topk) % a.h_kv);
  const int32_t b = a.block_idx[gid];
  if (b < 0 || b >= a.n_b) return;
  atomicOr(a.bitmap + ((int64_t)g * a.n_b + b) * a.nw + (row >> 5), 1u << (row & 31));
}

// Bitmap column of one 32-row word w for KV head g (workgroup (w, g)): the
// rows' kept blocks are ORed into an LDS copy of the n_b words, which is then
// written whole, so the bitmap needs no clearing and no global atomics.
constexpr int kMarkLdsBlocks = 16384;          // n_b up to this: the LDS column
__global__ __launch_bounds__(256) void bwd_mark_lds_kernel(BwdArgs a) {
  extern __shared__ uint32_t col[];
  const int w = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  for (int b = tid; b < a.n_b; b += 256) col[b] = 0u;
  __syncthreads();
  const int r0 = 32 * w;
  const int n_e = min(32, a.n_q - r0) * a.topk;
  for (int e = tid; e < n_e; e += 256) {
    const int rr = e / a.topk, i = e - rr * a.topk;
    const int32_t b = a.block_idx[((int64_t)(r0 + rr) * a.h_kv + g) * a.topk + i];
    if (b >= 0 && b < a.n_b) atomicOr(&col[b], 1u << rr);
  }
  __syncthreads();
  uint32_t* out = a.bitmap + (int64_t)g * a.n_b * a.nw + w;
  for (int b = tid; b < a.n_b; b += 256) out[(int64_t)b * a.nw] = col[b];
}

// one wave per (g, block): rows that kept it -> segments of seg_rows rows
__global__ __launch_bounds__(256) void bwd_count_kernel(BwdArgs a) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= a.h_kv * a.n_b) return;
  const uint32_t* w = a.bitmap + (int64_t)e * a.nw;
  int c = 0;
  for (int i = lane; i < a.nw; i += 64) c += __popc(w[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
  if (lane == 0) a.nseg[e] = (c + a.seg_rows - 1) / a.seg_rows;
}

__device__ __forceinline__ int dense_first_row(const BwdArgs& a, int chunk) {
  // rows at positions >= the chunk's first key: row i sits at n_k - n_q + i
  const int64_t r0 = (int64_t)chunk * kChunk - (a.n_k - a.n_q);
  return r0 < 0 ? 0 : (int)(r0 < a.n_q ? r0 : a.n_q);
}

// Work items in (KV head, chunk, segment) order.  Workgroup w owns units
// [w NT, (w+1) NT): it sums the item counts of all earlier units (its base),
// scans its own, and writes their items; the last workgroup stores the total.
__device__ __forceinline__ void plan_unit(const BwdArgs& a, int e, int units, int total_e,
                                          int& nseg, int& nch, int& c0, int& g) {
  nseg = 0; nch = 0; c0 = 0; g = 0;
  if (e >= total_e) return;
  g = e / units;
  const int u = e % units;
  if (a.dense) {
    const int cnt = a.n_q - dense_first_row(a, u);
    nseg = (cnt + a.seg_rows - 1) / a.seg_rows;
    nch = 1;
    c0 = u;
  } else {
    nseg = a.nseg[e];
    c0 = u * (a.B / kChunk);
    nch = min(a.B / kChunk, a.n_chunks - c0);
  }
}

__global__ __launch_bounds__(kPlanThreads1) void bwd_plan_kernel(BwdArgs a) {
  constexpr int NT = kPlanThreads1;
  __shared__ int scan_lds[NT / 64];
  const int tid = threadIdx.x;
  const int units = a.dense ? a.n_chunks : a.n_b;
  const int total_e = a.h_kv * units;
  const int e0 = blockIdx.x * NT;
  int before = 0;
  for (int e = tid; e < e0; e += NT) {
    int nseg, nch, c0, g;
    plan_unit(a, e, units, total_e, nseg, nch, c0, g);
    before += nseg * nch;
  }
  int base;
  block_excl_scan<NT>(before, &base, scan_lds);              // base = sum over threads
  int nseg, nch, c0, g;
  plan_unit(a, e0 + tid, units, total_e, nseg, nch, c0, g);
  const int cnt_items = nseg * nch;
  int tot;
  const int off = base + block_excl_scan<NT>(cnt_items, &tot, scan_lds);
  for (int i = 0; i < cnt_items; ++i) {
    if (off + i >= a.max_items) break;
    a.items[off + i] = make_int2(g * a.n_chunks + c0 + i / nseg, i % nseg);
  }
  if (blockIdx.x == gridDim.x - 1 && tid == 0) a.n_items[0] = min(base + tot, a.max_items);
}

// ---------------------------------------------------------------------------
// dK / dV, key-major.  Tiles of 32 (row, head) pairs of the item's segment
// are staged as [pair][d] rows, logical 16-byte chunk c of row r at chunk
// c ^ f(r), and read twice: as rows (16-byte reads) and transposed (8-byte
// transposing reads), with the swizzle made for that pair of patterns.
// ---------------------------------------------------------------------------
template <int D>
struct PairTile {
  static constexpr int RB = 2 * D;                  // bytes per pair row
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int BYTES = 32 * RB;             // one tensor (Q or dO)
  __device__ static __forceinline__ int f(int r) { return Swz16RT<D, Swz16V<D>>::f(r); }
  // byte offset of logical chunk c of pair row r
  __device__ static __forceinline__ uint32_t at(int r, int c) {
    return (uint32_t)(r * RB + ((c ^ f(r)) * 16));
  }
};

// One 4-byte-per-lane copy global -> LDS (lane l lands at lds_addr + 4 l).
__device__ __forceinline__ void lds_dma4(uint32_t lds_addr, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// Staging ring of the dK/dV kernel: per slot the Q and dO tiles of 32 pairs
// and, per wave, its own copy of the 32 pairs' (lse * log2 e, dsum).  The Q
// tiles of all slots come first, then the dO tiles, then the metadata, so
// that every tile byte lies below 64 KiB: with the slot known at compile
// time, a fragment read is its lane's base register plus an immediate.
constexpr int kDkdvStages = 4;
template <int D, int NW, int NS>
struct DkdvRing {
  static constexpr int TB = PairTile<D>::BYTES;
  static constexpr int META = 32 * 8;
  static constexpr int BYTES = 2 * NS * TB + NS * NW * META;
  static constexpr int q(int slot) { return slot * TB; }
  static constexpr int o(int slot) { return (NS + slot) * TB; }
  static constexpr int meta(int slot, int wave) { return 2 * NS * TB + (slot * NW + wave) * META; }
  static_assert(2 * NS * TB <= 65536, "tile bytes within the immediate offset range");
  // 16-byte copies per tile (Q then dO), split evenly over the NW waves
  static constexpr int INSTR = 2 * 32 * PairTile<D>::CPR / 64;
  static constexpr int PER_WAVE = INSTR / NW;
  static constexpr int KL = PER_WAVE + 1;           // + the meta copy
  static_assert(INSTR % NW == 0, "copies per wave");
};

// KT: 16-key tiles per wave; the workgroup's 4 / KT waves cover 64 keys.
template <int D, int G, int KT>
__global__ __launch_bounds__(256 / KT) __attribute__((amdgpu_waves_per_eu(KT == 1 ? 2 : 1)))
void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 4 / KT, NT = NW * 64, NS = kDkdvStages;
  constexpr int NKS = D / 32, NDT = D / 16;
  constexpr int SEG_ROWS = seg_rows_for(G);
  using PT = PairTile<D>;
  using RG = DkdvRing<D, NW, NS>;
  constexpr int KL = RG::KL;
  static_assert(KL * (NS - 2) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t ring[RG::BYTES];
  __shared__ int rows_lds[SEG_ROWS];
  // row * h_q + g * G (the pair index of the row's head 0), when a segment
  // has few enough rows that the table costs no occupancy
  constexpr bool kPbase = SEG_ROWS <= 1024;
  __shared__ uint32_t pbase_lds[kPbase ? SEG_ROWS : 1];
  __shared__ int scan_lds[NT / 64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if ((int)blockIdx.x >= a.n_items[0]) return;
  const int2 item = a.items[blockIdx.x];
  const int g = item.x / a.n_chunks, chunk = item.x % a.n_chunks, seg = item.y;
  const int key0 = chunk * kChunk;

  // ---- the segment's rows, ascending, into rows_lds
  int n_rows;
  if (a.dense) {
    const int r0 = dense_first_row(a, chunk) + seg * SEG_ROWS;
    n_rows = min(SEG_ROWS, a.n_q - r0);
    for (int i = tid; i < n_rows; i += NT) rows_lds[i] = r0 + i;
  } else {
    const int b = key0 / a.B;
    const uint32_t* words = a.bitmap + ((int64_t)g * a.n_b + b) * a.nw;
    const int per = (a.nw + NT - 1) / NT;
    const int w0 = tid * per, w1 = min(w0 + per, a.nw);
    int c = 0;
    for (int w = w0; w < w1; ++w) c += __popc(words[w]);
    int total;
    const int base = block_excl_scan<NT>(c, &total, scan_lds);
    const int lo = seg * SEG_ROWS, hi = min(lo + SEG_ROWS, total);
    if (base < hi && base + c > lo) {
      int r = base;
      for (int w = w0; w < w1 && r < hi; ++w) {
        uint32_t m = words[w];
        while (m) {
          const int bit = __builtin_ctz(m);
          m &= m - 1u;
          if (r >= lo && r < hi) rows_lds[r - lo] = w * 32 + bit;
          ++r;
        }
      }
    }
    n_rows = max(0, hi - lo);
  }
  __syncthreads();
  if constexpr (kPbase) {
    for (int i = tid; i < n_rows; i += NT)
      pbase_lds[i] = (uint32_t)rows_lds[i] * (uint32_t)a.h_q + (uint32_t)(g * G);
    __syncthreads();
  }
  const int n_pairs = n_rows * G;
  const int n_tiles = __builtin_amdgcn_readfirstlane((n_pairs + 31) / 32);
  if (n_tiles <= 0) return;

  // ---- this wave's 16 KT keys of K and V as B operands (key j of tile kt in
  // lane column j, dims 32 ks + 8 h .. +8); keys past n_k repeat the last key
  const int jj = lane & 15, hh = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // the wave index as a scalar
  const int kw0 = key0 + 16 * KT * wave_u;
  bf16x8 kf[KT][NKS], vf[KT][NKS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = min(kw0 + 16 * kt + jj, (int)a.n_k - 1);
    const uint16_t* kr = a.k + ((int64_t)g * a.cap + key) * D + 8 * hh;
    const uint16_t* vr = a.v + ((int64_t)g * a.cap + key) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 wk = ldg16(kr + 32 * ks), wv = ldg16(vr + 32 * ks);
      kf[kt][ks] = *reinterpret_cast<const bf16x8*>(&wk);
      vf[kt][ks] = *reinterpret_cast<const bf16x8*>(&wv);
    }
  }
  f32x4 dk[KT][NDT], dv[KT][NDT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      dk[kt][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      dv[kt][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  // K and V have arrived before the direct copies start (the compiler's own
  // waits do not see those copies)
  __builtin_amdgcn_s_waitcnt(0x0f70);

  // ---- direct copies of tile t into slot `slot`.  Pairs past the segment
  // repeat its last pair (finite data, masked by position).  Byte offsets
  // are 32-bit: the host keeps n_q * h_q * D * 2 below 4 GiB.
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ring;
  // (row * h_q + head) of pair p (clamped to the segment), 32-bit: the host
  // keeps n_q * h_q * D * 2 below 4 GiB
  const uint32_t n_pairs_u = (uint32_t)n_pairs, hq_u = (uint32_t)a.h_q, hg = (uint32_t)(g * G);
  auto pair_index = [&](uint32_t p) -> uint32_t {
    p = min(p, n_pairs_u - 1u);
    if constexpr (kPbase) return pbase_lds[p / G] + p % G;
    else return __umul24((uint32_t)rows_lds[p / G], hq_u) + hg + p % G;
  };
  // per lane and copy: pair row r and logical chunk c do not depend on the tile
  uint32_t cp_r[RG::PER_WAVE], cp_c16[RG::PER_WAVE];
#pragma unroll
  for (int i = 0; i < RG::PER_WAVE; ++i) {
    const int s = (wave_u * RG::PER_WAVE + i) * 64 + lane;
    const int r = (s / PT::CPR) % 32, pc = s % PT::CPR;
    cp_r[i] = (uint32_t)r;
    cp_c16[i] = (uint32_t)(16 * (pc ^ PT::f(r)));
  }
  // With G >= 16 (and kPbase) a tile's 32 pairs lie in 32 / G <= 2 rows: both
  // row bases are read once per tile into scalars.  A copy instruction
  // covers 64 / CPR consecutive pair rows, all of one row (G is a multiple
  // of that count), so each copy takes its row base as a scalar and adds a
  // tile-independent per-lane part (its pair's head and chunk).  The meta
  // copy's lanes span both rows: they add the scalar distance between the
  // bases under a per-lane mask.  Pairs past the segment take the last row
  // (finite data, masked by position).
  constexpr bool kTwoRows = kPbase && G >= 16;
  static_assert(!kTwoRows || (32 / G <= 2 && G % (64 / PT::CPR) == 0),
                "a tile spans at most two rows; a copy stays in one");
  uint32_t cp_fix[RG::PER_WAVE];
#pragma unroll
  for (int i = 0; i < RG::PER_WAVE; ++i) cp_fix[i] = (cp_r[i] % G) * (uint32_t)(2 * D) + cp_c16[i];
  const uint32_t m_pair = (uint32_t)(lane >> 1);
  const uint32_t m_fix = (m_pair % G) * 8u + 4u * (uint32_t)(lane & 1);
  const uint32_t m_hi = m_pair / G != 0u ? ~0u : 0u;
  auto issue = [&](int t, int slot) {
    const uint32_t p0 = (uint32_t)t * 32u;
    uint32_t b0 = 0u, b1 = 0u;
    if constexpr (kTwoRows) {
      const int row0 = (int)(p0 / G), last = max(n_rows - 1, 0);
      b0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)pbase_lds[min(row0, last)]);
      b1 = 32 / G > 1
               ? (uint32_t)__builtin_amdgcn_readfirstlane((int)pbase_lds[min(row0 + 1, last)])
               : b0;
    }
#pragma unroll
    for (int i = 0; i < RG::PER_WAVE; ++i) {
      const int j = wave_u * RG::PER_WAVE + i;              // copy index in the tile
      // the 64 slots of copy j lie in one tensor (a tensor is 32 CPR slots)
      constexpr int kPerTensor = 32 * PT::CPR / 64;
      const bool is_q = j < kPerTensor;
      const uint32_t dst = ring0 + (uint32_t)(is_q ? RG::q(slot) + j * 1024
                                                   : RG::o(slot) + (j - kPerTensor) * 1024);
      uint32_t voff;
      if constexpr (kTwoRows) {
        const bool second = ((j * (64 / PT::CPR)) % 32) / G != 0;   // the same in every lane
        voff = (second ? b1 : b0) * (uint32_t)(2 * D) + cp_fix[i];
      } else
        voff = pair_index(p0 + cp_r[i]) * (uint32_t)(2 * D) + cp_c16[i];
      lds_dma16(dst, is_q ? (const void*)a.q : (const void*)a.d_out, voff);
    }
    uint32_t moff;
    if constexpr (kTwoRows)
      moff = b0 * 8u + (m_hi & ((b1 - b0) * 8u)) + m_fix;
    else
      moff = pair_index(p0 + m_pair) * 8u + 4u * (uint32_t)(lane & 1);
    lds_dma4(ring0 + (uint32_t)RG::meta(slot, wave_u), a.meta, moff);
  };

  // 16-byte row reads: lane (jj, hh) reads pair row 16 pt + jj, logical chunk
  // 4 ks + hh.  The chunk bits never overlap the row bits and f depends on the
  // row mod 16, so k-step ks is an XOR of 64 ks on one per-lane base and pair
  // tile pt adds 16 rows (an immediate offset).
  // Transposing reads (d-tile dt, half c): pair row 16 c + 4 hh + jj / 4,
  // d 16 dt + 4 (jj % 4): an XOR of 32 dt on one base, half c adds 16 rows.
  const uint32_t rd_base = (uint32_t)(jj * PT::RB + ((hh ^ PT::f(jj)) * 16));
  const int tr_row = 4 * hh + (jj >> 2), tr_q = jj & 3;
  const uint32_t tr_base =
      (uint32_t)(tr_row * PT::RB + (((tr_q >> 1) ^ PT::f(tr_row)) * 16) + 8 * (tr_q & 1));
  int key_lane[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) key_lane[kt] = kw0 + 16 * kt + jj;
  const int qoff = (int)(a.n_k - a.n_q);

  auto compute = [&](int t, auto slot_tag) {
    constexpr int S = decltype(slot_tag)::value;
    const uint32_t qb = ring0 + (uint32_t)RG::q(S);
    const uint32_t ob = ring0 + (uint32_t)RG::o(S);
    const float2* meta = reinterpret_cast<const float2*>(&ring[RG::meta(S, 0) + wave * RG::META]);
    f32x4 s[2][KT], dp[2][KT];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[pt][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        dp[pt][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const uint32_t ra = (rd_base ^ (uint32_t)(64 * ks)) + (uint32_t)(16 * pt * PT::RB);
        const bf16x8 aq = lds_read16(qb + ra);
        const bf16x8 ao = lds_read16(ob + ra);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          s[pt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kf[kt][ks], s[pt][kt], 0, 0, 0);
          dp[pt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, vf[kt][ks], dp[pt][kt], 0, 0, 0);
        }
      }
    // P and dS; lane (jj, hh) holds pairs 16 pt + 4 hh + r of key 16 kt + jj.
    // Pairs are in ascending row order: when the tile's first row already
    // sees the wave's last key and every pair is in the segment, no mask.
    bf16x8 pb[KT], sb[KT];
    const uint32_t tp0 = (uint32_t)(t * 32);
    const bool whole = tp0 + 31u < n_pairs_u &&
                       __builtin_amdgcn_readfirstlane(qoff + rows_lds[tp0 / G]) >=
                           kw0 + 16 * KT - 1;
    auto p_ds = [&](bool masked) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pr = 16 * pt + 4 * hh + r;
          const uint32_t p = tp0 + (uint32_t)pr;
          const float2 m = meta[pr];
          const int pos = masked ? (p < n_pairs_u ? qoff + rows_lds[p / G] : -1) : 0;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const float e = fast_exp2(__builtin_fmaf(s[pt][kt][r], a.scale_log2, -m.x));
            const float pv = !masked || key_lane[kt] <= pos ? e : 0.0f;
            pb[kt][4 * pt + r] = (__bf16)pv;
            sb[kt][4 * pt + r] = (__bf16)(pv * (dp[pt][kt][r] - m.y));
          }
        }
    };
    if (whole) p_ds(false);
    else p_ds(true);
    // dV^T += dO^T P, dK^T += Q^T dS: A rows d of d-tile dt, reduction over
    // pairs in the order 4 hh + e (e < 4), 16 + 4 hh + e - 4 (e >= 4)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint32_t lo = tr_base ^ (uint32_t)(32 * dt);
      const uint32_t hi = lo + (uint32_t)(16 * PT::RB);
      const bf16x4 o0 = lds_read_tr8(ob + lo), o1 = lds_read_tr8(ob + hi);
      const bf16x4 q0 = lds_read_tr8(qb + lo), q1 = lds_read_tr8(qb + hi);
      const bf16x8 aot = __builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 aqt = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        dv[kt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aot, pb[kt], dv[kt][dt], 0, 0, 0);
        dk[kt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aqt, sb[kt], dk[kt][dt], 0, 0, 0);
      }
    }
  };

  // Tile t sits in slot t % NS.  Iteration t: wait for tile t (the copies
  // issued after it, of tiles t+1 .. t+NS-2, may still be in flight), meet
  // (every wave has finished tile t-1, so its slot is free), copy tile
  // t+NS-1 into that slot, compute tile t.
#pragma unroll
  for (int j = 0; j + 1 < NS; ++j)
    if (j < n_tiles) issue(j, j);
  auto step = [&](int t, auto slot_tag) {
    constexpr int S = decltype(slot_tag)::value;
    const int after = min(NS - 2, n_tiles - 1 - t);
    if (after >= 2) wait_vm_barrier<2 * KL>();
    else if (after == 1) wait_vm_barrier<KL>();
    else wait_vm_barrier<0>();
    if (t + NS - 1 < n_tiles) issue(t + NS - 1, (S + NS - 1) % NS);
    compute(t, slot_tag);
  };
  static_assert(NS == 4, "the tile loop is unrolled over four slots");
  for (int t = 0; t < n_tiles; t += NS) {
    step(t, StageTag<0>());
    if (t + 1 < n_tiles) step(t + 1, StageTag<1>());
    if (t + 2 < n_tiles) step(t + 2, StageTag<2>());
    if (t + 3 < n_tiles) step(t + 3, StageTag<3>());
  }

  // ---- accumulate.  Lane (jj, hh) holds key 16 kt + jj, d = 16 dt + 4 hh + r:
  // added as they are, an atomic instruction would touch 16 lines with 4
  // scattered floats each.  The wave's tile goes through LDS instead (the
  // ring is free once every wave has left the tile loop), so that each
  // atomic instruction covers whole 64-byte lines: 16 lanes per key row,
  // 4 rows per instruction.  dK, then dV, through the same staging, whose
  // rows are padded to D + 16 floats so the 4 rows of a read fall in
  // disjoint banks.  LDS operations of one wave complete in order.
  constexpr int kRowF = D + 16;
  static_assert(NW * 16 * KT * kRowF * 4 <= RG::BYTES, "the staging fits in the ring");
  __syncthreads();
  float* stg = reinterpret_cast<float*>(ring) + wave_u * (16 * KT * kRowF);
  auto put = [&](const f32x4 (&acc)[KT][NDT], float mul) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4*>(&stg[(16 * kt + jj) * kRowF + 16 * dt + 4 * hh]) =
            acc[kt][dt] * mul;
    __builtin_amdgcn_wave_barrier();
  };
  auto add_to = [&](float* dst) {
    const int rl = lane >> 4, dl = lane & 15;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = 16 * kt + 4 * it + rl;
        const int key = kw0 + row;
        float* o = dst + ((int64_t)g * a.cap + (key < a.n_k ? key : 0)) * D + dl;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          const float x = stg[row * kRowF + 16 * i + dl];
          if (key < a.n_k) unsafeAtomicAdd(o + 16 * i, x);
        }
      }
    __builtin_amdgcn_wave_barrier();
  };
  put(dk, a.scale);
  add_to(a.dk);
  put(dv, 1.0f);
  add_to(a.dv);
}

// ---------------------------------------------------------------------------
// dQ, query-major.  W waves of 16 (row, head) pairs: pair p of the workgroup
// is token p / G, head p % G of KV group g.  K and V tiles serve 16-byte row
// reads (S^T and dP^T) and, for K, transposing reads (dQ^T = K^T dS^T): the
// swizzle made for that pair of patterns.
// ---------------------------------------------------------------------------
// Four waves per SIMD (128 VGPRs, no spills): two 8-wave workgroups share a
// CU, and each hides the other's staging and LDS waits (1.83 -> 1.26 ms on
// the 128K chunk against two waves per SIMD at 158 VGPRs).
template <int D, int G, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = W * 64;
  constexpr int TT = (16 * W) / G;                 // tokens per workgroup
  static_assert(TT >= 1 && TT <= 32, "token bitmask is 32 bits");
  constexpr int NKS = D / 32, NDT = D / 16;
  using SW = Swz16RT<D, Swz16K<D>>;
  constexpr int TILE = SW::TILE;
  constexpr int RB = SW::RB;
  constexpr int SORT_N = TT * kSortCap;
  // 256-byte aligned: the fragment addresses below XOR bits 5..7 of ring
  // addresses (slot bases are multiples of 256)
  __shared__ __attribute__((aligned(256))) uint16_t stage[2 * 2 * TILE / 2];   // K[2] V[2]
  __shared__ int2 ents[TT * kSortCap];
  __shared__ int scan_lds[NT / 64];
  static_assert(SORT_N * 4 <= (int)sizeof(stage), "sort buffer aliases the staging ring");

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wi = xcd_contiguous_index(blockIdx.x, gridDim.x);
  const int g = wi / a.n_tiles, tile = wi % a.n_tiles;
  const int n_keys = (int)a.n_k;
  const int tok0 = tile * TT;
  const int n_tok = min(TT, a.n_q - tok0);
  const bool dense = a.dense != 0;
  const int cpb = a.B / kChunk;
  const uint32_t full_mask = n_tok >= 32 ? 0xffffffffu : ((1u << n_tok) - 1u);
  const int p0 = (int)(a.n_k - a.n_q) + tok0;

  int n_entries;
  if (dense) {
    n_entries = (p0 + n_tok - 1) / a.B + 1;
  } else {
    int N = 1;
    while (N < TT * a.topk) N <<= 1;
    n_entries = build_union<NT, TT>(a.block_idx, tok0, a.h_kv, g, n_tok, a.topk, a.n_b,
                                    reinterpret_cast<uint32_t*>(stage), N, ents, scan_lds);
  }
  const int n = __builtin_amdgcn_readfirstlane(n_entries * cpb);

  struct Unit { int key0, nv; uint32_t tm; };
  auto unit_of = [&](int u) -> Unit {
    Unit r = {0, 0, 0u};
    if (u >= n) return r;
    const int e = u / cpb, c = u - e * cpb;
    int b;
    if (dense) {
      b = e;
      const int t_min = b * a.B - p0;
      r.tm = t_min <= 0 ? full_mask : (t_min >= 32 ? 0u : (full_mask & (0xffffffffu << t_min)));
    } else {
      const int2 en = ents[e];
      b = en.x;
      r.tm = (uint32_t)en.y;
    }
    r.key0 = b * a.B + c * kChunk;
    r.nv = max(0, min(kChunk, min((b + 1) * a.B, n_keys) - r.key0));
    return r;
  };

  // this lane's pair: column jj of the wave's 16
  const int jj = lane & 15, hh = lane >> 4;
  const int pw = 16 * wave + jj;
  const int my_t = pw / G, my_head = g * G + pw % G;
  const bool my_ok = my_t < n_tok;
  const int my_row = tok0 + (my_ok ? my_t : 0);
  const int64_t ph = (int64_t)my_row * a.h_q + my_head;
  bf16x8 qf[NKS], of[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4 wq = {0u, 0u, 0u, 0u}, wo = {0u, 0u, 0u, 0u};
    if (my_ok) {
      wq = ldg16(a.q + ph * D + 32 * ks + 8 * hh);
      wo = ldg16(a.d_out + ph * D + 32 * ks + 8 * hh);
    }
    qf[ks] = *reinterpret_cast<const bf16x8*>(&wq);
    of[ks] = *reinterpret_cast<const bf16x8*>(&wo);
  }
  const float my_l2 = my_ok ? a.meta[2 * ph] : INFINITY;
  const float my_ds = my_ok ? a.meta[2 * ph + 1] : 0.0f;
  f32x4 dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dq[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // the wave's tokens: a unit is skipped unless one of them kept it
  const int wt0 = (16 * wave) / G, wt1 = (16 * wave + 15) / G;
  const uint32_t wave_tok_mask =
      wt0 >= 32 ? 0u : (((wt1 - wt0 + 1) >= 32 ? 0xffffffffu : ((1u << (wt1 - wt0 + 1)) - 1u)) << wt0);
  __builtin_amdgcn_s_waitcnt(0x0f70);

  using DT = DmaTile<D, NT, SW>;
  DT dma;
  dma.init(tid);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)stage;
  const uint16_t* kseq = a.k + (int64_t)g * a.cap * D;
  const uint16_t* vseq = a.v + (int64_t)g * a.cap * D;
  // K of slot s at lds0 + s TILE, V at lds0 + (2 + s) TILE
  auto issue = [&](const Unit& un, int slot) {
    const int64_t off = un.nv > 0 ? (int64_t)un.key0 * D : 0;
    dma.issue(lds0 + slot * TILE, kseq + off, un.nv, tid, wave_u);
    dma.issue(lds0 + (2 + slot) * TILE, vseq + off, un.nv, tid, wave_u);
  };
  // Fragment addresses.  The swizzle of a row reads only its low four bits,
  // so rows 16 m + jj share row jj's (16 m RB is an immediate offset), and
  // the chunk index enters as an XOR: 16-byte row reads (row 16 kt + jj,
  // chunk 4 ks + hh) are the k-step-0 offset XOR 64 ks; transposing reads
  // (row 32 sidx + 4 hh + jj / 4, chunk 2 dt + (jj % 4) / 2, half jj % 2)
  // are the d-tile-0 offset XOR 32 dt.  Slot bases are multiples of 256, so
  // the XORs hold on the absolute addresses too: one XOR per k-step or d-tile
  // and chunk, every row and slot offset an immediate.
  auto row_addr = [&](int r, int c) -> uint32_t {
    return (uint32_t)(r * RB + ((c ^ SW::f(r)) * 16));
  };
  static_assert(TILE % 256 == 0, "slot bases keep bits 0..7");
  const int tr_row = 4 * hh + (jj >> 2), tr_q = jj & 3;
  const uint32_t rd0 = row_addr(jj, hh);
  const uint32_t tr0 = row_addr(tr_row, tr_q >> 1) + 8u * (uint32_t)(tr_q & 1);

  Unit cur = unit_of(0);
  if (n > 0) issue(cur, 0);
  for (int i = 0; i < n; ++i) {
    const int slot = i & 1;
    wait_vm_barrier<0>();
    const Unit nxt = unit_of(i + 1);
    if (i + 1 < n) issue(nxt, slot ^ 1);
    if (cur.tm & wave_tok_mask) {
      const uint32_t kb = lds0 + slot * TILE;
      const uint32_t krd = kb + rd0, ktr = kb + tr0;
      int lim = -1;
      if (my_ok && ((cur.tm >> my_t) & 1u)) lim = min(p0 + my_t - cur.key0, cur.nv - 1);
      // per 32-key half sidx: S^T, dP^T of its two key tiles, then dS^T as
      // the B operand of that half's dQ^T k-step (element e <-> key
      // 16 (2 sidx + e / 4) + 4 hh + e % 4); halves keep 16 accumulators live
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) {
        f32x4 s[2], dp[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          s[t2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          dp[t2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            const uint32_t ra = (krd ^ (uint32_t)(64 * ks)) + (uint32_t)(16 * (2 * sidx + t2) * RB);
            s[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_read16(ra), qf[ks], s[t2],
                                                            0, 0, 0);
            dp[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_read16(ra + 2 * TILE), of[ks],
                                                             dp[t2], 0, 0, 0);
          }
        // lane (jj, hh): pair jj, keys 16 kt + 4 hh + r
        bf16x8 sb;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int off = 16 * (2 * sidx + t2) + 4 * hh + r;
            const float p = off <= lim
                                ? fast_exp2(__builtin_fmaf(s[t2][r], a.scale_log2, -my_l2))
                                : 0.0f;
            sb[4 * t2 + r] = (__bf16)(p * (dp[t2][r] - my_ds));
          }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t base = (ktr ^ (uint32_t)(32 * dt)) + (uint32_t)(32 * sidx * RB);
          const bf16x4 lo = lds_read_tr8(base);
          const bf16x4 hi = lds_read_tr8(base + 16u * RB);
          const bf16x8 ak = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          dq[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, sb, dq[dt], 0, 0, 0);
        }
      }
    }
    cur = nxt;
  }
  if (my_ok) {
    uint16_t* orow = a.dq + ph * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      u32x2 wv;
      wv.x = pack_bf16x2(a.scale * dq[dt][0], a.scale * dq[dt][1]);
      wv.y = pack_bf16x2(a.scale * dq[dt][2], a.scale * dq[dt][3]);
      *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * hh) = wv;
    }
  }
}

// ---------------------------------------------------------------------------
// float32 inputs: one wave per (row, head) on the vector ALU, for the
// exact-precision callers (small shapes).  Per 64-key piece of a kept block:
// lane j takes key j (s = q.k_j, dp = do.v_j, p, ds), then lane d accumulates
// dq[d] += ds_j k_j[d] and adds scale ds_j q[d], p_j do[d] into dk, dv with
// float32 atomics.  A block listed twice counts once.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void bwd_f32_kernel(BwdArgs a) {
  constexpr int R = D / 64;                        // dims per lane in the d phases
  __shared__ float qs[D], dos[D], ps[64], dss[64];
  const int rh = blockIdx.x, lane = threadIdx.x;
  const int row = rh / a.h_q, head = rh % a.h_q;
  const int G = a.h_q / a.h_kv, g = head / G;
  const float* qf = reinterpret_cast<const float*>(a.q);
  const float* kf = reinterpret_cast<const float*>(a.k);
  const float* vf = reinterpret_cast<const float*>(a.v);
  const float* dof = reinterpret_cast<const float*>(a.d_out);
  for (int d = lane; d < D; d += 64) {
    qs[d] = qf[(int64_t)rh * D + d];
    dos[d] = dof[(int64_t)rh * D + d];
  }
  __syncthreads();
  const float l2 = a.meta[2 * (int64_t)rh], dsum = a.meta[2 * (int64_t)rh + 1];
  const int64_t pos = a.n_k - a.n_q + row;
  const float* kg = kf + (int64_t)g * a.cap * D;
  const float* vg = vf + (int64_t)g * a.cap * D;
  float* dkg = a.dk + (int64_t)g * a.cap * D;
  float* dvg = a.dv + (int64_t)g * a.cap * D;
  float dq[R];
#pragma unroll
  for (int i = 0; i < R; ++i) dq[i] = 0.0f;
  const int64_t own = pos / a.B;
  const int n_list = a.dense ? (int)(own + 1) : a.topk;
  const int32_t* lst = a.dense ? nullptr : a.block_idx + ((int64_t)row * a.h_kv + g) * a.topk;
  for (int e = 0; e < n_list; ++e) {
    int64_t b = e;
    if (!a.dense) {
      b = lst[e];
      if (b < 0 || b >= a.n_b || b > own) continue;
      bool dup = false;
      for (int e2 = 0; e2 < e; ++e2) dup = dup || lst[e2] == b;
      if (dup) continue;
    }
    const int64_t k_end = min((b + 1) * (int64_t)a.B, pos + 1);
    for (int64_t key0 = b * a.B; key0 < k_end; key0 += 64) {
      const int nv = (int)min((int64_t)64, k_end - key0);
      float p = 0.0f, ds = 0.0f;
      if (lane < nv) {
        const float* kr = kg + (key0 + lane) * D;
        const float* vr = vg + (key0 + lane) * D;
        float s = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; d += 4) {
          const float4 k4 = *reinterpret_cast<const float4*>(kr + d);
          const float4 v4 = *reinterpret_cast<const float4*>(vr + d);
          s = __builtin_fmaf(qs[d], k4.x, s); s = __builtin_fmaf(qs[d + 1], k4.y, s);
          s = __builtin_fmaf(qs[d + 2], k4.z, s); s = __builtin_fmaf(qs[d + 3], k4.w, s);
          dp = __builtin_fmaf(dos[d], v4.x, dp); dp = __builtin_fmaf(dos[d + 1], v4.y, dp);
          dp = __builtin_fmaf(dos[d + 2], v4.z, dp); dp = __builtin_fmaf(dos[d + 3], v4.w, dp);
        }
        p = fast_exp2(__builtin_fmaf(s, a.scale_log2, -l2));
        ds = p * (dp - dsum);
      }
      ps[lane] = p;
      dss[lane] = ds;
      __syncthreads();
      for (int j = 0; j < nv; ++j) {
        const float pj = ps[j], dsj = dss[j];
        const int64_t kj = (key0 + j) * D;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int d = lane + 64 * i;
          dq[i] = __builtin_fmaf(dsj, kg[kj + d], dq[i]);
          unsafeAtomicAdd(dkg + kj + d, a.scale * dsj * qs[d]);
          unsafeAtomicAdd(dvg + kj + d, pj * dos[d]);
        }
      }
      __syncthreads();
    }
  }
  float* dqo = reinterpret_cast<float*>(a.dq) + (int64_t)rh * D;
#pragma unroll
  for (int i = 0; i < R; ++i) dqo[lane + 64 * i] = a.scale * dq[i];
}

}  // namespace infllmv2

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
using namespace infllmv2;

namespace {

int dq_waves(int G) { return G == 1 ? 2 : (G == 2 ? 4 : 8); }
int dq_tile_tokens(int G) { return 16 * dq_waves(G) / G; }

struct BwdPlan {
  int n_b, nw, n_chunks, seg_rows, max_items;
  bool dense;
  size_t off_dsum, off_bitmap, off_nseg, off_items, off_count, bytes;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdPlan bwd_plan(int n_q, int h_q, int h_kv, int64_t n_k, const Resolved& r) {
  BwdPlan p;
  const int G = h_q / h_kv;
  p.dense = n_k < r.dense_len;
  p.n_b = (int)ceil_div(n_k, r.B);
  p.n_chunks = (int)ceil_div(n_k, kChunk);
  p.nw = (int)ceil_div(n_q, 32);
  p.seg_rows = seg_rows_for(G);
  const int64_t cpb = r.B / kChunk;
  int64_t items;
  if (p.dense) {
    items = (int64_t)h_kv * p.n_chunks * ceil_div(n_q, p.seg_rows);
  } else {
    const int64_t kept = (int64_t)n_q * h_kv * (r.topk < p.n_b ? r.topk : p.n_b);
    items = cpb * ((int64_t)h_kv * p.n_b + ceil_div(kept, p.seg_rows));
  }
  p.max_items = items > INT32_MAX ? INT32_MAX : (int)items;
  size_t o = 0;
  p.off_dsum = o;   o += al256((size_t)n_q * h_q * 8);
  p.off_bitmap = o; o += p.dense ? 0 : al256((size_t)h_kv * p.n_b * p.nw * 4);
  p.off_nseg = o;   o += p.dense ? 0 : al256((size_t)h_kv * p.n_b * 4);
  p.off_items = o;  o += al256((size_t)p.max_items * 8);
  p.off_count = o;  o += 256;
  p.bytes = o;
  return p;
}

#ifndef INFLLMV2_DKDV_KT
#define INFLLMV2_DKDV_KT 1
#endif
constexpr int kDkdvKT = INFLLMV2_DKDV_KT;            // 16-key tiles per wave
template <int D>
int launch_dkdv(int G, const BwdArgs& a, dim3 grid, hipStream_t st) {
  constexpr int NT = 256 / kDkdvKT;
  switch (G) {
    case 1:  hipLaunchKernelGGL((bwd_dkdv_kernel<D, 1, kDkdvKT>), grid, dim3(NT), 0, st, a); break;
    case 2:  hipLaunchKernelGGL((bwd_dkdv_kernel<D, 2, kDkdvKT>), grid, dim3(NT), 0, st, a); break;
    case 4:  hipLaunchKernelGGL((bwd_dkdv_kernel<D, 4, kDkdvKT>), grid, dim3(NT), 0, st, a); break;
    case 8:  hipLaunchKernelGGL((bwd_dkdv_kernel<D, 8, kDkdvKT>), grid, dim3(NT), 0, st, a); break;
    case 16: hipLaunchKernelGGL((bwd_dkdv_kernel<D, 16, kDkdvKT>), grid, dim3(NT), 0, st, a); break;
    case 32: hipLaunchKernelGGL((bwd_dkdv_kernel<D, 32, kDkdvKT>), grid, dim3(NT), 0, st, a); break;
    default: return INFLLMV2_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

template <int D>
int launch_dq(int G, const BwdArgs& a, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1:  hipLaunchKernelGGL((bwd_dq_kernel<D, 1, 2>), grid, dim3(128), 0, st, a); break;
    case 2:  hipLaunchKernelGGL((bwd_dq_kernel<D, 2, 4>), grid, dim3(256), 0, st, a); break;
    case 4:  hipLaunchKernelGGL((bwd_dq_kernel<D, 4, 8>), grid, dim3(512), 0, st, a); break;
    case 8:  hipLaunchKernelGGL((bwd_dq_kernel<D, 8, 8>), grid, dim3(512), 0, st, a); break;
    case 16: hipLaunchKernelGGL((bwd_dq_kernel<D, 16, 8>), grid, dim3(512), 0, st, a); break;
    case 32: hipLaunchKernelGGL((bwd_dq_kernel<D, 32, 8>), grid, dim3(512), 0, st, a); break;
    default: return INFLLMV2_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

}  // namespace

namespace infllmv2 {
size_t prefill_bwd_workspace_bytes(int n_q, int h_q, int h_kv, int64_t n_k, const Resolved& r) {
  return bwd_plan(n_q, h_q, h_kv, n_k, r).bytes;
}
}  // namespace infllmv2

extern "C" int infllmv2_sparse_attn_prefill_backward(
    int dtype, const void* q, int32_t n_q, const void* k, const void* v, int64_t cap,
    int64_t n_k, int32_t h_q, int32_t h_kv, int32_t d, const int32_t* block_idx,
    const void* out, const float* lse, const void* d_out, void* dq, float* dk, float* dv,
    void* ws, size_t ws_bytes, const infllmv2_params* p, void* stream) {
  if (!dtype_ok(dtype)) return INFLLMV2_ERR_INVALID_ARG;
  INFLLMV2_TRY(check_heads(h_q, h_kv));
  if (!head_dim_ok(d)) return INFLLMV2_ERR_UNSUPPORTED;
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if (!q || !k || !v || !out || !lse || !d_out || !dq || !dk || !dv)
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_q < 0 || n_k <= 0 || cap < n_k || n_q > n_k) return INFLLMV2_ERR_INVALID_ARG;
  if (cap > INT32_MAX) return INFLLMV2_ERR_UNSUPPORTED;
  const bool dense = n_k < r.dense_len;
  if (!dense && !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(d_out) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return INFLLMV2_ERR_INVALID_ARG;
  const int G = h_q / h_kv;
  const bool f32 = dtype == INFLLMV2_F32;
  if (!f32 && (!group_ok_for_mfma(G) || r.B % kChunk != 0)) return INFLLMV2_ERR_UNSUPPORTED;
  // the dK/dV kernel's direct copies address Q, dO and meta with 32-bit
  // offsets, and multiplies row indices in 24 bits
  if ((int64_t)n_q * h_q * d * 2 >= (1ll << 32) || n_q >= (1 << 24))
    return INFLLMV2_ERR_UNSUPPORTED;
  const BwdPlan pl = bwd_plan(n_q, h_q, h_kv, n_k, r);
  if (!ws || ws_bytes < pl.bytes || ((uintptr_t)ws & 255u)) return INFLLMV2_ERR_WORKSPACE;
  if (n_q == 0) return INFLLMV2_OK;

  BwdArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.block_idx = dense ? nullptr : block_idx;
  a.out = (const uint16_t*)out; a.lse = lse; a.d_out = (const uint16_t*)d_out;
  a.dq = (uint16_t*)dq; a.dk = dk; a.dv = dv;
  char* w = (char*)ws;
  a.meta = (float*)(w + pl.off_dsum);
  a.bitmap = (uint32_t*)(w + pl.off_bitmap);
  a.nseg = (int32_t*)(w + pl.off_nseg);
  a.items = (int2*)(w + pl.off_items);
  a.n_items = (int32_t*)(w + pl.off_count);
  a.cap = cap; a.n_k = n_k; a.n_q = n_q; a.h_q = h_q; a.h_kv = h_kv; a.topk = r.topk;
  a.B = r.B; a.n_b = pl.n_b; a.nw = pl.nw; a.n_chunks = pl.n_chunks; a.seg_rows = pl.seg_rows;
  a.max_items = pl.max_items; a.dense = dense ? 1 : 0;
  a.scale = r.scale; a.scale_log2 = r.scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
#ifdef INFLLMV2_DEBUG
  if (!dense) INFLLMV2_TRY(debug_check_rows(block_idx, n_q, h_kv, r, n_k, n_q, nullptr, 0, st));
#endif
  if (f32) {
    if ((int64_t)n_q * h_q >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
    const unsigned blocks = (unsigned)ceil_div((int64_t)n_q * h_q * (d / 4), 256);
    if (d == 128) {
      hipLaunchKernelGGL((bwd_dsum_kernel<float, 128>), dim3(blocks), dim3(256), 0, st, a);
      hipLaunchKernelGGL((bwd_f32_kernel<128>), dim3((unsigned)(n_q * h_q)), dim3(64), 0, st, a);
    } else {
      hipLaunchKernelGGL((bwd_dsum_kernel<float, 64>), dim3(blocks), dim3(256), 0, st, a);
      hipLaunchKernelGGL((bwd_f32_kernel<64>), dim3((unsigned)(n_q * h_q)), dim3(64), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
  }
  const int TT = dq_tile_tokens(G);
  a.n_tiles = (int)ceil_div(n_q, TT);
  if ((int64_t)a.n_tiles * h_kv >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;

  const int64_t dsum_threads = (int64_t)n_q * h_q * (d / 8);
  const unsigned dsum_blocks = (unsigned)ceil_div(dsum_threads, 256);
  if (d == 128)
    hipLaunchKernelGGL((bwd_dsum_kernel<uint16_t, 128>), dim3(dsum_blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_dsum_kernel<uint16_t, 64>), dim3(dsum_blocks), dim3(256), 0, st, a);
  if (hipGetLastError() != hipSuccess) return INFLLMV2_ERR_HIP;
  if (!dense) {
    if (pl.n_b <= kMarkLdsBlocks) {
      hipLaunchKernelGGL(bwd_mark_lds_kernel, dim3((unsigned)pl.nw, (unsigned)h_kv), dim3(256),
                         (size_t)pl.n_b * 4, st, a);
    } else {
      const int64_t words = (int64_t)h_kv * pl.n_b * pl.nw;
      const int64_t fb = ceil_div(words, 256);
      hipLaunchKernelGGL(bwd_fill_kernel, dim3((unsigned)(fb < 4096 ? fb : 4096)), dim3(256), 0,
                         st, a.bitmap, words);
      const int64_t marks = (int64_t)n_q * h_kv * r.topk;
      hipLaunchKernelGGL(bwd_mark_kernel, dim3((unsigned)ceil_div(marks, 256)), dim3(256), 0, st,
                         a);
    }
    hipLaunchKernelGGL(bwd_count_kernel, dim3((unsigned)ceil_div((int64_t)h_kv * pl.n_b, 4)),
                       dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) return INFLLMV2_ERR_HIP;
  }
  const int plan_units = h_kv * (dense ? pl.n_chunks : pl.n_b);
  hipLaunchKernelGGL(bwd_plan_kernel, dim3((unsigned)ceil_div(plan_units, kPlanThreads1)),
                     dim3(kPlanThreads1), 0, st, a);
  if (hipGetLastError() != hipSuccess) return INFLLMV2_ERR_HIP;
  INFLLMV2_TRY(d == 128 ? launch_dkdv<128>(G, a, dim3((unsigned)pl.max_items), st)
                        : launch_dkdv<64>(G, a, dim3((unsigned)pl.max_items), st));
  const dim3 gq((unsigned)(a.n_tiles * h_kv));
  return d == 128 ? launch_dq<128>(G, a, gq, st) : launch_dq<64>(G, a, gq, st);
}
