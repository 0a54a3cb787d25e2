// Block-sparse causal attention over the kept blocks, bf16 inputs, float32
// accumulation, on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
// Sources: "MiniCPM4: running LLMs on phones and PCs" (xugj520.cn), section
// 1.1 (attention is computed on the selected blocks only; initial and local
// blocks always kept; uint64 tree mask); "MiniCPM 4.0" blog (shadowrocket9.top),
// InfLLM v2 section (64-token blocks, top-64, dense below 8192 tokens);
// pomoai.com CPM.cu article, sections 2 and 4 (tree verification inside the
// attention kernel, chunked prefill).
//
// Layout of the work inside a wave (64 lanes): the wave owns 32 query rows
// (32/G tokens x the G heads of one KV group, which share every selection).
// Scores are computed transposed, S^T = K Q^T, with K as the A operand
// (32 keys x 16 dims) and Q^T as the B operand held in registers, so each
// lane's accumulator column is ONE query row: the row max needs a single
// exchange between the two half-waves and the row sum none until the end.
// P^T then feeds the P.V product directly from the accumulator registers as
// the B operand of O^T = V^T P^T; V^T comes from LDS, where V is written
// transposed while it is staged.
//
// Work units are 64-key chunks of kept blocks.  A workgroup stages each chunk
// (K as [key][d], V as [d][key], both padded against bank conflicts) into a
// double-buffered LDS ring with one barrier per chunk; the next chunk is
// prefetched into registers while the current one is multiplied.
//   prefill: a workgroup owns TT consecutive query tokens of one KV head and
//            walks the union of their kept blocks (built in LDS by a bitonic
//            sort of the tokens' block lists); a wave skips chunks that none
//            of its tokens kept, and masks rows of tokens that did not keep it.
//   decode:  (sequence, KV head, split) workgroups walk a slice of the
//            sequence's kept blocks and write float32 partials (o, m, l).
//   tree:    (KV head, split) workgroups walk a slice of the union of all
//            drafts' kept blocks plus one chunk holding the draft tokens
//            (masked by the uint64 ancestor mask); partials as in decode.
//   combine: merges the split partials with their log-sum-exp weights.
#include "attn_common.h"

namespace infllmv2 {

template <int D>
struct Lds {
  static constexpr int kKStride = D + 8;         // bf16 elements per staged K row
  static constexpr int kVStride = kChunk + 8;    // bf16 elements per staged V^T row
  static constexpr int kKElems = kChunk * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kStageElems = kKElems + kVElems;
  static constexpr int kBytes = 2 * kStageElems * 2;   // double-buffered
};

// ---------------------------------------------------------------------------
// Staging of one 64-key chunk: keys [key0, key0 + nvalid) of a K/V row block.
// ---------------------------------------------------------------------------
// V^T rows hold the 64 keys of a chunk in a permuted order: key bits 2 and 3
// are swapped, so that the 8 keys one lane needs for a P.V k-step
// (16t + 4h + {0..3} and 16t + 8 + 4h + {0..3}) sit in 16 contiguous bytes.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D, int NT>
struct Stager {
  // K: thread t owns kKPer consecutive keys of one 16-byte column chunk:
  //    key = kKPer * (t / CPR) + i, chunk = t % CPR  (CPR = D/8 chunks per row).
  //    Its global pieces sit at immediate offsets 0, 2D, 4D, ... bytes.
  // V: thread t owns key pairs kp = t % 32 for chunks c = t / 32 + (NT/32) * i,
  //    i.e. rows 2kp and 2kp+1 of kVPer chunks (again immediate offsets).
  static constexpr int CPR = D / 8;
  static constexpr int kKPer = kChunk * CPR / NT;
  static constexpr int kVJobs = (kChunk / 2) * CPR;
  static constexpr int kVPer = (kVJobs + NT - 1) / NT;
  static_assert(kKPer >= 1 && (kChunk * CPR) % NT == 0, "K staging shape");
  u32x4 kr[kKPer];
  u32x4 vr[kVPer][2];

  __device__ static __forceinline__ int k_key0(int tid) { return kKPer * (tid / CPR); }
  __device__ static __forceinline__ int k_chunk(int tid) { return tid % CPR; }
  __device__ static __forceinline__ int v_pair(int tid) { return tid % (kChunk / 2); }
  __device__ static __forceinline__ int v_chunk(int tid, int i) {
    return tid / (kChunk / 2) + (NT / (kChunk / 2)) * i;
  }

  // kbase/vbase point at key 0 of the chunk (or at any valid row when
  // nvalid == 0); keys >= nvalid are zero-filled so that masked lanes never
  // multiply garbage.  Full chunks take the branch-free path.
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase,
                                       int nvalid, int tid) {
    const int kk0 = k_key0(tid), kc = k_chunk(tid);
    const int vk0 = 2 * v_pair(tid);
    if (nvalid == kChunk) {
      const uint16_t* kp = kbase + kk0 * D + kc * 8;
#pragma unroll
      for (int i = 0; i < kKPer; ++i) kr[i] = ldg16(kp + i * D);
      const uint16_t* vp = vbase + vk0 * D;
#pragma unroll
      for (int i = 0; i < kVPer; ++i) {
        const int c = v_chunk(tid, i);
        if (kVJobs % NT != 0 && c >= CPR) break;
        vr[i][0] = ldg16(vp + c * 8);
        vr[i][1] = ldg16(vp + D + c * 8);
      }
      return;
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int key = kk0 + i;
      const bool ok = key < nvalid;
      const u32x4 x = ldg16(kbase + (ok ? key : 0) * D + kc * 8);
      kr[i] = ok ? x : z;
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int c = v_chunk(tid, i);
      const bool in = c < CPR;
      const bool ok0 = in && vk0 < nvalid, ok1 = in && vk0 + 1 < nvalid;
      const u32x4 x0 = ldg16(vbase + (ok0 ? vk0 : 0) * D + (in ? c : 0) * 8);
      const u32x4 x1 = ldg16(vbase + (ok1 ? vk0 + 1 : 0) * D + (in ? c : 0) * 8);
      vr[i][0] = ok0 ? x0 : z;
      vr[i][1] = ok1 ? x1 : z;
    }
  }

  __device__ __forceinline__ void store(uint16_t* stage, int tid) const {
    uint16_t* Ks = stage + k_key0(tid) * Lds<D>::kKStride + k_chunk(tid) * 8;
#pragma unroll
    for (int i = 0; i < kKPer; ++i)
      *reinterpret_cast<u32x4*>(Ks + i * Lds<D>::kKStride) = kr[i];
    // keys 2kp, 2kp+1 stay adjacent in the permuted V^T row order
    uint16_t* Vt = stage + Lds<D>::kKElems + vt_pos(2 * v_pair(tid));
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int c = v_chunk(tid, i);
      if (kVJobs % NT != 0 && c >= CPR) break;
      const uint32_t a[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
      const uint32_t b[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims c*8 + 2e (low halves) and c*8 + 2e + 1 (high halves)
        const uint32_t lo = __builtin_amdgcn_perm(b[e], a[e], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(b[e], a[e], 0x07060302u);
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + 2 * e) * Lds<D>::kVStride) = lo;
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + 2 * e + 1) * Lds<D>::kVStride) = hi;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Per-wave online-softmax state for 32 query rows (one row per lane column).
// The running max m is only raised when a block's max exceeds it by more
// than kRescaleSlack (log2 units): exponentials then stay below 2^slack, which
// float32 sums and bf16 P fragments hold without loss, and the O rescale runs
// rarely.  The result is unchanged: numerator and denominator use the same m.
// ---------------------------------------------------------------------------
constexpr float kRescaleSlack = 8.0f;
template <int D>
struct RowState {
  bf16x8 q[D / 16];      // Q^T B-operand fragments (row = lane % 32)
  f32x16 o[D / 32];      // O^T accumulators: rows d = 32*dt + 8*(v/4) + 4*half + v%4
  float m, l;            // running max (log2 domain) and this half's sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] = 0.0f;
    m = kNoMax;
    l = 0.0f;
  }

  // One staged 64-key chunk.  `lim` = largest valid key offset (0..63) inside
  // the chunk for this lane's row, or -1 if the row keeps none of it.
  // `draft_bits` (tree chunk) restricts the valid offsets further.
  // P^T fragments of one chunk: k-step t of key tile kt.
  struct PFrag { bf16x8 f[2][2]; };

  // S^T = K Q^T for one staged chunk, masked online softmax; returns the
  // P^T fragments (and rescales O when the running max moves).
  __device__ __forceinline__ PFrag scores(const uint16_t* stage, int lim, bool use_bits,
                                          uint64_t draft_bits, float scale_log2) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const uint16_t* Ks = stage;
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = 0.0f;
      const uint16_t* krow = Ks + (32 * kt + col) * Lds<D>::kKStride + 8 * half;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * ks);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[ks], s[kt], 0, 0, 0);
      }
    }
    // Scale into the log2 domain, mask, row max, exponentials.  Common case
    // (every row of the wave keeps all 64 keys or none of them): no per-key
    // masking -- rows that keep nothing subtract +inf, so their p is 0.
    const bool partial = (lim >= 0 && lim < kChunk - 1) || use_bits;
    const bool keep = lim >= 0;
    float m_new, alpha, psum = 0.0f;
    if (!__ballot(partial)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
      mx = keep ? mx * scale_log2 : -INFINITY;
      mx = fmaxf(mx, swap_halves(mx));
      m_new = mx > m + kRescaleSlack ? mx : m;
      alpha = fast_exp2(m - m_new);
      const float msub = keep ? m_new : INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(s[kt][v], scale_log2, -msub));
          s[kt][v] = p;
          psum += p;
        }
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = 32 * kt + 8 * (v >> 2) + 4 * half + (v & 3);
          bool ok = off <= lim;
          if (use_bits) ok = ok && ((draft_bits >> off) & 1ull);
          const float x = ok ? s[kt][v] * scale_log2 : -INFINITY;
          s[kt][v] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, swap_halves(mx));
      m_new = mx > m + kRescaleSlack ? mx : m;
      alpha = fast_exp2(m - m_new);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(s[kt][v] - m_new);
          s[kt][v] = p;
          psum += p;
        }
    }
    m = m_new;
    l = l * alpha + psum;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
    }
    // P^T fragments: k-step t of key tile kt uses accumulator entries 8t..8t+7
    PFrag pf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf.f[kt][t][e] = (__bf16)s[kt][8 * t + e];
    return pf;
  }

  // O^T += V^T P^T; A-operand element e of half h <-> key 16t + 8(e/4) + 4h + e%4.
  // Run for every staged chunk (with zero P when the wave keeps none of it),
  // so that O flows through the same instructions on every iteration.
  __device__ __forceinline__ void pv(const uint16_t* stage, const PFrag& pf) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const uint16_t* Vt = stage + Lds<D>::kKElems;
    const auto& pb = pf.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint16_t* vrow = Vt + (32 * dt + col) * Lds<D>::kVStride + 8 * half;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          // keys 16t + 4h + {0..3} and 16t + 8 + 4h + {0..3}: permuted layout
          // puts them at positions 16t + 8h .. +8
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + 32 * kt + 16 * t);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][t], o[dt], 0, 0, 0);
        }
      }
    }
  }
};

// Load this lane's Q^T fragments: row `qrow` (NULL -> zeros).
template <int D>
__device__ __forceinline__ void load_q(RowState<D>& st, const uint16_t* qrow) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow) w = ldg16(qrow + 16 * ks + 8 * half);
    st.q[ks] = *reinterpret_cast<const bf16x8*>(&w);
  }
}

// ---------------------------------------------------------------------------
// Bitonic sort (ascending) of N uint32 keys in LDS by NT threads.
// ---------------------------------------------------------------------------
template <int NT>
__device__ void bitonic_sort(uint32_t* buf, int N) {
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < N; i += NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint32_t a = buf[i], b = buf[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) { buf[i] = b; buf[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
}

template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < NT / 64; ++w) {
    const int t = lds[w];
    if (w < wid) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Union of the kept-block lists of TT tokens: sorted unique block ids with a
// bitmask of the tokens (bit t) that kept each, written to ents[] as
// (block, mask).  `sortbuf` holds N >= TT*topk (power of two) words; returns
// the union length.
template <int NT, int TT>
__device__ int build_union(const int32_t* block_idx, int tok0, int h_kv, int g, int n_tok,
                           int topk, int n_b, uint32_t* sortbuf, int N, int2* ents,
                           int* scan_lds) {
  for (int i = threadIdx.x; i < N; i += NT) {
    uint32_t key = 0xffffffffu;
    const int t = i / topk, j = i % topk;
    if (t < n_tok && i < TT * topk) {
      const int32_t b = block_idx[((int64_t)(tok0 + t) * h_kv + g) * topk + j];
      if (b >= 0 && b < n_b) key = ((uint32_t)b << 5) | (uint32_t)t;
    }
    sortbuf[i] = key;
  }
  __syncthreads();
  bitonic_sort<NT>(sortbuf, N);
  const int C = N / NT;                         // N is a multiple of NT
  const int c0 = threadIdx.x * C;
  int heads = 0;
  for (int i = c0; i < c0 + C; ++i) {
    const uint32_t key = sortbuf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (sortbuf[i - 1] >> 5) != (key >> 5)) ++heads;
  }
  int total;
  int slot = block_excl_scan<NT>(heads, &total, scan_lds);
  for (int i = c0; i < c0 + C; ++i) {
    const uint32_t key = sortbuf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (sortbuf[i - 1] >> 5) != (key >> 5)) {
      uint32_t msk = 0;
      for (int i2 = i; i2 < N && sortbuf[i2] != 0xffffffffu && (sortbuf[i2] >> 5) == (key >> 5);
           ++i2)
        msk |= 1u << (sortbuf[i2] & 31u);
      ents[slot] = make_int2((int)(key >> 5), (int)msk);
      ++slot;
    }
  }
  __syncthreads();
  return total;
}

// Entries a split workgroup may hold in LDS (host keeps units per split below).
constexpr int kSplitEntryCap = 64;

// ---------------------------------------------------------------------------
// The attention kernel.
//   W waves, each 32 rows = TPW tokens x G heads; TT = W * TPW tokens.
// Indices are 32-bit inside the kernel: the host rejects caches with more
// than 2^31 - 1 tokens per (sequence, KV head).
// ---------------------------------------------------------------------------
template <int D, int G, int W, int MODE, int PF = 1>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = W * 64;
  constexpr int TPW = 32 / G;
  constexpr int TT = (MODE == kDecode) ? 1 : W * TPW;
  static_assert(TT <= 32, "token bitmask is 32 bits");
  static_assert(MODE != kPrefill || TT > 1, "prefill tiles hold several tokens");
  constexpr int SORT_N = (MODE == kPrefill) ? TT * kSortCap : 0;
  constexpr int ECAP = (MODE == kPrefill) ? TT * kSortCap : kSplitEntryCap;
  __shared__ __attribute__((aligned(16))) uint16_t stage[2 * Lds<D>::kStageElems];
  __shared__ int2 ents[ECAP];
  __shared__ int scan_lds[NT / 64];
  static_assert(SORT_N * 4 <= (int)sizeof(stage), "sort buffer aliases the staging ring");

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;

  // ---- work item ---------------------------------------------------------
  int g, tile = 0, seq = 0, split = 0;
  if constexpr (MODE == kPrefill) {
    const int w = xcd_contiguous_index(blockIdx.x, gridDim.x);
    g = w / a.n_tiles;
    tile = w % a.n_tiles;
  } else {
    split = blockIdx.x;
    g = blockIdx.y;
    if constexpr (MODE == kDecode) seq = blockIdx.z; else tile = blockIdx.z;
  }

  // tokens of this workgroup and their query positions
  int n_keys, tok0, n_tok;
  if constexpr (MODE == kDecode) {
    // lengths outside [1, max_seqlen] are clamped: wrong input, no fault
    const int L = a.seqlens[seq];
    n_keys = L < 1 ? 1 : (L > (int)a.n_k ? (int)a.n_k : L);
    tok0 = seq;
    n_tok = 1;
  } else {
    n_keys = (int)a.n_k;
    tok0 = tile * TT;
    n_tok = min(TT, a.n_rows - tok0);
  }
  const bool dense = n_keys < a.dense_len || a.block_idx == nullptr;
  const int n_b = (n_keys + a.B - 1) / a.B;
  const int cpb = (a.B + kChunk - 1) / kChunk;            // chunks per block
  const uint32_t full_mask = n_tok >= 32 ? 0xffffffffu : ((1u << n_tok) - 1u);
  // first query position of the tile (prefill: consecutive positions)
  const int p0 = (MODE == kPrefill) ? (int)a.n_k - a.n_rows + tok0 : n_keys - 1;

  // this lane's row
  const int t_in_wave = col / G, head_in_group = col % G;
  const int my_t = (MODE == kDecode) ? (wave == 0 && t_in_wave == 0 ? 0 : 32)
                                     : wave * TPW + t_in_wave;   // 32 = none
  const bool row_ok = my_t < n_tok;
  const int my_row = tok0 + (row_ok ? my_t : 0);
  const int my_head = g * G + head_in_group;
  const int my_pos = (MODE == kPrefill) ? p0 + (row_ok ? my_t : 0) : n_keys - 1;

  // ---- entries (kept blocks with token masks) and this workgroup's units ---
  const bool has_draft = MODE == kTree;
  int n_entries;
  if constexpr (MODE == kPrefill) {
    if (dense) {
      n_entries = (p0 + n_tok - 1) / a.B + 1;
    } else {
      int N = 1;
      while (N < TT * a.topk) N <<= 1;
      if (N < NT) N = NT;
      n_entries = build_union<NT, TT>(a.block_idx, tok0, a.h_kv, g, n_tok, a.topk, n_b,
                                      reinterpret_cast<uint32_t*>(stage), N, ents, scan_lds);
    }
  } else if constexpr (MODE == kDecode) {
    if (dense) {
      n_entries = n_b;
    } else {
      const int32_t* lst = a.block_idx + ((int64_t)seq * a.h_kv + g) * a.topk;
      int n = 0;
      while (n < a.topk && lst[n] >= 0 && lst[n] < n_b) ++n;
      n_entries = n;
    }
  } else {
    n_entries = dense ? n_b : a.union_len[g];
  }
  const int n_units_total = n_entries * cpb + (has_draft ? 1 : 0);
  int u_begin = 0, u_end = n_units_total;
  if constexpr (MODE != kPrefill) {
    // balanced contiguous slices of this row's units over the n_split splits
    const int per = (n_units_total + a.n_split - 1) / a.n_split;
    u_begin = min(n_units_total, split * per);
    u_end = min(n_units_total, u_begin + per);
  }
  // split modes: copy this slice's entries into LDS (entry e -> ents[e - e_base])
  int e_base = 0;
  if constexpr (MODE != kPrefill) {
    if (!dense) {
      e_base = u_begin / cpb;
      const int e_end = min(n_entries, (u_end + cpb - 1) / cpb);
      for (int e = e_base + tid; e < e_end && e - e_base < kSplitEntryCap; e += NT) {
        if constexpr (MODE == kDecode) {
          ents[e - e_base] = make_int2(a.block_idx[((int64_t)seq * a.h_kv + g) * a.topk + e], 1);
        } else {
          const int64_t ix = (int64_t)g * a.union_cap + e;
          ents[e - e_base] = make_int2(a.union_blk[ix], (int)(uint32_t)(a.union_mask[ix] >> tok0));
        }
      }
      __syncthreads();
    }
  }

  // unit -> first key, #valid keys, token mask, draft flag
  struct UnitInfo { int key0, nv; uint32_t tm; bool isd; };
  auto unit_info = [&](int u) -> UnitInfo {
    UnitInfo r;
    r.isd = has_draft && u == n_entries * cpb;
    if (r.isd) {
      r.key0 = 0; r.nv = a.n_rows; r.tm = full_mask;
      return r;
    }
    int e = u, c = 0;
    if (cpb != 1) { e = u / cpb; c = u - e * cpb; }
    int b;
    if (dense) {
      b = e;
      if constexpr (MODE == kPrefill) {
        // token t keeps block b iff b <= (p0 + t) / B, i.e. t >= b*B - p0
        const int t_min = b * a.B - p0;
        r.tm = t_min <= 0 ? full_mask : (t_min >= 32 ? 0u : (full_mask & (0xffffffffu << t_min)));
      } else {
        r.tm = full_mask;
      }
    } else {
      const int2 en = ents[e - e_base];
      b = en.x;
      r.tm = (uint32_t)en.y;
    }
    r.key0 = b * a.B + c * kChunk;
    const int blk_end = min((b + 1) * a.B, n_keys);
    r.nv = max(0, min(kChunk, blk_end - r.key0));
    // identical in every lane: keep them in scalar registers
    r.key0 = __builtin_amdgcn_readfirstlane(r.key0);
    r.nv = __builtin_amdgcn_readfirstlane(r.nv);
    r.tm = __builtin_amdgcn_readfirstlane(r.tm);
    return r;
  };

  const int64_t kv_head_off = (MODE == kDecode ? ((int64_t)seq * a.h_kv + g) : (int64_t)g) *
                              a.cap * D;
  const uint16_t* kbase_seq = a.k + kv_head_off;
  const uint16_t* vbase_seq = a.v + kv_head_off;
  const uint16_t* kdraft = has_draft ? a.k_draft + (int64_t)g * a.n_rows * D : nullptr;
  const uint16_t* vdraft = has_draft ? a.v_draft + (int64_t)g * a.n_rows * D : nullptr;
  auto kptr = [&](const UnitInfo& ui) {
    return ui.isd ? kdraft : kbase_seq + (ui.nv > 0 ? (int64_t)ui.key0 * D : 0);
  };
  auto vptr = [&](const UnitInfo& ui) {
    return ui.isd ? vdraft : vbase_seq + (ui.nv > 0 ? (int64_t)ui.key0 * D : 0);
  };

  RowState<D> st;
  st.init();
  load_q<D>(st, row_ok ? a.q + ((int64_t)my_row * a.h_q + my_head) * D : nullptr);
  uint64_t my_bits = 0;
  if (has_draft && row_ok) {
    const uint64_t full = a.n_rows >= 64 ? ~0ull : ((1ull << a.n_rows) - 1ull);
    my_bits = (a.tree_mask[my_row] & full) | (1ull << my_row);
  }

  // one staged chunk: which of my rows use it, up to which key offset
  auto compute_chunk = [&](const uint16_t* buf, const UnitInfo& ui) {
    int lim = -1;
    if (row_ok && ((ui.tm >> my_t) & 1u)) {
      const int last = (ui.isd ? ui.nv - 1 : min(my_pos - ui.key0, ui.nv - 1));
      lim = last < 0 ? -1 : last;
    }
    typename RowState<D>::PFrag pf;
    if (__ballot(lim >= 0)) {
      pf = st.scores(buf, lim, ui.isd, my_bits, a.scale_log2);
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf.f[kt][t][e] = (__bf16)0.0f;
    }
    st.pv(buf, pf);
  };

  if constexpr (PF == 1) {
    // register prefetch one chunk ahead; store -> barrier -> prefetch -> compute
    Stager<D, NT> sg;
    UnitInfo cur = {0, 0, 0u, false};
    if (u_begin < u_end) {
      cur = unit_info(u_begin);
      sg.load(kptr(cur), vptr(cur), cur.nv, tid);
    }
    for (int u = u_begin; u < u_end; ++u) {
      uint16_t* buf = stage + ((u - u_begin) & 1) * Lds<D>::kStageElems;
      sg.store(buf, tid);
      __syncthreads();
      UnitInfo nxt = cur;
      if (u + 1 < u_end) {
        nxt = unit_info(u + 1);
        sg.load(kptr(nxt), vptr(nxt), nxt.nv, tid);
      }
      compute_chunk(buf, cur);
      cur = nxt;
    }
  } else {
    // two register sets: chunk u+1 is stored while chunk u is multiplied,
    // and the loads of chunk u+3 go out into the set just stored, so every
    // chunk has two iterations to arrive.  Iteration i (u = u_begin + i):
    //   barrier; store set[(i+1)&1] -> stage[(i+1)&1]; load u+3 -> that set;
    //   compute stage[i&1].
    Stager<D, NT> sgA, sgB;
    auto fetch = [&](Stager<D, NT>& sg, int u) {
      if (u < u_end) {
        const UnitInfo ui = unit_info(u);
        sg.load(kptr(ui), vptr(ui), ui.nv, tid);
      }
    };
    fetch(sgA, u_begin);
    fetch(sgB, u_begin + 1);
    if (u_begin < u_end) sgA.store(stage, tid);
    fetch(sgA, u_begin + 2);
    auto iter = [&](int i, Stager<D, NT>& nxt_set) {
      const int u = u_begin + i;
      __syncthreads();
      if (u + 1 < u_end) {
        nxt_set.store(stage + ((i + 1) & 1) * Lds<D>::kStageElems, tid);
        fetch(nxt_set, u + 3);
      }
      compute_chunk(stage + (i & 1) * Lds<D>::kStageElems, unit_info(u));
    };
    const int n = u_end - u_begin;
    for (int i = 0; i < n; i += 2) {
      iter(i, sgB);                       // stores chunk u+1 from set B
      if (i + 1 < n) iter(i + 1, sgA);    // stores chunk u+2 from set A
    }
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = st.l + swap_halves(st.l);
  if constexpr (MODE == kPrefill) {
    if (row_ok) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      uint16_t* orow = a.out + ((int64_t)my_row * a.h_q + my_head) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int d0 = 32 * dt + 8 * qd + 4 * half;
          u32x2 w;
          w.x = pack_bf16x2(st.o[dt][4 * qd + 0] * inv, st.o[dt][4 * qd + 1] * inv);
          w.y = pack_bf16x2(st.o[dt][4 * qd + 2] * inv, st.o[dt][4 * qd + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      if (a.lse && half == 0)
        a.lse[(int64_t)my_row * a.h_q + my_head] = (st.m + __log2f(l_tot)) * kLn2;
    }
  } else {
    if (row_ok) {
      float* part = a.ws + (((int64_t)my_row * a.h_q + my_head) * a.n_split + split) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int d0 = 32 * dt + 8 * qd + 4 * half;
          f32x4 w = {st.o[dt][4 * qd + 0], st.o[dt][4 * qd + 1], st.o[dt][4 * qd + 2],
                     st.o[dt][4 * qd + 3]};
          *reinterpret_cast<f32x4*>(part + d0) = w;
        }
      if (half == 0) {
        part[D] = st.m;
        part[D + 1] = l_tot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tree planner: union of the drafts' kept blocks per KV head (sorted, with the
// bitmask of drafts that kept each block).  One workgroup per KV head.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 512;
__global__ __launch_bounds__(kPlanThreads) void tree_union_kernel(
    const int32_t* block_idx, int n_draft, int h_kv, int topk, int64_t n_b, int32_t* ublk,
    uint64_t* umask, int32_t* ulen, int union_cap) {
  __shared__ uint32_t buf[64 * kSortCap];
  __shared__ int scan_lds[kPlanThreads / 64];
  const int g = blockIdx.x;
  int N = 1;
  while (N < n_draft * topk) N <<= 1;
  if (N < kPlanThreads) N = kPlanThreads;
  for (int i = threadIdx.x; i < N; i += kPlanThreads) {
    uint32_t key = 0xffffffffu;
    if (i < n_draft * topk) {
      const int t = i / topk, j = i % topk;
      const int32_t b = block_idx[((int64_t)t * h_kv + g) * topk + j];
      if (b >= 0 && b < n_b) key = ((uint32_t)b << 6) | (uint32_t)t;
    }
    buf[i] = key;
  }
  __syncthreads();
  bitonic_sort<kPlanThreads>(buf, N);
  const int C = N / kPlanThreads;
  const int c0 = threadIdx.x * C;
  int heads = 0;
  for (int i = c0; i < c0 + C; ++i) {
    const uint32_t key = buf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (buf[i - 1] >> 6) != (key >> 6)) ++heads;
  }
  int total;
  int slot = block_excl_scan<kPlanThreads>(heads, &total, scan_lds);
  for (int i = c0; i < c0 + C; ++i) {
    const uint32_t key = buf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (buf[i - 1] >> 6) != (key >> 6)) {
      uint64_t msk = 0;
      for (int i2 = i; i2 < N && buf[i2] != 0xffffffffu && (buf[i2] >> 6) == (key >> 6); ++i2)
        msk |= 1ull << (buf[i2] & 63u);
      if (slot < union_cap) {
        ublk[(int64_t)g * union_cap + slot] = (int32_t)(key >> 6);
        umask[(int64_t)g * union_cap + slot] = msk;
      }
      ++slot;
    }
  }
  if (threadIdx.x == 0) ulen[g] = total < union_cap ? total : union_cap;
}

// ---------------------------------------------------------------------------
// Merge of split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// ---------------------------------------------------------------------------
template <int D, typename TOut>
__global__ __launch_bounds__(64) void combine_kernel(const float* ws, int n_split, TOut* out,
                                                     float* lse) {
  constexpr int kMaxSplit = 64;
  __shared__ float wsh[kMaxSplit];
  const int rh = blockIdx.x;   // row * h_q + head
  const int lane = threadIdx.x;
  const float* base = ws + (int64_t)rh * n_split * (D + 2);
  // lane s holds split s (n_split <= 64): max, weights and normaliser in
  // parallel over the splits
  float m = kNoMax, l = 0.0f;
  if (lane < n_split) {
    l = base[lane * (D + 2) + D + 1];
    m = l > 0.0f ? base[lane * (D + 2) + D] : kNoMax;
  }
  const float M = wave_max(m);
  const float w = l > 0.0f ? fast_exp2(m - M) : 0.0f;
  const float L = wave_sum(w * l);
  if (lane < kMaxSplit) wsh[lane] = w;
  __syncthreads();
  float acc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.0f;
  for (int s = 0; s < n_split; ++s) {
    const float ww = wsh[s];
    if (ww == 0.0f) continue;
    const float* p = base + s * (D + 2);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) acc[i] += ww * p[lane + 64 * i];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
    Elem<TOut>::store(out + (int64_t)rh * D + lane + 64 * i, acc[i] * inv);
  if (lse && lane == 0) lse[rh] = (M + __log2f(L)) * kLn2;
}

}  // namespace infllmv2

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
using namespace infllmv2;

namespace {

// Splits per (row, KV head): enough workgroups to cover the GPU for batched
// decode and tree verification while keeping the float32 partials small.
constexpr int kMaxDecodeSplits = 32;
constexpr int kMaxTreeSplits = 32;
constexpr int kMaxCombineSplits = 64;      // lanes of the combine kernel

template <int D, int G, int W, int MODE, int PF = 1>
int launch_attn(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, G, W, MODE, PF>), grid, dim3(W * 64), 0, st, a);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

// Prefill uses W = min(4, G) waves (TT = 32/G * W <= 32 tokens per tile).
template <int D>
int dispatch_prefill(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1:  return launch_attn<D, 1, 1, kPrefill>(a, grid, st);
    case 2:  return launch_attn<D, 2, 2, kPrefill>(a, grid, st);
    case 4:  return launch_attn<D, 4, 4, kPrefill>(a, grid, st);
    case 8:  return launch_attn<D, 8, 4, kPrefill>(a, grid, st);
    case 16: return launch_attn<D, 16, 4, kPrefill>(a, grid, st);
    case 32: return launch_attn<D, 32, 4, kPrefill>(a, grid, st);
  }
  return INFLLMV2_ERR_UNSUPPORTED;
}

// tokens per prefill tile for a group size (must match dispatch_group)
int prefill_tile_tokens(int G) {
  switch (G) {
    case 1: return 32;
    case 2: return 32;
    case 4: return 32;
    case 8: return 16;
    case 16: return 8;
    case 32: return 4;
  }
  return 0;
}

// Tree verification uses all drafts in one tile when they fit: W = 8 waves.
template <int D>
int dispatch_tree(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1:  return launch_attn<D, 1, 1, kTree>(a, grid, st);
    case 2:  return launch_attn<D, 2, 2, kTree>(a, grid, st);
    case 4:  return launch_attn<D, 4, 4, kTree>(a, grid, st);
    case 8:  return launch_attn<D, 8, 8, kTree>(a, grid, st);
    case 16: return launch_attn<D, 16, 8, kTree>(a, grid, st);
    case 32: return launch_attn<D, 32, 8, kTree>(a, grid, st);
  }
  return INFLLMV2_ERR_UNSUPPORTED;
}
int tree_tile_tokens(int G) {
  switch (G) {
    case 1: return 32;
    case 2: return 32;
    case 4: return 32;
    case 8: return 32;
    case 16: return 16;
    case 32: return 8;
  }
  return 0;
}

template <int D>
int dispatch_decode(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1:  return launch_attn<D, 1, 4, kDecode>(a, grid, st);
    case 2:  return launch_attn<D, 2, 4, kDecode>(a, grid, st);
    case 4:  return launch_attn<D, 4, 4, kDecode>(a, grid, st);
    case 8:  return launch_attn<D, 8, 4, kDecode>(a, grid, st);
    case 16: return launch_attn<D, 16, 4, kDecode>(a, grid, st);
    case 32: return launch_attn<D, 32, 4, kDecode>(a, grid, st);
  }
  return INFLLMV2_ERR_UNSUPPORTED;
}

}  // namespace

namespace infllmv2 {

// Largest number of entries (kept blocks or all blocks) one decode row walks.
int64_t decode_max_entries(int64_t max_seqlen, const Resolved& r) {
  if (max_seqlen < r.dense_len) return ceil_div(max_seqlen, r.B);
  const int64_t dense_max = ceil_div(r.dense_len > 1 ? r.dense_len - 1 : 1, r.B);
  return r.topk > dense_max ? r.topk : dense_max;
}

// Split count for `units` 64-key units: at most `max_default` splits, but
// enough that one split's entries fit the kernel's LDS list.  Callers reject
// counts above kMaxCombineSplits.
int64_t split_count(int64_t units, int64_t cpb, int64_t max_default) {
  int64_t n = units < max_default ? units : max_default;
  const int64_t need = ceil_div(units, (int64_t)(kSplitEntryCap - 1) * cpb);
  return n < need ? need : (n < 1 ? 1 : n);
}

int64_t decode_splits(int64_t max_seqlen, const Resolved& r) {
  const int64_t cpb = ceil_div(r.B, kChunk);
  return split_count(decode_max_entries(max_seqlen, r) * cpb, cpb, kMaxDecodeSplits);
}

int64_t tree_union_cap(int n_draft, int64_t n_ctx, const Resolved& r) {
  const int64_t n_b = ceil_div(n_ctx, r.B);
  const int64_t u = (int64_t)n_draft * r.topk;
  return u < n_b ? u : n_b;
}

int64_t tree_splits(int n_draft, int64_t n_ctx, const Resolved& r) {
  const int64_t n_b = ceil_div(n_ctx, r.B);
  const int64_t entries = n_ctx < r.dense_len ? n_b : tree_union_cap(n_draft, n_ctx, r);
  // + 1 entry's worth for the chunk of draft tokens
  const int64_t cpb = ceil_div(r.B, kChunk);
  const int64_t units = entries * cpb + 1;
  return split_count(units, cpb, kMaxTreeSplits);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t partial_bytes(int rows, int h_q, int d, int64_t n_split) {
  return align256((size_t)rows * h_q * n_split * (d + 2) * sizeof(float));
}

}  // namespace infllmv2

static int common_attn_checks(int dtype, int h_q, int h_kv, int d) {
  if (!dtype_ok(dtype)) return INFLLMV2_ERR_INVALID_ARG;
  INFLLMV2_TRY(check_heads(h_q, h_kv));
  if (!head_dim_ok(d)) return INFLLMV2_ERR_UNSUPPORTED;
  return INFLLMV2_OK;
}


extern "C" int infllmv2_sparse_attn_prefill(int dtype, const void* q, int32_t n_q,
                                            const void* k, const void* v, int64_t cap,
                                            int64_t n_k, int32_t h_q, int32_t h_kv, int32_t d,
                                            const int32_t* block_idx, void* out, float* lse,
                                            const infllmv2_params* p, void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if (!q || !k || !v || !out) return INFLLMV2_ERR_INVALID_ARG;
  if (n_q < 0 || n_k <= 0 || cap < n_k || n_q > n_k) return INFLLMV2_ERR_INVALID_ARG;
  if (cap > INT32_MAX) return INFLLMV2_ERR_UNSUPPORTED;
  const bool dense = n_k < r.dense_len;
  if (!dense && !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_q == 0) return INFLLMV2_OK;
  AttnArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.block_idx = dense ? nullptr : block_idx;
  a.out = (uint16_t*)out; a.lse = lse;
  a.cap = cap; a.n_k = n_k; a.n_rows = n_q; a.h_q = h_q; a.h_kv = h_kv; a.topk = r.topk;
  a.B = r.B; a.dense_len = r.dense_len; a.scale_log2 = r.scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == INFLLMV2_F32) return prefill_f32(a, d, st);
  const int G = h_q / h_kv;
  if (!group_ok_for_mfma(G)) return INFLLMV2_ERR_UNSUPPORTED;
  const int TT = prefill_tile_tokens(G);
  a.n_tiles = (int)ceil_div(n_q, TT);
  const int64_t nblocks = (int64_t)a.n_tiles * h_kv;
  if (nblocks >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
  dim3 grid((unsigned)nblocks);
  return d == 128 ? dispatch_prefill<128>(G, a, grid, st) : dispatch_prefill<64>(G, a, grid, st);
}

extern "C" int infllmv2_sparse_attn_decode(int dtype, const void* q, int32_t batch,
                                           const void* k, const void* v, int64_t cap,
                                           const int32_t* seqlens, int32_t max_seqlen,
                                           int32_t h_q, int32_t h_kv, int32_t d,
                                           const int32_t* block_idx, void* out, float* lse,
                                           void* ws, size_t ws_bytes,
                                           const infllmv2_params* p, void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if (!q || !k || !v || !out || !seqlens) return INFLLMV2_ERR_INVALID_ARG;
  if (batch < 0 || max_seqlen <= 0 || cap < max_seqlen) return INFLLMV2_ERR_INVALID_ARG;
  if (cap > INT32_MAX) return INFLLMV2_ERR_UNSUPPORTED;
  if (max_seqlen >= r.dense_len && !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return INFLLMV2_ERR_INVALID_ARG;
  if (batch == 0) return INFLLMV2_OK;
  const int64_t n_split = decode_splits(max_seqlen, r);
  if (n_split > kMaxCombineSplits) return INFLLMV2_ERR_UNSUPPORTED;
  const size_t need = partial_bytes(batch, h_q, d, n_split);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return INFLLMV2_ERR_WORKSPACE;
  AttnArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.block_idx = block_idx; a.seqlens = seqlens;
  a.out = (uint16_t*)out; a.lse = lse; a.ws = (float*)ws;
  a.cap = cap; a.n_k = max_seqlen; a.n_rows = batch; a.h_q = h_q; a.h_kv = h_kv;
  a.topk = r.topk; a.B = r.B; a.dense_len = r.dense_len; a.scale_log2 = r.scale * kLog2e;
  a.n_split = (int)n_split;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == INFLLMV2_F32) return decode_f32(a, d, st);
  const int G = h_q / h_kv;
  if (!group_ok_for_mfma(G)) return INFLLMV2_ERR_UNSUPPORTED;
  dim3 grid((unsigned)n_split, h_kv, batch);
  INFLLMV2_TRY(d == 128 ? dispatch_decode<128>(G, a, grid, st)
                        : dispatch_decode<64>(G, a, grid, st));
  if (d == 128)
    hipLaunchKernelGGL((combine_kernel<128, uint16_t>), dim3(batch * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL((combine_kernel<64, uint16_t>), dim3(batch * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

namespace infllmv2 {
size_t tree_workspace_bytes(int n_draft, int h_q, int h_kv, int d, int64_t n_ctx,
                            const Resolved& r) {
  const int64_t ucap = tree_union_cap(n_draft, n_ctx, r);
  return partial_bytes(n_draft, h_q, d, tree_splits(n_draft, n_ctx, r)) +
         align256((size_t)h_kv * ucap * 4) + align256((size_t)h_kv * ucap * 8) +
         align256((size_t)h_kv * 4);
}
size_t decode_workspace_bytes(int batch, int h_q, int d, int64_t max_seqlen,
                              const Resolved& r) {
  return partial_bytes(batch, h_q, d, decode_splits(max_seqlen, r));
}
}  // namespace infllmv2

extern "C" int infllmv2_tree_verify(int dtype, const void* q, int32_t n_draft, const void* k,
                                    const void* v, int64_t cap, int64_t n_ctx,
                                    const void* k_draft, const void* v_draft,
                                    const uint64_t* tree_mask, int32_t h_q, int32_t h_kv,
                                    int32_t d, const int32_t* block_idx, void* out, float* lse,
                                    void* ws, size_t ws_bytes, const infllmv2_params* p,
                                    void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if (!q || !k || !v || !k_draft || !v_draft || !tree_mask || !out)
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_draft < 0 || n_draft > 64 || n_ctx <= 0 || cap < n_ctx) return INFLLMV2_ERR_INVALID_ARG;
  if (cap > INT32_MAX) return INFLLMV2_ERR_UNSUPPORTED;
  const bool dense = n_ctx < r.dense_len;
  if (!dense && !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(k_draft) || !aligned16(v_draft))
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_draft == 0) return INFLLMV2_OK;
  const int64_t n_split = tree_splits(n_draft, n_ctx, r);
  if (n_split > kMaxCombineSplits) return INFLLMV2_ERR_UNSUPPORTED;
  const size_t need = tree_workspace_bytes(n_draft, h_q, h_kv, d, n_ctx, r);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return INFLLMV2_ERR_WORKSPACE;
  const int64_t ucap = tree_union_cap(n_draft, n_ctx, r);
  AttnArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.block_idx = dense ? nullptr : block_idx;
  a.k_draft = (const uint16_t*)k_draft; a.v_draft = (const uint16_t*)v_draft;
  a.tree_mask = tree_mask;
  a.out = (uint16_t*)out; a.lse = lse; a.ws = (float*)ws;
  char* tail = (char*)ws + partial_bytes(n_draft, h_q, d, n_split);
  a.union_blk = (const int32_t*)tail;
  a.union_mask = (const uint64_t*)(tail + align256((size_t)h_kv * ucap * 4));
  a.union_len = (const int32_t*)(tail + align256((size_t)h_kv * ucap * 4) +
                                 align256((size_t)h_kv * ucap * 8));
  a.union_cap = (int)ucap;
  a.cap = cap; a.n_k = n_ctx; a.n_rows = n_draft; a.h_q = h_q; a.h_kv = h_kv;
  a.topk = r.topk; a.B = r.B; a.dense_len = r.dense_len; a.scale_log2 = r.scale * kLog2e;
  a.n_split = (int)n_split;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == INFLLMV2_F32) return tree_f32(a, d, st);
  const int G = h_q / h_kv;
  if (!group_ok_for_mfma(G)) return INFLLMV2_ERR_UNSUPPORTED;
  const int TT = tree_tile_tokens(G);
  if (!dense) {
    hipLaunchKernelGGL(tree_union_kernel, dim3(h_kv), dim3(kPlanThreads), 0, st, block_idx,
                       n_draft, h_kv, r.topk, ceil_div(n_ctx, r.B), (int32_t*)a.union_blk,
                       (uint64_t*)a.union_mask, (int32_t*)a.union_len, a.union_cap);
    if (hipGetLastError() != hipSuccess) return INFLLMV2_ERR_HIP;
  }
  dim3 grid((unsigned)n_split, h_kv, (unsigned)ceil_div(n_draft, TT));
  INFLLMV2_TRY(d == 128 ? dispatch_tree<128>(G, a, grid, st) : dispatch_tree<64>(G, a, grid, st));
  if (d == 128)
    hipLaunchKernelGGL((combine_kernel<128, uint16_t>), dim3(n_draft * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL((combine_kernel<64, uint16_t>), dim3(n_draft * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}
