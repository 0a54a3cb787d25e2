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
  static constexpr int kVStride = kChunk + 4;    // bf16 elements per staged V^T row
  static constexpr int kKElems = kChunk * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kStageElems = kKElems + kVElems;
  static constexpr int kBytes = 2 * kStageElems * 2;   // double-buffered
};

// ---------------------------------------------------------------------------
// Staging of one 64-key chunk: keys [key0, key0 + nvalid) of a K/V row block.
// ---------------------------------------------------------------------------
template <int D, int NT>
struct Stager {
  static constexpr int kKPieces = kChunk * D / 8;        // 16-byte pieces of K
  static constexpr int kKPer = (kKPieces + NT - 1) / NT;
  static constexpr int kVJobs = (kChunk / 2) * (D / 8);  // (key pair, 8 dims)
  static constexpr int kVPer = (kVJobs + NT - 1) / NT;
  u32x4 kr[kKPer];
  u32x4 vr[kVPer][2];

  // kbase/vbase point at key 0 of the chunk; nvalid keys are real, the rest
  // are zero-filled so that masked lanes never multiply garbage.
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase,
                                       int nvalid, int tid) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int pc = tid + i * NT;
      const int key = pc / (D / 8), c = pc % (D / 8);
      kr[i] = (pc < kKPieces && key < nvalid) ? ldg16(kbase + (int64_t)key * D + c * 8) : z;
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int jb = tid + i * NT;
      const int kp = jb % (kChunk / 2), c = jb / (kChunk / 2);
      const int k0 = 2 * kp;
      const bool in = jb < kVJobs;
      vr[i][0] = (in && k0 < nvalid) ? ldg16(vbase + (int64_t)k0 * D + c * 8) : z;
      vr[i][1] = (in && k0 + 1 < nvalid) ? ldg16(vbase + (int64_t)(k0 + 1) * D + c * 8) : z;
    }
  }

  __device__ __forceinline__ void store(uint16_t* stage, int tid) const {
    uint16_t* Ks = stage;
    uint16_t* Vt = stage + Lds<D>::kKElems;
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int pc = tid + i * NT;
      if (pc >= kKPieces) break;
      const int key = pc / (D / 8), c = pc % (D / 8);
      *reinterpret_cast<u32x4*>(Ks + key * Lds<D>::kKStride + c * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int jb = tid + i * NT;
      if (jb >= kVJobs) break;
      const int kp = jb % (kChunk / 2), c = jb / (kChunk / 2);
      const uint32_t a[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
      const uint32_t b[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims c*8 + 2e (low halves) and c*8 + 2e + 1 (high halves)
        const uint32_t lo = (a[e] & 0xffffu) | (b[e] << 16);
        const uint32_t hi = (a[e] >> 16) | (b[e] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + 2 * e) * Lds<D>::kVStride + 2 * kp) = lo;
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + 2 * e + 1) * Lds<D>::kVStride + 2 * kp) = hi;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Per-wave online-softmax state for 32 query rows (one row per lane column).
// ---------------------------------------------------------------------------
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
  __device__ __forceinline__ void step(const uint16_t* stage, int lim, bool use_bits,
                                       uint64_t draft_bits, float scale_log2, bool tile1) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const uint16_t* Ks = stage;
    const uint16_t* Vt = stage + Lds<D>::kKElems;
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = 0.0f;
      if (kt == 1 && !tile1) continue;
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
    const bool partial = (lim >= 0 && lim < 63) || use_bits;
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
      m_new = fmaxf(m, mx);
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
      m_new = fmaxf(m, mx);
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
    bf16x8 pb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kt][t][e] = (__bf16)s[kt][8 * t + e];
    // O^T += V^T P^T; A-operand element e of half h <-> key 16t + 8(e/4) + 4h + e%4
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint16_t* vrow = Vt + (32 * dt + col) * Lds<D>::kVStride + 4 * half;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt == 1 && !tile1) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint16_t* src = vrow + 32 * kt + 16 * t;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8);
          u32x4 w = {lo.x, lo.y, hi.x, hi.y};
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&w);
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
// bitmask of the tokens (bit t) that kept each.  `sortbuf` holds N >= TT*topk
// (power of two) words; returns the union length.
template <int NT, int TT>
__device__ int build_union(const int32_t* block_idx, int tok0, int h_kv, int g, int n_tok,
                           int topk, int64_t n_b, uint32_t* sortbuf, int N, int32_t* ublk,
                           uint32_t* umask, int* scan_lds) {
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
      ublk[slot] = (int32_t)(key >> 5);
      umask[slot] = msk;
      ++slot;
    }
  }
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// The attention kernel.
//   W waves, each 32 rows = TPW tokens x G heads; TT = W * TPW tokens.
// ---------------------------------------------------------------------------
template <int D, int G, int W, int MODE>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = W * 64;
  constexpr int TPW = 32 / G;
  constexpr int TT = (MODE == kDecode) ? 1 : W * TPW;
  static_assert(TT <= 32, "token bitmask is 32 bits");
  static_assert(MODE != kPrefill || TT > 1, "prefill tiles hold several tokens");
  constexpr int SORT_N = (MODE == kPrefill) ? TT * kSortCap : 0;
  constexpr int UCAP = (MODE == kPrefill) ? TT * kSortCap : 1;
  __shared__ __attribute__((aligned(16))) uint16_t stage[2 * Lds<D>::kStageElems];
  __shared__ int32_t ublk[UCAP];
  __shared__ uint32_t umask[UCAP];
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
  int64_t n_keys;                   // keys of the sequence (context for tree)
  int tok0, n_tok;
  if constexpr (MODE == kPrefill) {
    n_keys = a.n_k;
    tok0 = tile * TT;
    n_tok = min(TT, a.n_rows - tok0);
  } else if constexpr (MODE == kDecode) {
    // lengths outside [1, max_seqlen] are clamped: wrong input, no fault
    int64_t L = a.seqlens[seq];
    n_keys = L < 1 ? 1 : (L > a.n_k ? a.n_k : L);
    tok0 = seq;
    n_tok = 1;
  } else {
    n_keys = a.n_k;
    tok0 = tile * TT;
    n_tok = min(TT, a.n_rows - tok0);
  }
  const bool dense = n_keys < a.dense_len || a.block_idx == nullptr;
  const int64_t n_b = (n_keys + a.B - 1) / a.B;
  const int cpb = (a.B + kChunk - 1) / kChunk;            // chunks per block

  // this lane's row
  const int t_in_wave = col / G, head_in_group = col % G;
  const int my_t = (MODE == kDecode) ? (wave == 0 && t_in_wave == 0 ? 0 : 32)
                                     : wave * TPW + t_in_wave;   // 32 = none
  const bool row_ok = my_t < n_tok;
  const int my_row = tok0 + (row_ok ? my_t : 0);
  const int my_head = g * G + head_in_group;
  int64_t my_pos;
  if constexpr (MODE == kPrefill) my_pos = a.n_k - a.n_rows + my_row;
  else my_pos = n_keys - 1;
  const int64_t my_bown = my_pos / a.B;

  // ---- unit list -----------------------------------------------------------
  // entries: kept blocks (or all blocks when dense), plus the draft chunk
  int n_entries;
  const int32_t* dec_list = nullptr;
  if constexpr (MODE == kPrefill) {
    if (dense) {
      const int64_t last_pos = a.n_k - a.n_rows + tok0 + n_tok - 1;
      n_entries = (int)(last_pos / a.B + 1);
    } else {
      int N = 1;
      while (N < TT * a.topk) N <<= 1;
      if (N < NT) N = NT;
      n_entries = build_union<NT, TT>(a.block_idx, tok0, a.h_kv, g, n_tok, a.topk, n_b,
                                      reinterpret_cast<uint32_t*>(stage), N, ublk, umask,
                                      scan_lds);
    }
  } else if constexpr (MODE == kDecode) {
    if (dense) {
      n_entries = (int)n_b;
    } else {
      dec_list = a.block_idx + ((int64_t)seq * a.h_kv + g) * a.topk;
      int n = 0;
      while (n < a.topk && dec_list[n] >= 0 && dec_list[n] < n_b) ++n;
      n_entries = n;
    }
  } else {
    n_entries = dense ? (int)n_b : a.union_len[g];
  }
  const bool has_draft = MODE == kTree;
  const int n_units_total = n_entries * cpb + (has_draft ? 1 : 0);
  int u_begin = 0, u_end = n_units_total;
  if constexpr (MODE != kPrefill) {
    // balanced contiguous slices of this row's units over the n_split splits
    const int per = (n_units_total + a.n_split - 1) / a.n_split;
    u_begin = min(n_units_total, split * per);
    u_end = min(n_units_total, u_begin + per);
  }

  // unit -> (block id, key0 of the chunk, #valid keys, token bitmask)
  auto unit_info = [&](int u, int64_t& key0, int& nvalid, uint32_t& tmask, bool& is_draft) {
    is_draft = has_draft && u == n_entries * cpb;
    if (is_draft) {
      key0 = 0;
      nvalid = a.n_rows;
      tmask = 0xffffffffu;
      return;
    }
    const int e = u / cpb, c = u % cpb;
    int64_t b;
    if (dense) {
      b = e;
      // token t keeps block b iff b <= its own block
      tmask = 0;
      if constexpr (MODE == kPrefill) {
        const int64_t p0 = a.n_k - a.n_rows + tok0;
        for (int t = 0; t < n_tok; ++t)
          if (b <= (p0 + t) / a.B) tmask |= 1u << t;
      } else {
        tmask = (1u << n_tok) - 1u;
        if (n_tok == 32) tmask = 0xffffffffu;
      }
    } else if constexpr (MODE == kPrefill) {
      b = ublk[e];
      tmask = umask[e];
    } else if constexpr (MODE == kDecode) {
      b = dec_list[e];
      tmask = 1u;
    } else {
      b = a.union_blk[(int64_t)g * a.union_cap + e];
      tmask = (uint32_t)(a.union_mask[(int64_t)g * a.union_cap + e] >> tok0);
    }
    key0 = b * a.B + (int64_t)c * kChunk;
    const int64_t blk_end = min((b + 1) * (int64_t)a.B, n_keys);
    const int64_t nv = blk_end - key0;
    nvalid = nv > kChunk ? kChunk : (nv < 0 ? 0 : (int)nv);
  };

  const int64_t kv_head_off = (MODE == kDecode ? ((int64_t)seq * a.h_kv + g) : (int64_t)g) *
                              a.cap * D;
  const uint16_t* kbase_seq = a.k + kv_head_off;
  const uint16_t* vbase_seq = a.v + kv_head_off;
  const uint16_t* kdraft = has_draft ? a.k_draft + (int64_t)g * a.n_rows * D : nullptr;
  const uint16_t* vdraft = has_draft ? a.v_draft + (int64_t)g * a.n_rows * D : nullptr;

  RowState<D> st;
  st.init();
  load_q<D>(st, row_ok ? a.q + ((int64_t)my_row * a.h_q + my_head) * D : nullptr);
  uint64_t my_bits = 0;
  if (has_draft && row_ok) {
    const uint64_t full = a.n_rows >= 64 ? ~0ull : ((1ull << a.n_rows) - 1ull);
    my_bits = (a.tree_mask[my_row] & full) | (1ull << my_row);
  }

  Stager<D, NT> sg;
  if (u_begin < u_end) {
    int64_t key0; int nv; uint32_t tm; bool isd;
    unit_info(u_begin, key0, nv, tm, isd);
    sg.load(isd ? kdraft : kbase_seq + key0 * D, isd ? vdraft : vbase_seq + key0 * D, nv, tid);
  }
  for (int u = u_begin; u < u_end; ++u) {
    uint16_t* buf = stage + ((u - u_begin) & 1) * Lds<D>::kStageElems;
    sg.store(buf, tid);
    __syncthreads();
    int64_t key0; int nv; uint32_t tm; bool isd;
    unit_info(u, key0, nv, tm, isd);
    if (u + 1 < u_end) {
      int64_t k1; int n1; uint32_t t1; bool d1;
      unit_info(u + 1, k1, n1, t1, d1);
      sg.load(d1 ? kdraft : kbase_seq + k1 * D, d1 ? vdraft : vbase_seq + k1 * D, n1, tid);
    }
    // which of my rows use this chunk, and up to which key offset
    const bool keep = row_ok && ((tm >> my_t) & 1u);
    int lim = -1;
    if (keep) {
      if (isd) {
        lim = nv - 1;
      } else {
        const int64_t last = min(my_pos, key0 + nv - 1) - key0;
        lim = last < 0 ? -1 : (int)last;
      }
    }
    if (__ballot(lim >= 0)) st.step(buf, lim, isd, my_bits, a.scale_log2, nv > 32);
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

template <int D, int G, int W, int MODE>
int launch_attn(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, G, W, MODE>), grid, dim3(W * 64), 0, st, a);
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

int64_t decode_splits(int64_t max_seqlen, const Resolved& r) {
  const int64_t units = decode_max_entries(max_seqlen, r) * ceil_div(r.B, kChunk);
  return units < kMaxDecodeSplits ? units : kMaxDecodeSplits;
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
  return units < kMaxTreeSplits ? units : kMaxTreeSplits;
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
  if (max_seqlen >= r.dense_len && !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return INFLLMV2_ERR_INVALID_ARG;
  if (batch == 0) return INFLLMV2_OK;
  const int64_t n_split = decode_splits(max_seqlen, r);
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
  const bool dense = n_ctx < r.dense_len;
  if (!dense && !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(k_draft) || !aligned16(v_draft))
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_draft == 0) return INFLLMV2_OK;
  const size_t need = tree_workspace_bytes(n_draft, h_q, h_kv, d, n_ctx, r);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return INFLLMV2_ERR_WORKSPACE;
  const int64_t n_split = tree_splits(n_draft, n_ctx, r);
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
