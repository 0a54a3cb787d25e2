// Top-k block selection shared by the selection kernels: arguments, the
// workgroup scan, the ballot threshold search and the workgroup-per-row
// selection (one 256-thread workgroup selects one (row, KV head)).
// Sources: "MiniCPM 4.0" blog (shadowrocket9.top), InfLLM v2 section (each
// query keeps its top-k most relevant blocks, k = 64); "MiniCPM4: running
// LLMs on phones and PCs" (xugj520.cn), section 1.1 (initial tokens and a
// sliding window are always kept).
#pragma once

#include "device_common.h"

namespace infllmv2 {

constexpr int kTopkThreads = 256;

struct TopkArgs {
  const float* scores;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const int32_t* seqlens;
  int32_t* block_idx;
  int64_t nb_cap;
  int h_kv, B, topk, init, local, dense_len, batch;
};

// Exclusive prefix sum over the 256 threads of the workgroup (thread order).
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* lds4) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds4[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int t = lds4[w];
    if (w < wid) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// ---------------------------------------------------------------------------
// Keys a wave keeps in LDS for the threshold search after the lower-bound filter.
constexpr int kSurvivors = 256;
constexpr int kMaxTopk = 128;          // the host rejects larger topk
// up to this many (row, KV head) units a workgroup per row beats a wave per row
constexpr int kFewRows = 512;

// Set bits of a wave mask in the lanes below this one (v_mbcnt).
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// k-th largest (1 <= k <= 64) of one value per lane: bitonic sort across the
// wave (ascending), then the value at lane 64 - k; *largest = the maximum.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, int k, int lane,
                                                     uint32_t* largest) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t other = (uint32_t)__shfl_xor((int)v, stride, 64);
      const bool up = (lane & size) == 0;
      const bool low = (lane & stride) == 0;
      const uint32_t mn = v < other ? v : other, mx = v < other ? other : v;
      v = (low == up) ? mn : mx;
    }
  }
  *largest = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 64 - k);
}

// Largest (MAX) or smallest value over the wave, in every lane: row
// reductions by DPP, then the cross-row swaps.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extreme_u32(uint32_t v) {
  auto pick = [](uint32_t x, uint32_t y) { return (MAX ? x > y : x < y) ? x : y; };
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false)); // row half mirror
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false)); // row mirror
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = pick(s16[0], s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return pick(s32[0], s32[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_extreme_u32<true>(v); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_extreme_u32<false>(v); }

// Exclusive prefix sum over the lanes of a wave; *total = sum over all lanes.
__device__ __forceinline__ int wave_excl_scan(int v, int* total, int lane) {
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  *total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Largest T with #(key >= T) >= need over the wave's N keys per lane (keys
// of 0 never count), found bit by bit from the top; *exact is set when the
// count reaches need exactly (then T is the need-th largest and no tie
// remains to break).  The keys may be only those >= lo (a lower bound of the
// answer): below lo the counts are too small, which never changes a
// `cnt >= need` decision there (all of them pass), but an exact count only
// means something at candidates >= lo.  T lies in [lo, hi] (hi = the largest
// key), so it shares the bits above the highest bit where lo and hi differ:
// the search starts there, from those common bits.
template <int N>
__device__ __forceinline__ uint32_t threshold_search(const uint32_t (&key)[N], int need,
                                                     uint32_t lo, uint32_t hi, bool* exact) {
  // lo and hi are the same in every lane: scalar registers keep the loop's
  // candidate and counts off the vector ALU
  lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)lo);
  hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)hi);
  const uint32_t diff = lo ^ hi;
  const int top = diff ? 31 - __builtin_clz(diff) : -1;
  uint32_t T = top >= 0 ? lo & ~((2u << top) - 1u) : lo;
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) cnt += __popcll(__ballot(key[j] >= cand));
    if (cnt >= need) {
      T = cand;
      if (cnt == need && cand >= lo) { *exact = true; break; }
    }
  }
  return T;
}

template <int N>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&x)[N], int c) {
  uint32_t v = 0u;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    int ahead = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) ahead += (x[i] > x[j]) || (i < j && x[i] == x[j]);
    v = ahead == c - 1 ? x[j] : v;
  }
  return v;
}

// Selection of one (row, KV head) by one 256-thread workgroup (every thread
// of the workgroup calls it; it synchronises the workgroup).  KPT consecutive
// blocks per thread, so rows of up to 256 * KPT eligible blocks.
template <int KPT>
__device__ __forceinline__ void topk_block_core(const TopkArgs& a, int r, int g, int64_t pos);

template <int KPT>
__device__ __forceinline__ void topk_block_row(const TopkArgs& a, const int r, const int g) {
  const int tid = threadIdx.x;
  int32_t* out = a.block_idx + ((int64_t)r * a.h_kv + g) * a.topk;
  const int seq = a.row_seq ? a.row_seq[r] : 0;
  bool skip = seq < 0 || seq >= a.batch;
  const int64_t L = skip ? 0 : a.seqlens[seq];
  const int64_t pos = a.row_pos ? a.row_pos[r] : L - 1;
  skip = skip || L < a.dense_len || pos < 0 || pos >= L || pos / a.B + 1 > a.nb_cap;
  if (skip) {
    for (int i = tid; i < a.topk; i += kTopkThreads) out[i] = -1;
    return;
  }
  topk_block_core<KPT>(a, r, g, pos);
}

// The selection of a sparse row whose position is known to be valid
// (0 <= pos < its length, pos / B < nb_cap); every thread of the workgroup
// calls it.
template <int KPT>
__device__ __forceinline__ void topk_block_core(const TopkArgs& a, const int r, const int g,
                                                const int64_t pos) {
  __shared__ uint32_t surv[kSurvivors];
  __shared__ int scan4[kTopkThreads / 64];
  __shared__ uint32_t wave_lo[kTopkThreads / 64], wave_hi[kTopkThreads / 64];
  __shared__ uint32_t sh_T, sh_hi;
  __shared__ int sh_exact;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* out = a.block_idx + ((int64_t)r * a.h_kv + g) * a.topk;
  const int b_own = (int)(pos / a.B);
  const int n_elig = b_own + 1;
  if (n_elig <= a.topk) {
    for (int i = tid; i < a.topk; i += kTopkThreads) out[i] = i < n_elig ? i : -1;
    return;
  }
  const int f_init = a.init < n_elig ? a.init : n_elig;
  const int f_lo = b_own - a.local + 1 > 0 ? b_own - a.local + 1 : 0;
  const int overlap = f_init > f_lo ? f_init - f_lo : 0;
  const int n_forced = f_init + (n_elig - f_lo) - overlap;
  const int need = a.topk - n_forced;
  const float* S = a.scores + ((int64_t)r * a.h_kv + g) * a.nb_cap;

  uint32_t key[KPT];
  uint32_t forced_bits = 0u, mx = 0u;
  const int b0 = KPT * tid;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int b = b0 + j;
    const float x = S[b < n_elig ? b : n_elig - 1];
    const uint32_t k = orderable_key(x);
    key[j] = (b < n_elig && b >= f_init && b < f_lo) ? (k == 0 ? 1u : k) : 0u;
    forced_bits |= (b < n_elig && (b < f_init || b >= f_lo)) ? (1u << j) : 0u;
    mx = key[j] > mx ? key[j] : mx;
  }

  uint32_t T = 0u;
  bool exact = need <= 0;
  if (need > 0) {
    // Lower bound.  Only the first n_act threads hold eligible blocks; with
    // c = ceil(need / n_act) keys per thread, let v be each thread's c-th
    // largest key: any x with ceil(need / c) threads at v >= x has at least
    // need keys >= x, so the ceil(need / c)-th largest v bounds the threshold
    // from below (c = 1: the thread maxima).  Wave 0 finds it with the
    // bitwise search over the 256 values (4 per lane), starting below the
    // bits they all share.  A row of at most kSurvivors eligible blocks
    // needs no bound: all its keys (>= 1) survive.  hi is the row's largest
    // key.
    uint32_t lo = 0u, hi = 0xffffffffu;
    if (need <= kTopkThreads) {
      const int n_act = (n_elig + KPT - 1) / KPT;
      const int c = min(KPT, (need + n_act - 1) / n_act);
      const int need_t = (need + c - 1) / c;
      surv[tid] = c > 1 ? kth_largest<KPT>(key, c) : mx;   // surv is free until the survivors
      uint32_t wm = mx;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t y = (uint32_t)__shfl_xor((int)wm, o, 64);
        wm = y > wm ? y : wm;
      }
      if (lane == 0) wave_hi[wv] = wm;
      __syncthreads();
      if (wv == 0) {
        uint32_t m4[kTopkThreads / 64];
        uint32_t mn = 0xffffffffu, mxx = 0u, top = 0u;
#pragma unroll
        for (int j = 0; j < kTopkThreads / 64; ++j) {
          m4[j] = surv[lane + 64 * j];
          mn = m4[j] < mn ? m4[j] : mn;
          mxx = m4[j] > mxx ? m4[j] : mxx;
          top = wave_hi[j] > top ? wave_hi[j] : top;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const uint32_t a1 = (uint32_t)__shfl_xor((int)mn, o, 64);
          const uint32_t a2 = (uint32_t)__shfl_xor((int)mxx, o, 64);
          mn = a1 < mn ? a1 : mn;
          mxx = a2 > mxx ? a2 : mxx;
        }
        bool ex = false;
        const uint32_t wl = n_elig <= kSurvivors
                                ? 1u
                                : threshold_search<kTopkThreads / 64>(m4, need_t, mn, mxx, &ex);
        if (lane == 0) { wave_lo[0] = wl; sh_hi = top; }
      }
      __syncthreads();
      lo = wave_lo[0];
      hi = sh_hi;
    }
    int mine = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) mine += key[j] >= lo && key[j] != 0u;
    int total;
    const int off = block_exclusive_scan(mine, &total, scan4);
    if (lo != 0u && total <= kSurvivors) {
      for (int i = tid; i < kSurvivors; i += kTopkThreads) surv[i] = 0u;
      __syncthreads();
      int o = off;
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (key[j] >= lo && key[j] != 0u) surv[o++] = key[j];
      __syncthreads();
      if (wv == 0) {
        uint32_t sk[kSurvivors / 64];
#pragma unroll
        for (int j = 0; j < kSurvivors / 64; ++j) sk[j] = surv[lane + 64 * j];
        bool ex = false;
        const uint32_t t = threshold_search<kSurvivors / 64>(sk, need, lo, hi, &ex);
        if (lane == 0) { sh_T = t; sh_exact = ex ? 1 : 0; }
      }
    } else {
      // block-wide bitwise search over all keys
      if (tid == 0) { sh_T = 0u; sh_exact = 0; }
      __syncthreads();
      uint32_t t = 0u;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = t | (1u << bit);
        int c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += key[j] >= cand;
        int cnt;
        (void)block_exclusive_scan(c, &cnt, scan4);
        if (cnt >= need) {
          t = cand;
          if (cnt == need) { if (tid == 0) sh_exact = 1; break; }
        }
      }
      if (tid == 0) sh_T = t;
    }
    __syncthreads();
    T = sh_T;
    exact = sh_exact != 0;
  }
  // selection: forced, keys > T, and of the keys == T the lowest-indexed
  // `take` ones (rank from a block scan of the per-thread tie counts)
  int take = 0;
  int eq_before = 0;
  if (!exact) {
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      gt += key[j] > T;
      eq += key[j] == T;
    }
    int gt_tot, eq_tot;
    (void)block_exclusive_scan(gt, &gt_tot, scan4);
    eq_before = block_exclusive_scan(eq, &eq_tot, scan4);
    take = need - gt_tot;
  }
  uint32_t sel_bits = 0u;
  int rank = eq_before;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool forced = (forced_bits >> j) & 1u;
    bool sel;
    if (need <= 0) {
      sel = forced;
    } else if (exact) {
      sel = forced || key[j] >= T;
    } else {
      const bool tie = key[j] == T;
      sel = forced || key[j] > T || (tie && rank < take);
      rank += tie ? 1 : 0;
    }
    sel_bits |= sel ? (1u << j) : 0u;
  }
  int n_sel;
  int slot = block_exclusive_scan(__popc(sel_bits), &n_sel, scan4);
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((sel_bits >> j) & 1u) {
      if (slot < a.topk) out[slot] = b0 + j;
      ++slot;
    }
  for (int i = n_sel + tid; i < a.topk; i += kTopkThreads) out[i] = -1;
}

}  // namespace infllmv2
