// Top-k block selection helpers: arguments, the workgroup scan, wave
// reductions and the ballot threshold search.
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
  const int32_t* row_seq;     // NULL: row r is sequence r if row_is_seq, else 0
  const int32_t* row_pos;
  const int32_t* seqlens;     // NULL: every sequence has length fixed_len
  int32_t* block_idx;
  int64_t nb_cap;
  int64_t fixed_len;
  int h_kv, B, topk, init, local, dense_len, batch, row_is_seq;
};

// Queues the selection of rows * h_kv rows (host side, topk.hip).
int launch_select_topk(const TopkArgs& a, int rows, hipStream_t st);

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
constexpr int kMaxTopk = 128;          // the host rejects larger topk

// Set bits of a wave mask in the lanes below this one (v_mbcnt).
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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

}  // namespace infllmv2
