// Top-k block selection with forced initial and local blocks.
// Sources: "MiniCPM 4.0" blog (shadowrocket9.top), InfLLM v2 section (each
// query keeps its top-k most relevant blocks, k = 64); "MiniCPM4: running
// LLMs on phones and PCs" (xugj520.cn), section 1.1 (initial tokens and a
// sliding window are always kept).
//
// One workgroup per (row, KV head).  Scores become order-preserving uint32
// keys (staged in LDS when they fit); an MSB-first radix select (four 8-bit
// digits, LDS histogram, suffix scan to pick the digit) finds the threshold
// key T of the need-th best non-forced block.  Blocks with key > T are kept,
// and of the blocks with key == T the lowest-indexed ones fill the rest, which
// gives exactly the (score descending, index ascending) order.  An ordered
// scan then writes the kept block ids in ascending order.
#include "device_common.h"
#include "host_common.h"

namespace infllmv2 {

constexpr int kTopkThreads = 256;
constexpr int kTopkLdsKeys = 8192;

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

__global__ __launch_bounds__(kTopkThreads) void select_topk_kernel(TopkArgs a) {
  __shared__ uint32_t keys[kTopkLdsKeys];
  __shared__ int hist[256];
  __shared__ int scan4[kTopkThreads / 64];
  __shared__ int sh_digit, sh_below;

  const int r = blockIdx.x / a.h_kv, g = blockIdx.x % a.h_kv;
  const int tid = threadIdx.x;
  int32_t* out = a.block_idx + ((int64_t)r * a.h_kv + g) * a.topk;
  const int seq = a.row_seq ? a.row_seq[r] : 0;
  bool skip = seq < 0 || seq >= a.batch;
  int64_t L = skip ? 0 : a.seqlens[seq];
  const int64_t pos = a.row_pos ? a.row_pos[r] : L - 1;
  skip = skip || L < a.dense_len || pos < 0 || pos >= L || pos / a.B + 1 > a.nb_cap;
  if (skip) {                       // dense (or malformed) row: nothing selected
    for (int i = tid; i < a.topk; i += kTopkThreads) out[i] = -1;
    return;
  }
  const int64_t b_own = pos / a.B;
  const int64_t n_elig = b_own + 1;
  if (n_elig <= a.topk) {           // every eligible block fits
    for (int i = tid; i < a.topk; i += kTopkThreads) out[i] = i < n_elig ? i : -1;
    return;
  }
  // forced = [0, init) U [b_own - local + 1, b_own], all inside [0, n_elig)
  const int64_t f_init = a.init < n_elig ? a.init : n_elig;
  const int64_t f_lo = b_own - a.local + 1 > 0 ? b_own - a.local + 1 : 0;
  const int64_t overlap = (f_init > f_lo) ? f_init - f_lo : 0;
  const int64_t n_forced = f_init + (n_elig - f_lo) - overlap;
  const int need = a.topk - (int)n_forced;      // topk >= init + local >= n_forced
  auto forced = [&](int64_t b) { return b < f_init || b >= f_lo; };

  const float* S = a.scores + ((int64_t)r * a.h_kv + g) * a.nb_cap;
  const bool in_lds = n_elig <= kTopkLdsKeys;
  if (in_lds) {
    for (int64_t b = tid; b < n_elig; b += kTopkThreads) keys[b] = orderable_key(S[b]);
    __syncthreads();
  }
  auto key_of = [&](int64_t b) -> uint32_t {
    return in_lds ? keys[b] : orderable_key(S[b]);
  };

  // radix select of the need-th largest key among non-forced blocks
  uint32_t prefix = 0, pmask = 0;
  int krem = need;
  if (need > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int64_t b = tid; b < n_elig; b += kTopkThreads) {
        if (forced(b)) continue;
        const uint32_t k = key_of(b);
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      // suffix sums: thread t holds count of digits >= 255 - t ... via reversed scan
      const int rev = 255 - tid;
      const int c = hist[rev];
      int tot;
      const int excl = block_exclusive_scan(c, &tot, scan4);   // keys with digit > rev
      if (excl < krem && excl + c >= krem) {
        sh_digit = rev;
        sh_below = excl;
      }
      __syncthreads();
      const int dgt = sh_digit;
      krem -= sh_below;
      prefix |= (uint32_t)dgt << shift;
      pmask |= 0xffu << shift;
      __syncthreads();
    }
  }
  const uint32_t T = prefix;
  // krem = how many blocks with key == T to keep (lowest index first)

  // ordered walk: thread t owns the contiguous range [t*C, t*C + C)
  const int64_t C = (n_elig + kTopkThreads - 1) / kTopkThreads;
  const int64_t c0 = tid * C;
  const int64_t c1 = c0 + C < n_elig ? c0 + C : n_elig;
  int n_eq = 0;
  if (need > 0)
    for (int64_t b = c0; b < c1; ++b)
      if (!forced(b) && key_of(b) == T) ++n_eq;
  int tot;
  const int eq_base = block_exclusive_scan(n_eq, &tot, scan4);
  auto kept = [&](int64_t b, int& eq_seen) -> bool {
    if (forced(b)) return true;
    if (need == 0) return false;
    const uint32_t k = key_of(b);
    if (k > T) return true;
    if (k == T) return eq_base + (eq_seen++) < krem;
    return false;
  };
  int n_sel = 0, eq_seen = 0;
  for (int64_t b = c0; b < c1; ++b) n_sel += kept(b, eq_seen) ? 1 : 0;
  const int sel_base = block_exclusive_scan(n_sel, &tot, scan4);
  eq_seen = 0;
  int slot = sel_base;
  for (int64_t b = c0; b < c1; ++b)
    if (kept(b, eq_seen) && slot < a.topk) out[slot++] = (int32_t)b;
  for (int i = tot + tid; i < a.topk; i += kTopkThreads) out[i] = -1;
}


// ---------------------------------------------------------------------------
// One wave per (row, KV head) when the eligible blocks fit in registers
// (64 * KPL of them).  Keys live in registers (KPL per lane, block
// b = lane + 64 j); a bitwise search builds the threshold T from the most
// significant bit down, counting keys >= candidate with ballots and scalar
// popcounts -- no LDS atomics, no barriers.  The search stops early as soon
// as some candidate admits exactly `need` keys.  The ascending output order
// comes from ballot prefix counts (block b = lane + 64 j precedes b' when
// j < j', or j == j' and lane < lane').
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

template <int KPL>
__global__ __launch_bounds__(256) void select_topk_wave_kernel(TopkArgs a, int n_units) {
  // per wave: survivors (+ one dummy slot per lane) and the ordered selection
  // (+ one dummy slot per lane), so that no lane needs a branch to write
  __shared__ uint32_t surv[4][kSurvivors + 64];
  __shared__ int32_t sel_lds[4][kMaxTopk + 64];
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= n_units) return;                   // whole wave leaves
  const int lane = threadIdx.x & 63;
  const int r = unit / a.h_kv, g = unit % a.h_kv;
  int32_t* out = a.block_idx + ((int64_t)r * a.h_kv + g) * a.topk;
  const int seq = a.row_seq ? a.row_seq[r] : 0;
  bool skip = seq < 0 || seq >= a.batch;
  const int64_t L = skip ? 0 : a.seqlens[seq];
  const int64_t pos = a.row_pos ? a.row_pos[r] : L - 1;
  skip = skip || L < a.dense_len || pos < 0 || pos >= L || pos / a.B + 1 > a.nb_cap;
  if (skip) {
    for (int i = lane; i < a.topk; i += 64) out[i] = -1;
    return;
  }
  const int b_own = (int)(pos / a.B);
  const int n_elig = b_own + 1;
  if (n_elig <= a.topk) {
    for (int i = lane; i < a.topk; i += 64) out[i] = i < n_elig ? i : -1;
    return;
  }
  const int f_init = a.init < n_elig ? a.init : n_elig;
  const int f_lo = b_own - a.local + 1 > 0 ? b_own - a.local + 1 : 0;
  const int overlap = f_init > f_lo ? f_init - f_lo : 0;
  const int n_forced = f_init + (n_elig - f_lo) - overlap;
  const int need = a.topk - n_forced;
  const float* S = a.scores + ((int64_t)r * a.h_kv + g) * a.nb_cap;

  // Here n_elig > topk >= init + local, so the forced blocks are the two
  // disjoint runs [0, f_init) and [f_lo, n_elig), and the candidates are
  // exactly the blocks in between: [f_init, f_lo).  The output is the first
  // run, the chosen candidates in ascending order, then the second run.
  // key 0 = not a candidate; candidates >= 1.  Every lane loads (an in-range
  // index), then selects: no divergent branch.
  // Entries past n_elig but inside the row (< nb_cap) are read as they are
  // and never become candidates, so a row of at least 64 * KPL entries needs
  // no index clamp.
  uint32_t key[KPL];
  const uint32_t span = (uint32_t)(f_lo - f_init);
  auto prep = [&](int j, float x) {
    const uint32_t k = orderable_key(x);
    key[j] = (uint32_t)(lane + 64 * j - f_init) < span ? (k > 1u ? k : 1u) : 0u;
  };
  if (a.nb_cap >= 64 * KPL) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) prep(j, S[lane + 64 * j]);
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int b = lane + 64 * j;
      prep(j, S[b < n_elig ? b : n_elig - 1]);
    }
  }
  // T = largest value with #(key >= T) >= need (the need-th largest key)
  uint32_t T = 0;
  bool exact = need <= 0;       // nothing to choose, or #(key >= T) == need
  if (need > 0) {
    // Lower bound: at least `need` lanes hold a key >= the need-th largest
    // lane maximum, so T >= it and smaller keys cannot matter.  The keys at
    // or above it usually number a few hundred: the search then runs on them
    // (kSurvivors per wave in LDS) instead of on all 64 * KPL keys.
    uint32_t lo = 0, hi = 0xffffffffu;
    if (need <= 64) {
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) mx = key[j] > mx ? key[j] : mx;
      lo = wave_kth_largest(mx, need, lane, &hi);
    }
    int mine = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) mine += key[j] >= lo && key[j] != 0u;
    int total;
    const int off = wave_excl_scan(mine, &total, lane);
    uint32_t* sv = surv[threadIdx.x >> 6];
    if (lo != 0u && total <= kSurvivors) {
      for (int i = lane; i < kSurvivors; i += 64) sv[i] = 0u;
      __builtin_amdgcn_wave_barrier();
      int o = off;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const bool keep = key[j] >= lo && key[j] != 0u;
        sv[keep ? o : kSurvivors + lane] = key[j];
        o += keep ? 1 : 0;
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t sk[kSurvivors / 64];
#pragma unroll
      for (int j = 0; j < kSurvivors / 64; ++j) sk[j] = sv[lane + 64 * j];
      T = threshold_search<kSurvivors / 64>(sk, need, lo, hi, &exact);
    } else {
      T = threshold_search<KPL>(key, need, 0u, hi, &exact);
    }
  }
  // keys > T are kept; of the keys == T the lowest-indexed ones fill the rest
  int take = 0;
  if (!exact) {
    int gt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) gt += __popcll(__ballot(key[j] > T));
    take = need - gt;
  }
  // chosen candidates go to slots f_init, f_init + 1, ... in ascending order;
  // the two forced runs fill the slots around them.  Separate loops on
  // wave-uniform conditions keep the unrolled bodies free of branches.
  const int wv = threadIdx.x >> 6;
  int base = f_init;
  const int lim = f_init + (need > 0 ? need : 0);
  auto emit = [&](int j, bool sel) {
    const uint64_t selm = __ballot(sel);
    const int slot = base + lanes_below(selm);
    const int ok = (int)sel & (int)(slot < lim);            // no short-circuit branch
    sel_lds[wv][ok ? slot : kMaxTopk + lane] = lane + 64 * j;
    base += __popcll(selm);
  };
  const int mode = __builtin_amdgcn_readfirstlane(need <= 0 ? 0 : (exact ? 1 : 2));
  if (mode == 1) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) emit(j, key[j] >= T);
  } else if (mode == 2) {
    int eq_seen = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const uint64_t eqm = __ballot(key[j] == T);
      const int rank = eq_seen + lanes_below(eqm);
      eq_seen += __popcll(eqm);
      emit(j, (int)(key[j] > T) | ((int)(key[j] == T) & (int)(rank < take)));
    }
  }
  __builtin_amdgcn_wave_barrier();
  // slots: [0, f_init) init run, [f_init, lim) chosen, then the local run
  const int n_local = n_elig - f_lo;
  for (int i = lane; i < a.topk; i += 64) {
    int v = -1;
    if (i < f_init) v = i;
    else if (i < lim) v = sel_lds[wv][i];
    else if (i < lim + n_local) v = f_lo + (i - lim);
    out[i] = v;
  }
}

// ---------------------------------------------------------------------------
// Few rows (decode, tree verification): one 256-thread workgroup per (row,
// KV head), so a row's work is spread over four waves instead of one.
// Thread t owns the KPT consecutive blocks [KPT t, KPT t + KPT) (coalesced
// loads; ascending block order = thread order, so ties and the output order
// come from block prefix scans).
//   lower bound: each wave's need-th largest lane maximum is a lower bound of
//     the threshold (that wave alone holds `need` keys at or above it), so is
//     their maximum;
//   keys at or above it (<= kSurvivors) go to LDS and wave 0 runs the bitwise
//     threshold search on them; a full block-wide search is the fallback.
// ---------------------------------------------------------------------------
// c-th largest (1 <= c <= N) of N values: the one with exactly c - 1 values
// ahead of it in (value descending, index ascending) order.
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

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void select_topk_block_kernel(TopkArgs a) {
  __shared__ uint32_t surv[kSurvivors];
  __shared__ int scan4[kTopkThreads / 64];
  __shared__ uint32_t wave_lo[kTopkThreads / 64], wave_hi[kTopkThreads / 64];
  __shared__ uint32_t sh_T, sh_hi;
  __shared__ int sh_exact;
  const int r = blockIdx.x / a.h_kv, g = blockIdx.x % a.h_kv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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

using namespace infllmv2;

extern "C" int infllmv2_select_topk(const float* scores, int32_t rows,
                                    const int32_t* row_seq, const int32_t* row_pos,
                                    int32_t h_kv, int64_t nb_cap, const int32_t* seqlens,
                                    int32_t batch, int32_t* block_idx,
                                    const infllmv2_params* p, void* stream) {
  if (!scores || !seqlens || !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (rows < 0 || h_kv <= 0 || nb_cap <= 0 || batch <= 0) return INFLLMV2_ERR_INVALID_ARG;
  Resolved r;
  INFLLMV2_TRY(check_params(p, 128, &r));
  if (rows == 0) return INFLLMV2_OK;
  if ((int64_t)rows * h_kv >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
  TopkArgs a;
  a.scores = scores; a.row_seq = row_seq; a.row_pos = row_pos; a.seqlens = seqlens;
  a.block_idx = block_idx; a.nb_cap = nb_cap; a.h_kv = h_kv; a.B = r.B; a.topk = r.topk;
  a.init = r.init; a.local = r.local; a.dense_len = r.dense_len; a.batch = batch;
  const int n_units = rows * h_kv;
  hipStream_t st = (hipStream_t)stream;
  // few rows: a workgroup per row (KPT consecutive blocks per thread)
  if (n_units <= kFewRows && nb_cap <= (int64_t)kTopkThreads * 16) {
    if (nb_cap <= kTopkThreads * 8)
      hipLaunchKernelGGL(select_topk_block_kernel<8>, dim3((unsigned)n_units),
                         dim3(kTopkThreads), 0, st, a);
    else
      hipLaunchKernelGGL(select_topk_block_kernel<16>, dim3((unsigned)n_units),
                         dim3(kTopkThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
  }
  // eligible blocks per row <= nb_cap: registers hold 64 * KPL keys per wave
  if (nb_cap <= 64 * 32)
    hipLaunchKernelGGL(select_topk_wave_kernel<32>, dim3((unsigned)((n_units + 3) / 4)),
                       dim3(256), 0, st, a, n_units);
  else if (nb_cap <= 64 * 64)
    hipLaunchKernelGGL(select_topk_wave_kernel<64>, dim3((unsigned)((n_units + 3) / 4)),
                       dim3(256), 0, st, a, n_units);
  else
    hipLaunchKernelGGL(select_topk_kernel, dim3((unsigned)n_units), dim3(kTopkThreads), 0, st,
                       a);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}
