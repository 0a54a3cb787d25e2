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
#include "host_common.h"
#include "topk_common.h"

namespace infllmv2 {

constexpr int kTopkLdsKeys = 8192;

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
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void select_topk_block_kernel(TopkArgs a) {
  topk_block_row<KPT>(a, blockIdx.x / a.h_kv, blockIdx.x % a.h_kv);
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
