// Top-k block selection with forced initial and local blocks.
// Sources: "MiniCPM 4.0" blog (shadowrocket9.top), InfLLM v2 section (each
// query keeps its top-k most relevant blocks, k = 64); "MiniCPM4: running
// LLMs on phones and PCs" (xugj520.cn), section 1.1 (initial tokens and a
// sliding window are always kept).
//
// Rows of up to 4096 eligible blocks take one wave per (row, KV head)
// (select_topk_wave_kernel, below).  Longer rows: one workgroup per (row,
// KV head).  Scores become order-preserving uint32
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
// (64 * KPL of them): lane l holds the scores of blocks b = l + 64 j
// (coalesced loads; ascending block order is (j, lane) order).
//   1. Non-candidates (forced blocks, blocks past the row) become NaN, which
//      no comparison admits; only the 64-block pieces that reach them are
//      touched.
//   2. Lower bound lo: at least `need` lanes hold a score >= the need-th
//      largest lane maximum, so the threshold is >= it.  A bitwise search
//      over the 64 lane-maximum keys finds it.
//   3. Survivors (score >= lo, typically 100-260 of 2048) are compacted
//      into LDS as (score, block) in ascending block order, from ballots.
//   4. The threshold T (the need-th largest survivor key), the ranks of the
//      ties at T (lowest index first) and the output slots all come from
//      ballots over the survivors, at most kWaveSurvivors / 64 per lane.
// Rows where the bound is not finite (fewer than `need` finite lane maxima,
// or need > 64) or whose survivors overflow take a search over every key.
// Scores compare as floats in steps 1-3 (-0 == +0); keys are the
// order-preserving uint32 images, NaN candidates ranking below -inf.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float vmax3(float x, float y, float z) {
  // plain v_max3_f32: NaN operands are ignored, and no canonicalising
  // instructions are inserted for loaded values
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

constexpr int kWaveSurvivors = 512;   // per wave; a 2048-block row keeps ~100-260

// The k-th largest of one key per lane (1 <= k <= 64; hi = the largest).
// Close to either end (top-64 rows need the 61st largest = 4th smallest,
// top-6 rows the 3rd largest), a few wave extrema, each removing all lanes
// equal to it, find it; otherwise the bitwise search, whose early stop may
// land between two lane values, then the smallest lane value at or above.
__device__ __forceinline__ uint32_t kth_largest_of_lanes(uint32_t v, int k, uint32_t hi) {
  const bool from_top = k <= 32;
  int r = from_top ? k : 65 - k;         // rank from the nearer end
  if (r <= 8) {
    for (;;) {
      const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(from_top ? wave_max_u32(v) : wave_min_u32(v)));
      const int c = __popcll(__ballot(v == e));
      if (c >= r) return e;
      r -= c;
      v = v == e ? (from_top ? 0u : 0xffffffffu) : v;
    }
  }
  const uint32_t key[1] = {v};
  bool ex = false;
  const uint32_t t = threshold_search<1>(key, k, 0u, hi, &ex);
  return t == 0u ? 0u
                 : (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)wave_min_u32(v >= t ? v : 0xffffffffu));
}

// Step 4 over n_s survivors held as (score bits, block) in ascending block
// order, SPL per lane (n_s <= 64 SPL): the need-th largest key T, the ties
// at T taken lowest index first, the chosen blocks written to out[f_init ..
// f_init + need) in ascending order.
template <int SPL>
__device__ __forceinline__ void select_survivors(const int2* svw, int n_s, int need,
                                                 uint32_t lo_key, uint32_t hi_key, int f_init,
                                                 int32_t* out, int lane) {
  uint32_t sk[SPL];
  int32_t sbk[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int q = lane + 64 * i;
    const int2 e = svw[q];
    sk[i] = q < n_s ? orderable_key(__int_as_float(e.x)) : 0u;   // survivors: keys > 0
    sbk[i] = e.y;
  }
  bool exact = false;
  const uint32_t T = threshold_search<SPL>(sk, need, lo_key, hi_key, &exact);
  int take = 0;
  if (!exact) {
    int gt = 0;
#pragma unroll
    for (int i = 0; i < SPL; ++i) gt += __popcll(__ballot(sk[i] > T));
    take = need - gt;
  }
  // (i, lane) order is block order
  int slot = f_init, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    bool sel;
    if (exact) {
      sel = sk[i] >= T;
    } else {
      const uint64_t eqm = __ballot(sk[i] == T);
      const int rank = eq_seen + lanes_below(eqm);
      eq_seen += __popcll(eqm);
      sel = sk[i] > T || (sk[i] == T && rank < take);
    }
    const uint64_t selm = __ballot(sel);
    if (sel) out[slot + lanes_below(selm)] = sbk[i];
    slot += __popcll(selm);
  }
}

template <int KPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KPL <= 32 ? 6 : 1)))
void select_topk_wave_kernel(TopkArgs a, int n_units) {
  // per wave: survivors (+ one dummy slot per lane, so that no lane needs a
  // branch to write); the full-search path reuses sv_b for its selection
  __shared__ int2 sv[4][kWaveSurvivors + 64];   // (score bits, block)
  static_assert(kWaveSurvivors >= kMaxTopk, "selection staging fits the survivor slots");
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int unit = blockIdx.x * 4 + wv;
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
  // Entries past n_elig but inside the row (< nb_cap) are read as they are
  // and never become candidates, so a row of at least 64 * KPL entries needs
  // no index clamp.
  const uint32_t span = (uint32_t)(f_lo - f_init);
  auto is_cand = [&](int j) { return (uint32_t)(lane + 64 * j - f_init) < span; };
  float x[KPL];
  if (a.nb_cap >= 64 * KPL) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) x[j] = S[lane + 64 * j];
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int b = lane + 64 * j;
      x[j] = S[b < n_elig ? b : n_elig - 1];
    }
  }
  // the out slots: [0, f_init) init run, [f_init, lim) chosen, then the local run
  const int lim = f_init + (need > 0 ? need : 0);
  const int n_local = n_elig - f_lo;
  int2* svw = sv[wv];

  // fast path: steps 1-4 above
  bool done = need <= 0;
  if (need > 0 && need <= 64) {
    // in place: a candidate keeps its score (the full search below tests
    // is_cand itself and reads candidates only)
    // (on the vector ALU: the scalar unit carries this kernel's searches)
    const float qnan = __builtin_nanf("");
    const uint32_t c0 = (uint32_t)(lane - f_init);
#pragma unroll
    for (int j = 0; j < KPL; ++j) x[j] = c0 + 64u * j < span ? x[j] : qnan;
    float mx = x[0];
    int j0 = 1;
#pragma unroll
    for (; j0 + 1 < KPL; j0 += 2) mx = vmax3(mx, x[j0], x[j0 + 1]);
    if (j0 < KPL) mx = vmax3(mx, x[j0], x[j0]);
    // lane maximum key (NaN: no candidate -> 0) and the wave's largest
    const uint32_t mk[1] = {orderable_key(mx)};
    const uint32_t hk = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_max_u32(mk[0]));
    // the need-th largest lane maximum (0 if fewer than `need` lanes hold
    // one; empty lanes hold 0)
    const uint32_t lo_key = kth_largest_of_lanes(mk[0], need, hk);
    if (lo_key > orderable_key(-INFINITY)) {
      // lo as a float, by the inverse of the key map: y >= lo  <=>
      // key(y) >= lo_key for every non-NaN y (lo_key is a lane maximum's key,
      // at most key(+inf))
      const float lo = __uint_as_float((lo_key & 0x80000000u) ? (lo_key & 0x7fffffffu) : ~lo_key);
      // n_s only grows: once a piece does not fit, no later one does, and
      // n_s > kWaveSurvivors afterwards sends the row to the full search.
      // Lanes that keep nothing write a dummy slot (no branch per piece).
      int n_s = 0;                 // wave-uniform
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const bool keep = x[j] >= lo;
        const uint64_t m = __ballot(keep);
        const int c = __popcll(m);
        const bool ok = keep && n_s + c <= kWaveSurvivors;
        svw[ok ? n_s + lanes_below(m) : kWaveSurvivors + lane] =
            make_int2(__float_as_int(x[j]), lane + 64 * j);
        n_s += c;
      }
      if (n_s <= kWaveSurvivors) {
        __builtin_amdgcn_wave_barrier();
        if (n_s <= 256)
          select_survivors<4>(svw, n_s, need, lo_key, hk, f_init, out, lane);
        else
          select_survivors<kWaveSurvivors / 64>(svw, n_s, need, lo_key, hk, f_init, out, lane);
        done = true;
      }
    }
  }
  if (!done) {
    // every key: the bitwise search over all of them
    uint32_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const uint32_t k = orderable_key(x[j]);
      key[j] = is_cand(j) ? (k > 1u ? k : 1u) : 0u;
    }
    uint32_t hi = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) hi = key[j] > hi ? key[j] : hi;
    hi = wave_max_u32(hi);
    bool exact = false;
    const uint32_t T = threshold_search<KPL>(key, need, 0u, hi, &exact);
    int take = 0;
    if (!exact) {
      int gt = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) gt += __popcll(__ballot(key[j] > T));
      take = need - gt;
    }
    // chosen candidates go to slots f_init, f_init + 1, ... in ascending
    // order, staged in LDS
    int base = f_init, eq_seen = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      bool sel;
      if (exact) {
        sel = key[j] >= T;
      } else {
        const uint64_t eqm = __ballot(key[j] == T);
        const int rank = eq_seen + lanes_below(eqm);
        eq_seen += __popcll(eqm);
        sel = key[j] > T || (key[j] == T && rank < take);
      }
      const uint64_t selm = __ballot(sel);
      const int slot = base + lanes_below(selm);
      const int ok = (int)sel & (int)(slot < lim);           // no short-circuit branch
      svw[ok ? slot : kWaveSurvivors + lane].y = lane + 64 * j;
      base += __popcll(selm);
    }
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < a.topk; i += 64)
      if (i >= f_init && i < lim) out[i] = svw[i].y;
  }
  // the forced runs and the padding
  for (int i = lane; i < a.topk; i += 64) {
    if (i < f_init) out[i] = i;
    else if (i >= lim) out[i] = i < lim + n_local ? f_lo + (i - lim) : -1;
  }
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
  // rows of up to 64 * KPL eligible blocks: a wave per row, the keys in
  // registers (for a handful of decode rows too: one wave per row finishes
  // sooner than a workgroup per row with barriers)
  if (nb_cap <= 64 * 16)
    hipLaunchKernelGGL(select_topk_wave_kernel<16>, dim3((unsigned)((n_units + 3) / 4)),
                       dim3(256), 0, st, a, n_units);
  else if (nb_cap <= 64 * 32)
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
