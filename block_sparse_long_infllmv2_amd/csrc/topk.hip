// Top-k block selection with forced initial and local blocks.
// Sources: "MiniCPM 4.0" blog (shadowrocket9.top), InfLLM v2 section (each
// query keeps its top-k most relevant blocks, k = 64); "MiniCPM4: running
// LLMs on phones and PCs" (xugj520.cn), section 1.1 (initial tokens and a
// sliding window are always kept).
//
// Rows of up to 4096 eligible blocks take one wave per (row, KV head)
// (select_topk_wave_kernel, below, with the per-row selection of
// topk_wave.h).  Longer rows: one workgroup per (row, KV head).  Scores become order-preserving uint32
// keys (staged in LDS when they fit); an MSB-first radix select (four 8-bit
// digits, LDS histogram, suffix scan to pick the digit) finds the threshold
// key T of the need-th best non-forced block.  Blocks with key > T are kept,
// and of the blocks with key == T the lowest-indexed ones fill the rest, which
// gives exactly the (score descending, index ascending) order.  An ordered
// scan then writes the kept block ids in ascending order.
#include "host_common.h"
#include "topk_wave.h"

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
  const int seq = a.row_seq ? a.row_seq[r] : (a.row_is_seq ? r : 0);
  bool skip = seq < 0 || seq >= a.batch;
  int64_t L = skip ? 0 : (a.seqlens ? a.seqlens[seq] : a.fixed_len);
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

template <int KPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KPL <= 32 ? 6 : 1)))
void select_topk_wave_kernel(TopkArgs a, int n_units) {
  // per wave: survivors (+ one dummy slot per lane, so that no lane needs a
  // branch to write); the full-search path reuses them for its selection
  __shared__ int2 sv[4][kWaveSurvivors + 64];   // (score bits, block)
  static_assert(kWaveSurvivors >= kMaxTopk, "selection staging fits the survivor slots");
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int unit = blockIdx.x * 4 + wv;
  if (unit >= n_units) return;                   // whole wave leaves
  const int lane = threadIdx.x & 63;
  const int r = unit / a.h_kv, g = unit % a.h_kv;
  int32_t* out = a.block_idx + ((int64_t)r * a.h_kv + g) * a.topk;
  const int seq = a.row_seq ? a.row_seq[r] : (a.row_is_seq ? r : 0);
  bool skip = seq < 0 || seq >= a.batch;
  const int64_t L = skip ? 0 : (a.seqlens ? a.seqlens[seq] : a.fixed_len);
  const int64_t pos = a.row_pos ? a.row_pos[r] : L - 1;
  skip = skip || L < a.dense_len || pos < 0 || pos >= L || pos / a.B + 1 > a.nb_cap;
  if (skip) {
    for (int i = lane; i < a.topk; i += 64) out[i] = -1;
    return;
  }
  wave_select_row<KPL>(a.scores + ((int64_t)r * a.h_kv + g) * a.nb_cap, a.nb_cap,
                       (int)(pos / a.B), a.topk, a.init, a.local, sv[wv], out, lane);
}

int launch_select_topk(const TopkArgs& a, int rows, hipStream_t st) {
  const int n_units = rows * a.h_kv;
  const int64_t nb_cap = a.nb_cap;
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
  TopkArgs a = {};
  a.scores = scores; a.row_seq = row_seq; a.row_pos = row_pos; a.seqlens = seqlens;
  a.block_idx = block_idx; a.nb_cap = nb_cap; a.h_kv = h_kv; a.B = r.B; a.topk = r.topk;
  a.init = r.init; a.local = r.local; a.dense_len = r.dense_len; a.batch = batch;
  return launch_select_topk(a, rows, (hipStream_t)stream);
}
