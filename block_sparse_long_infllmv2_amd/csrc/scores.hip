// Block relevance scores: each query row's GQA group scores the semantic
// kernels it can see, and the kernel scores are max-pooled onto the blocks
// they overlap.
// Source: "MiniCPM4: running LLMs on phones and PCs" (xugj520.cn), section 1.1
// InfLLM v2 (queries are scored against semantic kernels and blocks are chosen
// from those scores, avoiding token-level work).
//
//   sigma[m] = scale * (sum_{h in g} q_h) . ck[g][m],  window m visible iff
//              m*s + ks - 1 <= pos
//   S[b]     = max over visible windows m overlapping block b (-inf if none)
//
// Streaming kernel (one workgroup per (row, KV head, chunk of blocks)): the
// group-summed query sits in LDS, d/E threads dot one compressed-key row,
// the window scores of the chunk go to LDS and one thread per block pools
// them.  It is HBM-bound for decode-sized row counts.
#include "device_common.h"
#include "host_common.h"

namespace infllmv2 {

constexpr int kScoreThreads = 256;
constexpr int kScoreMaxWindows = 1024;   // window scores held in LDS per chunk

struct ScoreArgs {
  const void* q;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const void* ck;
  const int32_t* seqlens;
  float* scores;
  int64_t nc_cap, nb_cap;
  int h_q, h_kv, B, ks, s, dense_len, blocks_per_wg, chunks_per_row, batch, max_pos;
  float scale;
};

// First window whose span [m*s, m*s+ks) reaches block b (i.e. m*s+ks-1 >= b*B).
__device__ __forceinline__ int64_t first_window_of_block(int64_t b, int B, int ks, int s) {
  const int64_t t = b * B - ks + 1;
  return t <= 0 ? 0 : (t + s - 1) / s;
}
// Last window starting inside block b (m*s <= (b+1)*B - 1).
__device__ __forceinline__ int64_t last_window_of_block(int64_t b, int B, int s) {
  return ((b + 1) * B - 1) / s;
}

template <typename T, int D>
__global__ __launch_bounds__(kScoreThreads) void block_scores_stream_kernel(ScoreArgs a) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int TPW = D / E;                       // threads per window row
  constexpr int WPP = kScoreThreads / TPW;         // windows per pass
  __shared__ float qs[D];
  __shared__ float sig[kScoreMaxWindows];

  const int r = blockIdx.x / a.chunks_per_row, g = blockIdx.y;
  const int chunk = blockIdx.x % a.chunks_per_row;
  const int seq = a.row_seq ? a.row_seq[r] : 0;
  if (seq < 0 || seq >= a.batch) return;           // malformed row: skipped
  const int64_t L = a.seqlens[seq];
  if (L < a.dense_len) return;                     // dense sequence: no scores
  const int64_t pos = a.row_pos ? a.row_pos[r] : L - 1;
  if (pos < 0 || pos >= L || pos > a.max_pos) return;  // outside the launch bounds
  const int64_t b_own = pos / a.B;
  const int64_t b0 = (int64_t)chunk * a.blocks_per_wg;
  if (b0 > b_own) return;
  const int64_t b1 = min(b0 + a.blocks_per_wg - 1, b_own);
  const int64_t n_vis = pos >= a.ks - 1 ? (pos - a.ks + 1) / a.s + 1 : 0;
  const int64_t m_lo = first_window_of_block(b0, a.B, a.ks, a.s);
  const int64_t m_hi = min(last_window_of_block(b1, a.B, a.s), n_vis - 1);

  // group-summed query, pre-multiplied by the softmax scale
  const int G = a.h_q / a.h_kv;
  const T* qrow = (const T*)a.q + ((int64_t)r * a.h_q + (int64_t)g * G) * D;
  for (int d = threadIdx.x; d < D; d += kScoreThreads) {
    float acc = 0.0f;
    for (int h = 0; h < G; ++h) acc += Elem<T>::load(qrow + h * D + d);
    qs[d] = acc * a.scale;
  }
  __syncthreads();

  const int sub = threadIdx.x / TPW, lane = threadIdx.x % TPW;
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = qs[lane * E + e];
  const T* ckb = (const T*)a.ck + ((int64_t)seq * a.h_kv + g) * a.nc_cap * D + lane * E;
  for (int64_t m0 = m_lo; m0 <= m_hi; m0 += WPP) {
    const int64_t m = m0 + sub;
    float part = 0.0f;
    if (m <= m_hi) {
      float x[E];
      Elem<T>::unpack(ldg16(ckb + m * D), x);
#pragma unroll
      for (int e = 0; e < E; ++e) part += qv[e] * x[e];
    }
#pragma unroll
    for (int o = TPW / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == 0 && m <= m_hi) sig[m - m_lo] = part;
  }
  __syncthreads();

  float* out = a.scores + ((int64_t)r * a.h_kv + g) * a.nb_cap;
  for (int64_t b = b0 + threadIdx.x; b <= b1; b += kScoreThreads) {
    const int64_t lo = first_window_of_block(b, a.B, a.ks, a.s);
    const int64_t hi = min(last_window_of_block(b, a.B, a.s), m_hi);
    float v = -INFINITY;
    for (int64_t m = lo; m <= hi; ++m) v = fmaxf(v, sig[m - m_lo]);
    out[b] = v;
  }
}

template <typename T, int D>
static int launch_scores(const ScoreArgs& a, int rows, hipStream_t st) {
  dim3 grid((unsigned)((int64_t)a.chunks_per_row * rows), a.h_kv, 1);
  hipLaunchKernelGGL((block_scores_stream_kernel<T, D>), grid, dim3(kScoreThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

}  // namespace infllmv2

using namespace infllmv2;

extern "C" int infllmv2_block_scores(int dtype, const void* q, int32_t rows,
                                     const int32_t* row_seq, const int32_t* row_pos,
                                     int32_t h_q, int32_t h_kv, int32_t d, const void* ck,
                                     int32_t batch, int64_t nc_cap, const int32_t* seqlens,
                                     float* scores, int64_t nb_cap, int32_t max_pos,
                                     const infllmv2_params* p, void* stream) {
  if (!dtype_ok(dtype)) return INFLLMV2_ERR_INVALID_ARG;
  if (!q || !ck || !seqlens || !scores) return INFLLMV2_ERR_INVALID_ARG;
  if (rows < 0 || batch <= 0 || nc_cap <= 0 || nb_cap <= 0 || max_pos < 0)
    return INFLLMV2_ERR_INVALID_ARG;
  INFLLMV2_TRY(check_heads(h_q, h_kv));
  if (!head_dim_ok(d)) return INFLLMV2_ERR_UNSUPPORTED;
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if ((int64_t)max_pos / r.B + 1 > nb_cap) return INFLLMV2_ERR_INVALID_ARG;
  if (num_windows((int64_t)max_pos + 1, r.ks, r.s) > nc_cap) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(ck) || !aligned16(q)) return INFLLMV2_ERR_INVALID_ARG;
  if (rows == 0) return INFLLMV2_OK;
  ScoreArgs a;
  a.q = q; a.row_seq = row_seq; a.row_pos = row_pos; a.ck = ck; a.seqlens = seqlens;
  a.scores = scores; a.nc_cap = nc_cap; a.nb_cap = nb_cap; a.h_q = h_q; a.h_kv = h_kv;
  a.B = r.B; a.ks = r.ks; a.s = r.s; a.dense_len = r.dense_len; a.scale = r.scale;
  a.batch = batch; a.max_pos = max_pos;
  // blocks per workgroup: as many as keep the chunk's windows within the LDS
  // buffer (a chunk of n blocks spans at most (n*B + ks - 2)/s + 2 windows)
  int bpw = (int)(((int64_t)(kScoreMaxWindows - 2) * r.s - r.ks + 2) / r.B);
  if (bpw > 64) bpw = 64;
  if (bpw < 1) return INFLLMV2_ERR_UNSUPPORTED;
  a.blocks_per_wg = bpw;
  const int64_t nb_launch = (int64_t)max_pos / r.B + 1;
  a.chunks_per_row = (int)ceil_div(nb_launch, bpw);
  if ((int64_t)a.chunks_per_row * rows >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == INFLLMV2_BF16)
    return d == 128 ? launch_scores<uint16_t, 128>(a, rows, st)
                    : launch_scores<uint16_t, 64>(a, rows, st);
  return d == 128 ? launch_scores<float, 128>(a, rows, st)
                  : launch_scores<float, 64>(a, rows, st);
}
