// Semantic-kernel key compression: mean of the keys of each overlapping
// window [m*s, m*s+ks) (32 tokens, stride 16 by default), per KV head.
// Source: "MiniCPM4: running LLMs on phones and PCs" (xugj520.cn), section 1.1
// InfLLM v2 (semantic kernels of 32 tokens, stride 16); the kernels add no
// parameters ("MiniCPM 4.0" blog, shadowrocket9.top, InfLLM v2 section).
//
// HBM-bound stream; overlapping windows re-read their shared rows, which hit
// in L2.
#include "device_common.h"
#include "host_common.h"

namespace infllmv2 {

constexpr int kCompressThreads = 256;
constexpr int kCompressSplit = 4;       // thread groups sharing one window's rows

// A window is summed by kCompressSplit groups of d/E threads; group q adds
// rows t = q, q + 4, ... of the window, each thread one 16-byte column chunk
// (a window row is read as one coalesced 256-byte segment for bf16, d=128).
// The partial sums meet in LDS.  The sum is rounded in float32: once the
// window's values spread over more than ~16 binary orders of magnitude a
// partial sum drops low bits, so another summation order can move the
// stored bf16 mean by one unit in the last place in rare cases.  Tests allow
// for that (at most 1 in 10^4 elements differ from a float64 mean).
template <typename T, int D>
__global__ __launch_bounds__(kCompressThreads) void compress_keys_kernel(
    const T* __restrict__ k, int h_kv, int64_t cap, const int32_t* __restrict__ seqlens,
    int64_t m_begin, int64_t m_end, T* __restrict__ ck, int64_t nc_cap, int ks, int s) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int TPW = D / E;                                  // threads per row chunk set
  constexpr int WPB = kCompressThreads / (TPW * kCompressSplit);  // windows per block
  __shared__ float part[WPB][kCompressSplit - 1][D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t L = seqlens[b];
  // windows whose tokens lie inside the sequence: m*s + ks <= L
  const int64_t n_full = L < ks ? 0 : (L - ks) / s + 1;
  const int64_t stop = m_end < n_full ? m_end : n_full;
  const int tid = threadIdx.x;
  const int lane = tid % TPW, q = (tid / TPW) % kCompressSplit, wl = tid / (TPW * kCompressSplit);
  const int64_t m = m_begin + (int64_t)blockIdx.x * WPB + wl;
  const bool live = m < stop;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  if (live) {
    const T* src = k + ((int64_t)b * h_kv + g) * cap * D + m * s * D + lane * E;
    for (int t = q; t < ks; t += kCompressSplit) {
      float x[E];
      Elem<T>::unpack(ldg16(src + (int64_t)t * D), x);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += x[e];
    }
  }
  if (q > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) part[wl][q - 1][lane * E + e] = acc[e];
  }
  __syncthreads();
  if (q != 0 || !live) return;
#pragma unroll
  for (int j = 0; j < kCompressSplit - 1; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += part[wl][j][lane * E + e];
  // Divide (rather than multiply by a rounded reciprocal): for the default
  // ks = 32 the division is exact, so the only rounding is the final one to
  // the storage type.
  const float fks = (float)ks;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = acc[e] / fks;
  u32x4 w;
  if constexpr (E == 8) {
    w.x = pack_bf16x2(acc[0], acc[1]);
    w.y = pack_bf16x2(acc[2], acc[3]);
    w.z = pack_bf16x2(acc[4], acc[5]);
    w.w = pack_bf16x2(acc[6], acc[7]);
  } else {
    w.x = __float_as_uint(acc[0]);
    w.y = __float_as_uint(acc[1]);
    w.z = __float_as_uint(acc[2]);
    w.w = __float_as_uint(acc[3]);
  }
  T* dst = ck + ((int64_t)b * h_kv + g) * nc_cap * D + m * D + lane * E;
  *reinterpret_cast<u32x4*>(dst) = w;
}

template <typename T, int D>
static int launch_compress(const void* k, int32_t batch, int32_t h_kv, int64_t cap,
                           const int32_t* seqlens, int64_t m_begin, int64_t m_end, void* ck,
                           int64_t nc_cap, const Resolved& r, hipStream_t st) {
  const int64_t n = m_end - m_begin;
  constexpr int WPB = kCompressThreads / ((D / Elem<T>::kPer16B) * kCompressSplit);
  dim3 grid((unsigned)ceil_div(n, WPB), h_kv, batch);
  hipLaunchKernelGGL((compress_keys_kernel<T, D>), grid, dim3(kCompressThreads), 0, st,
                     (const T*)k, h_kv, cap, seqlens, m_begin, m_end, (T*)ck, nc_cap, r.ks,
                     r.s);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

}  // namespace infllmv2

using namespace infllmv2;

extern "C" int infllmv2_compress_keys(int dtype, const void* k, int32_t batch, int32_t h_kv,
                                      int64_t cap, int32_t d, const int32_t* seqlens,
                                      int64_t m_begin, int64_t m_end, void* ck,
                                      int64_t nc_cap, const infllmv2_params* p,
                                      void* stream) {
  if (!dtype_ok(dtype)) return INFLLMV2_ERR_INVALID_ARG;
  if (!k || !ck || !seqlens) return INFLLMV2_ERR_INVALID_ARG;
  if (batch <= 0 || h_kv <= 0 || cap <= 0 || nc_cap <= 0) return INFLLMV2_ERR_INVALID_ARG;
  if (!head_dim_ok(d)) return INFLLMV2_ERR_UNSUPPORTED;
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if (m_begin < 0 || m_end < m_begin || m_end > nc_cap) return INFLLMV2_ERR_INVALID_ARG;
  if (m_end > m_begin && (m_end - 1) * r.s + r.ks > cap) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(ck)) return INFLLMV2_ERR_INVALID_ARG;
  if (m_end == m_begin) return INFLLMV2_OK;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == INFLLMV2_BF16)
    return d == 128 ? launch_compress<uint16_t, 128>(k, batch, h_kv, cap, seqlens, m_begin,
                                                     m_end, ck, nc_cap, r, st)
                    : launch_compress<uint16_t, 64>(k, batch, h_kv, cap, seqlens, m_begin,
                                                    m_end, ck, nc_cap, r, st);
  return d == 128 ? launch_compress<float, 128>(k, batch, h_kv, cap, seqlens, m_begin, m_end,
                                                ck, nc_cap, r, st)
                  : launch_compress<float, 64>(k, batch, h_kv, cap, seqlens, m_begin, m_end,
                                               ck, nc_cap, r, st);
}
