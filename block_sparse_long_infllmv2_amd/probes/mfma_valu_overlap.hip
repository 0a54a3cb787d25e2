// Does gfx950 run one wave's matrix-core (MFMA) work and another wave's
// vector-ALU work on the same SIMD at the same time?
//
// The sparse prefill attention alternates, per 64-key chunk and per wave, a
// matrix-core phase (QK^T and PV, 32 MFMAs of 16x16x32 bf16) with a vector
// phase of about the same issue time (online softmax: fma, exp2, add, bf16
// packing).  Whether such phases of different waves overlap sets the
// kernel's ceiling (about 50% of the bf16 peak if they never do).  This
// program measures it directly.
//
// One 8-wave workgroup per CU (its LDS request leaves no room for a second);
// waves w and w+4 share a SIMD when a workgroup's waves are dealt to the
// four SIMDs in turn.  Each wave runs either an MFMA loop (8 independent
// accumulators, no data dependence between consecutive MFMAs) or a VALU loop
// (8 independent chains of fma -> exp2 -> add, R times per iteration), and
// the kernel time is taken with HIP events (median of repeated launches):
//   all_mfma      every wave MFMA            -> 2 m per SIMD
//   all_valu      every wave VALU            -> 2 v per SIMD
//   split_simd    waves 0-3 MFMA, 4-7 VALU   -> one of each per SIMD:
//                 max(m, v) if the SIMD overlaps them, m + v if it does not
//   split_pairs   even waves MFMA, odd VALU  -> pairs of like waves per SIMD
//                 (2 m and 2 v on different SIMDs): max(2m, 2v)
//   same_wave     each wave: the MFMA loop and the VALU loop interleaved
//                 (independent), one wave's own overlap -> 2 max(m, v) .. 2 (m + v)
// It prints one JSON line per (layout, R) and a summary: the overlap share
// (m + v - t_split) / min(m, v), 1 = full overlap, 0 = none.
//
// Build: hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang
// -packed-fp32-ops -o mfma_valu_overlap mfma_valu_overlap.hip
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Layout { kAllMfma = 0, kAllValu = 1, kSplitSimd = 2, kSplitPairs = 3, kSameWave = 4 };
static const char* kNames[] = {"all_mfma", "all_valu", "split_simd", "split_pairs", "same_wave"};

constexpr int kWaves = 8;
constexpr int kLdsBytes = 96 * 1024;   // > half of a CU's 160 KB: one workgroup per CU

__device__ __forceinline__ void mfma_step(f32x4 (&c)[8], bf16x8 a, bf16x8 b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
}

template <int R>
__device__ __forceinline__ void valu_step(float (&x)[8], float s, float m) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], s, -m));
      x[j] = p + x[j] * 0.5f;
    }
}

template <int R>
__global__ __launch_bounds__(kWaves * 64) void probe_kernel(int layout, int iters, float* out) {
  extern __shared__ float lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  bool do_mfma, do_valu;
  switch (layout) {
    case kAllMfma: do_mfma = true; do_valu = false; break;
    case kAllValu: do_mfma = false; do_valu = true; break;
    case kSplitSimd: do_mfma = w < 4; do_valu = w >= 4; break;
    case kSplitPairs: do_mfma = (w & 1) == 0; do_valu = (w & 1) == 1; break;
    default: do_mfma = true; do_valu = true; break;
  }
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.01f * (float)(lane + j);
  const float s = 0.25f, m = 1.0f;
  if (do_mfma && do_valu) {
    for (int i = 0; i < iters; ++i) {
      mfma_step(c, a, b);
      valu_step<R>(x, s, m);
    }
  } else if (do_mfma) {
    for (int i = 0; i < iters; ++i) mfma_step(c, a, b);
  } else {
    for (int i = 0; i < iters; ++i) valu_step<R>(x, s, m);
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc += c[j][0] + c[j][1] + c[j][2] + c[j][3] + x[j];
  if (lane == 0) lds[w] = acc;          // keeps the LDS request (and the work) alive
  __syncthreads();
  out[blockIdx.x * kWaves * 64 + threadIdx.x] = acc + lds[(w + 1) % kWaves];
}

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

template <int R>
static int run(int layout, int iters, int n_cu, float* out, float* ms) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<float> t;
  for (int rep = 0; rep < 12; ++rep) {
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(probe_kernel<R>, dim3(n_cu), dim3(kWaves * 64), kLdsBytes, 0, layout,
                       iters, out);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float x;
    CHECK(hipEventElapsedTime(&x, e0, e1));
    if (rep >= 2) t.push_back(x);        // the first launches warm the clocks up
  }
  std::sort(t.begin(), t.end());
  *ms = t[t.size() / 2];
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return 0;
}

int main() {
  int dev = 0;
  CHECK(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, dev));
  const int n_cu = prop.multiProcessorCount;
  CHECK(hipFuncSetAttribute((const void*)probe_kernel<1>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  CHECK(hipFuncSetAttribute((const void*)probe_kernel<2>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)n_cu * kWaves * 64 * sizeof(float)));
  const int iters = 20000;
  // bf16 16x16x32 MFMA = 16384 flop
  const double mfma_flop_per_wave = 8.0 * 16384.0 * iters;
  for (int R = 1; R <= 2; ++R) {
    float t[5];
    for (int layout = 0; layout < 5; ++layout) {
      const int rc = R == 1 ? run<1>(layout, iters, n_cu, out, &t[layout])
                            : run<2>(layout, iters, n_cu, out, &t[layout]);
      if (rc) return rc;
      const int mfma_waves = layout == kAllMfma || layout == kSameWave ? 8
                             : layout == kAllValu ? 0 : 4;
      const double tflops = mfma_flop_per_wave * mfma_waves * n_cu / (t[layout] * 1e-3) / 1e12;
      printf("{\"layout\": \"%s\", \"valu_reps\": %d, \"iters\": %d, \"cus\": %d, "
             "\"ms\": %.4f, \"mfma_tflops\": %.1f}\n",
             kNames[layout], R, iters, n_cu, t[layout], tflops);
    }
    // per-SIMD work of one wave: m = all_mfma / 2, v = all_valu / 2
    const double m = t[kAllMfma] / 2, v = t[kAllValu] / 2;
    const double share = (m + v - t[kSplitSimd]) / std::min(m, v);
    const double share_pairs = (m + v - t[kSplitPairs]) / std::min(m, v);
    const double share_wave = (2 * (m + v) - t[kSameWave]) / (2 * std::min(m, v));
    printf("{\"summary\": true, \"valu_reps\": %d, \"m_ms\": %.4f, \"v_ms\": %.4f, "
           "\"overlap_split_simd\": %.3f, \"overlap_split_pairs\": %.3f, "
           "\"overlap_same_wave\": %.3f}\n",
           R, m, v, share, share_pairs, share_wave);
  }
  CHECK(hipFree(out));
  return 0;
}
