// Which 16-byte-chunk swizzle lets one LDS tile serve both read patterns of
// the backward dK/dV kernel without bank conflicts?
//
// That kernel stages tiles of 32 (row, head) pairs x D = 128 bf16 (256-byte
// rows of 16 chunks of 16 bytes) and reads each tile twice:
//   A  as rows, 16-byte reads (ds_read_b128): lane (jj = lane % 16,
//      hh = lane / 16) reads row jj (+16), logical chunk 4 ks + hh;
//   B  transposed, 8-byte transposing reads (ds_read_b64_tr_b16): lane reads
//      row 4 hh + jj / 4 (+16), logical chunk 2 dt + (jj % 4) / 2, half jj % 2.
// Logical chunk c of row r is stored at chunk c ^ f(r).  This program times,
// for every f that is an invertible XOR-linear map of the row's low four
// bits (20160 maps), a loop of each pattern run by the 16 waves of one
// workgroup per CU (its LDS request leaves no room for a second), so that
// the LDS, not the latency of one wave's reads, sets the time; wave 0 reads
// the shader clock between barriers.  Conflict-free patterns run at the
// LDS's rate; conflicts add cycles.  It
// prints the cycles of the swizzles in use (K: f(r) = r, V: bits rotated)
// and of the best maps for A + B.
//
// Build: hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang
// -packed-fp32-ops -o lds_swizzle_search lds_swizzle_search.hip
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kRows = 64;                  // two 32-row tiles (alternated by iteration)
constexpr int kRowBytes = 256;
constexpr int kLdsBytes = 96 * 1024;       // one workgroup per CU

constexpr int kWaves = 16;

__global__ __launch_bounds__(kWaves * 64) void swizzle_kernel(const uint8_t* cands, int n_cand,
                                                              int iters, unsigned long long* out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int c = blockIdx.x;
  if (c >= n_cand) return;
  const int tid = threadIdx.x, lane = tid & 63, jj = lane & 15, hh = lane >> 4;
  for (int i = tid; i < kRows * kRowBytes / 4; i += kWaves * 64)
    reinterpret_cast<uint32_t*>(lds)[i] = (uint32_t)i * 2654435761u;
  const uint8_t* f = cands + c * 16;
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  const uint32_t rd = (uint32_t)(jj * kRowBytes + ((hh ^ f[jj]) * 16));
  const int tr_row = 4 * hh + (jj >> 2), tq = jj & 3;
  const uint32_t tr = (uint32_t)(tr_row * kRowBytes + (((tq >> 1) ^ f[tr_row]) * 16) + 8 * (tq & 1));
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x2 acc2 = {0u, 0u};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const uint32_t tile = base + (uint32_t)((it & 1) * 32 * kRowBytes);
    u32x4 v[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const uint32_t a = tile + ((rd ^ (uint32_t)(64 * ks)) + (uint32_t)(16 * pt * kRowBytes));
        const bf16x8 x = *reinterpret_cast<const lds_bf16x8*>((uintptr_t)a);
        v[2 * ks + pt] = *reinterpret_cast<const u32x4*>(&x);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i];
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const uint32_t tile = base + (uint32_t)((it & 1) * 32 * kRowBytes);
    u32x2 v[16];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint32_t lo = tile + (tr ^ (uint32_t)(32 * dt));
      const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)lo);
      const bf16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(uintptr_t)(lo + 16 * kRowBytes));
      v[2 * dt] = *reinterpret_cast<const u32x2*>(&x);
      v[2 * dt + 1] = *reinterpret_cast<const u32x2*>(&y);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc2 ^= v[i];
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __syncthreads();
  const unsigned long long t2 = __builtin_amdgcn_s_memtime();
  if (tid == 0) {
    out[3 * c] = t1 - t0;
    out[3 * c + 1] = t2 - t1;
  }
  // keep the reads alive
  const uint32_t keep = acc.x ^ acc.y ^ acc.z ^ acc.w ^ acc2.x ^ acc2.y;
  if (keep == 0x9e3779b9u) out[3 * c + 2] = keep;
}

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

int main() {
  // every invertible XOR-linear map of 4 bits: columns c0..c3 independent
  std::vector<uint8_t> cands;
  std::vector<unsigned> cols;
  for (unsigned m = 0; m < 65536; ++m) {
    const unsigned c0 = m & 15, c1 = (m >> 4) & 15, c2 = (m >> 8) & 15, c3 = (m >> 12) & 15;
    bool seen[16] = {};
    bool ok = true;
    uint8_t f[16];
    for (int r = 0; r < 16 && ok; ++r) {
      const unsigned v = ((r & 1) ? c0 : 0) ^ ((r & 2) ? c1 : 0) ^ ((r & 4) ? c2 : 0) ^
                         ((r & 8) ? c3 : 0);
      ok = !seen[v];
      seen[v] = true;
      f[r] = (uint8_t)v;
    }
    if (!ok) continue;
    cands.insert(cands.end(), f, f + 16);
    cols.push_back(m);
  }
  const int n = (int)(cands.size() / 16);
  uint8_t* d_c = nullptr;
  unsigned long long* d_o = nullptr;
  CHECK(hipMalloc(&d_c, cands.size()));
  CHECK(hipMalloc(&d_o, (size_t)n * 3 * sizeof(unsigned long long)));
  CHECK(hipMemcpy(d_c, cands.data(), cands.size(), hipMemcpyHostToDevice));
  CHECK(hipFuncSetAttribute((const void*)swizzle_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
  const int iters = 32;
  for (int rep = 0; rep < 2; ++rep) {          // the first launch warms the clocks
    hipLaunchKernelGGL(swizzle_kernel, dim3(n), dim3(kWaves * 64), kLdsBytes, 0, d_c, n, iters,
                       d_o);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  std::vector<unsigned long long> o((size_t)n * 3);
  CHECK(hipMemcpy(o.data(), d_o, o.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  auto find = [&](const uint8_t* f) {
    for (int i = 0; i < n; ++i)
      if (std::equal(f, f + 16, &cands[16 * i])) return i;
    return -1;
  };
  uint8_t fk[16], fv[16];
  for (int r = 0; r < 16; ++r) {
    fk[r] = (uint8_t)r;
    fv[r] = (uint8_t)(2 * (r & 7) + ((r >> 3) & 1));
  }
  unsigned long long minA = ~0ull, minB = ~0ull;
  for (int i = 0; i < n; ++i) {
    minA = std::min(minA, o[3 * i]);
    minB = std::min(minB, o[3 * i + 1]);
  }
  printf("{\"maps\": %d, \"iters\": %d, \"min_cycles_A\": %llu, \"min_cycles_B\": %llu}\n", n,
         iters, minA, minB);
  for (const auto& kv : {std::make_pair("K_swizzle_r", fk), std::make_pair("V_swizzle_rot", fv)}) {
    const int i = find(kv.second);
    printf("{\"swizzle\": \"%s\", \"cycles_A\": %llu, \"cycles_B\": %llu}\n", kv.first, o[3 * i],
           o[3 * i + 1]);
  }
  std::vector<int> idx(n);
  for (int i = 0; i < n; ++i) idx[i] = i;
  std::sort(idx.begin(), idx.end(), [&](int x, int y) {
    return o[3 * x] + o[3 * x + 1] < o[3 * y] + o[3 * y + 1];
  });
  int both = 0;
  for (int i = 0; i < n; ++i)
    both += (o[3 * i] <= minA * 105 / 100 && o[3 * i + 1] <= minB * 105 / 100);
  printf("{\"maps_within_5pct_of_both_minima\": %d}\n", both);
  for (int k = 0; k < 8 && k < n; ++k) {
    const int i = idx[k];
    printf("{\"rank\": %d, \"cycles_A\": %llu, \"cycles_B\": %llu, \"f\": [", k, o[3 * i],
           o[3 * i + 1]);
    for (int r = 0; r < 16; ++r) printf("%d%s", cands[16 * i + r], r < 15 ? ", " : "]}\n");
  }
  CHECK(hipFree(d_c));
  CHECK(hipFree(d_o));
  return 0;
}
