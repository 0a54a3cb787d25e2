// Device-side helpers shared by the gfx950 kernels: bfloat16 conversion,
// vector types for the MFMA builtins, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infllmv2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no key seen yet" in online softmax: exp2 of
// (kNoMax - kNoMax) is 1 and exp2(-inf - kNoMax) is 0, so no NaN appears.
constexpr float kNoMax = -1.0e30f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

// float -> bfloat16 bits, round to nearest, ties to even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return float_to_bf16_bits(lo) | (float_to_bf16_bits(hi) << 16);
}

// Element loaders: T is float or uint16_t (bfloat16 bits).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static __forceinline__ void unpack(const u32x4& w, float* o) {
    o[0] = __uint_as_float(w.x); o[1] = __uint_as_float(w.y);
    o[2] = __uint_as_float(w.z); o[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;
  __device__ static __forceinline__ void unpack(const u32x4& w, float* o) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(a[i] << 16);
      o[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ float load(const uint16_t* p) {
    return bf16_bits_to_float(*p);
  }
  __device__ static __forceinline__ void store(uint16_t* p, float v) {
    *p = (uint16_t)float_to_bf16_bits(v);
  }
};

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Wave64 butterfly reductions (all lanes receive the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Exchange a value with the lane 32 positions away (the other half-wave).
// v_permlane32_swap (VALU, no LDS round trip): with both operands = v it
// returns r[0] = v of lane (l mod 32) and r[1] = v of lane (l mod 32) + 32,
// so the partner's value is r[1] in the lower half-wave and r[0] in the upper.
__device__ __forceinline__ float swap_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving float -> uint32 key (larger float -> larger key).  -0 is
// folded onto +0 and NaN onto the smallest key, so neither wins a selection.
__device__ __forceinline__ uint32_t orderable_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Map blockIdx.x so that each XCD (workgroups are dealt round-robin over the
// 8 XCDs) receives a contiguous range of work items: neighbouring items
// share K/V blocks and then hit in the same XCD's L2.
__device__ __forceinline__ int xcd_contiguous_index(int bid, int nblocks) {
  const int kXcd = 8;
  const int per = nblocks / kXcd, rem = nblocks % kXcd;
  const int xcd = bid % kXcd, slot = bid / kXcd;
  // XCDs < rem own per+1 items, the others own per.
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + slot;
}

}  // namespace infllmv2
