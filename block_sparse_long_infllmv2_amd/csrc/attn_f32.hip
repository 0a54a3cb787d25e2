// Block-sparse causal attention for float32 inputs on the vector ALUs.
// Same definition as the bf16 matrix-core path (see attn_bf16.hip): keys of
// the kept blocks up to the query position (dense below dense_len), plus the
// ancestor drafts for tree verification.
//
// One wave per (query row, head).  Each 64-key sub-chunk is scored one key
// per lane (the query row sits in LDS), merged into an online softmax with
// wave reductions, and accumulated into the output with one output dimension
// per lane.  This path favours exactness over speed: it exists for float32
// callers and small problems.
#include "attn_common.h"

namespace infllmv2 {

template <int D, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[D];
  __shared__ float ps[64];
  const float* q = reinterpret_cast<const float*>(a.q);
  const float* kc = reinterpret_cast<const float*>(a.k);
  const float* vc = reinterpret_cast<const float*>(a.v);
  const int lane = threadIdx.x;
  const int row = blockIdx.x / a.h_q, head = blockIdx.x % a.h_q;
  const int G = a.h_q / a.h_kv;
  const int g = head / G;

  int64_t n_keys, pos;
  int seq = 0;
  if constexpr (MODE == kPrefill) {
    n_keys = a.n_k;
    pos = a.n_k - a.n_rows + row;
  } else if constexpr (MODE == kDecode) {
    seq = row;
    const int64_t L = a.seqlens[seq];
    n_keys = L < 1 ? 1 : (L > a.n_k ? a.n_k : L);
    pos = n_keys - 1;
  } else {
    n_keys = a.n_k;
    pos = a.n_k - 1;
  }
  const bool dense = n_keys < a.dense_len || a.block_idx == nullptr;
  const int64_t n_b = (n_keys + a.B - 1) / a.B;
  const int64_t b_own = pos / a.B;

  for (int d = lane; d < D; d += 64)
    qs[d] = q[((int64_t)row * a.h_q + head) * D + d] * a.scale_log2;
  __syncthreads();

  const int64_t head_off = (MODE == kDecode ? ((int64_t)seq * a.h_kv + g) : (int64_t)g) * a.cap;
  const float* kh = kc + head_off * D;
  const float* vh = vc + head_off * D;
  const int32_t* lst = dense ? nullptr : a.block_idx + ((int64_t)row * a.h_kv + g) * a.topk;

  float m = kNoMax, l = 0.0f;
  float acc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.0f;

  // keys [k0, k1) of `kp`/`vp`, optionally filtered by a draft bitmask
  auto consume = [&](const float* kp, const float* vp, int64_t k0, int64_t k1, bool use_bits,
                     uint64_t bits) {
    for (int64_t c0 = k0; c0 < k1; c0 += 64) {
      const int64_t key = c0 + lane;
      bool ok = key < k1;
      if (use_bits) ok = ok && ((bits >> key) & 1ull);
      float s = -INFINITY;
      if (ok) {
        float dot = 0.0f;
        const float* kr = kp + key * D;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
        s = dot;
      }
      const float mx = wave_max(s);
      const float m_new = fmaxf(m, mx);
      const float alpha = exp2f(m - m_new);
      const float p = ok ? exp2f(s - m_new) : 0.0f;
      l = l * alpha + wave_sum(p);
      m = m_new;
      ps[lane] = p;
      __syncthreads();
      const int nk = (int)min((int64_t)64, k1 - c0);
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        float x = acc[i] * alpha;
        for (int j = 0; j < nk; ++j) x = fmaf(ps[j], vp[(c0 + j) * D + lane + 64 * i], x);
        acc[i] = x;
      }
      __syncthreads();
    }
  };

  const int64_t n_ent = dense ? b_own + 1 : a.topk;
  for (int64_t e = 0; e < n_ent; ++e) {
    int64_t b;
    if (dense) {
      b = e;
    } else {
      b = lst[e];
      if (b < 0 || b >= n_b || b > b_own) continue;
    }
    const int64_t k0 = b * a.B;
    int64_t k1 = (b + 1) * a.B;
    if (k1 > pos + 1) k1 = pos + 1;
    consume(kh, vh, k0, k1, false, 0);
  }
  if constexpr (MODE == kTree) {
    const uint64_t full = a.n_rows >= 64 ? ~0ull : ((1ull << a.n_rows) - 1ull);
    const uint64_t bits = (a.tree_mask[row] & full) | (1ull << row);
    const float* kd = reinterpret_cast<const float*>(a.k_draft) + (int64_t)g * a.n_rows * D;
    const float* vd = reinterpret_cast<const float*>(a.v_draft) + (int64_t)g * a.n_rows * D;
    consume(kd, vd, 0, a.n_rows, true, bits);
  }

  float* out = reinterpret_cast<float*>(a.out) + ((int64_t)row * a.h_q + head) * D;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) out[lane + 64 * i] = acc[i] * inv;
  if (a.lse && lane == 0) a.lse[(int64_t)row * a.h_q + head] = (m + log2f(l)) * kLn2;
}

template <int MODE>
static int launch_f32(const AttnArgs& a, int d, hipStream_t st) {
  const int64_t n = (int64_t)a.n_rows * a.h_q;
  if (n >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
  if (d == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128, MODE>), dim3((unsigned)n), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64, MODE>), dim3((unsigned)n), dim3(64), 0, st, a);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

int prefill_f32(const AttnArgs& a, int d, hipStream_t st) { return launch_f32<kPrefill>(a, d, st); }
int decode_f32(const AttnArgs& a, int d, hipStream_t st) { return launch_f32<kDecode>(a, d, st); }
int tree_f32(const AttnArgs& a, int d, hipStream_t st) { return launch_f32<kTree>(a, d, st); }

}  // namespace infllmv2
