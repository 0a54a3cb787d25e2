// Host-side argument checks and parameter resolution shared by the entry
// points.  Nothing here touches the GPU.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/infllmv2.h"

namespace infllmv2 {

// Parameters after defaults are applied (scale resolved for head_dim d).
struct Resolved {
  int B, ks, s, topk, init, local, dense_len, score_mode;
  float scale;
};

inline int check_params(const infllmv2_params* p, int d, Resolved* r) {
  if (!p) return INFLLMV2_ERR_INVALID_ARG;
  if (p->block_size <= 0 || p->kernel_size <= 0 || p->kernel_stride <= 0 ||
      p->topk <= 0 || p->init_blocks < 0 || p->local_blocks < 0 ||
      p->dense_len < 0 || !(p->scale >= 0.0f) || isinf(p->scale))
    return INFLLMV2_ERR_INVALID_ARG;
  if (p->init_blocks + p->local_blocks > p->topk) return INFLLMV2_ERR_INVALID_ARG;
  if (p->kernel_stride > p->kernel_size) return INFLLMV2_ERR_UNSUPPORTED;
  if (p->block_size % 32 != 0 || p->block_size > 256) return INFLLMV2_ERR_UNSUPPORTED;
  if (p->topk > 128) return INFLLMV2_ERR_UNSUPPORTED;
  if (p->score_mode != 0 && p->score_mode != 1) return INFLLMV2_ERR_INVALID_ARG;
  r->B = p->block_size;
  r->ks = p->kernel_size;
  r->s = p->kernel_stride;
  r->topk = p->topk;
  r->init = p->init_blocks;
  r->local = p->local_blocks;
  r->dense_len = p->dense_len;
  r->score_mode = p->score_mode;
  r->scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)d);
  return INFLLMV2_OK;
}

inline bool dtype_ok(int dtype) { return dtype == INFLLMV2_F32 || dtype == INFLLMV2_BF16; }
inline bool head_dim_ok(int d) { return d == 64 || d == 128; }
inline size_t dtype_bytes(int dtype) { return dtype == INFLLMV2_F32 ? 4 : 2; }

inline int check_heads(int h_q, int h_kv) {
  if (h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0) return INFLLMV2_ERR_INVALID_ARG;
  return INFLLMV2_OK;
}

inline bool group_ok_for_mfma(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of full kernel windows inside n tokens.
inline int64_t num_windows(int64_t n, int ks, int s) {
  return n < ks ? 0 : (n - ks) / s + 1;
}

}  // namespace infllmv2

#define INFLLMV2_TRY(expr)            \
  do {                                \
    int _st = (expr);                 \
    if (_st != INFLLMV2_OK) return _st; \
  } while (0)
