// Host-only entry points: defaults, status strings, version, workspace sizes.
#include "attn_common.h"

namespace infllmv2 {
size_t tree_workspace_bytes(int n_draft, int h_q, int h_kv, int d, int64_t n_ctx,
                            const Resolved& r);
size_t decode_workspace_bytes(int batch, int h_q, int h_kv, int d, int64_t max_seqlen,
                              const Resolved& r);
size_t prefill_bwd_workspace_bytes(int n_q, int h_q, int h_kv, int64_t n_k, const Resolved& r);
}  // namespace infllmv2

using namespace infllmv2;

extern "C" void infllmv2_default_params(infllmv2_params* p) {
  if (!p) return;
  // 64-token blocks, 32/16 semantic kernels, top-64, dense below 8192 tokens
  // (shadowrocket9.top, InfLLM v2 section and its sparse_config dict;
  // xugj520.cn, section 1.1); 1 initial block and a 2-block local window.
  p->block_size = 64;
  p->kernel_size = 32;
  p->kernel_stride = 16;
  p->topk = 64;
  p->init_blocks = 1;
  p->local_blocks = 2;
  p->dense_len = 8192;
  p->scale = 0.0f;
  p->score_mode = 0;         // summed-query reading of the group score
}

extern "C" const char* infllmv2_status_string(int status) {
  switch (status) {
    case INFLLMV2_OK: return "ok";
    case INFLLMV2_ERR_INVALID_ARG: return "invalid argument";
    case INFLLMV2_ERR_UNSUPPORTED: return "unsupported configuration";
    case INFLLMV2_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case INFLLMV2_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

extern "C" int infllmv2_version(void) { return 101; }

extern "C" size_t infllmv2_workspace_size(int op, int32_t n, int32_t h_q, int32_t h_kv,
                                          int32_t d, int64_t max_len,
                                          const infllmv2_params* p) {
  Resolved r;
  if (n < 0 || max_len <= 0 || check_heads(h_q, h_kv) != INFLLMV2_OK || !head_dim_ok(d) ||
      check_params(p, d, &r) != INFLLMV2_OK)
    return 0;
  if (op == INFLLMV2_OP_DECODE) return decode_workspace_bytes(n, h_q, h_kv, d, max_len, r);
  if (op == INFLLMV2_OP_TREE) {
    if (n > 64) return 0;
    return tree_workspace_bytes(n, h_q, h_kv, d, max_len, r);
  }
  if (op == INFLLMV2_OP_PREFILL_BWD) {
    if (max_len > INT32_MAX || n > max_len) return 0;
    return prefill_bwd_workspace_bytes(n, h_q, h_kv, max_len, r);
  }
  return 0;
}
