// Input checks of the debug build (-DINFLLMV2_DEBUG): before its attention
// kernels, every attention call runs the kept-block rows (and tree masks) it
// is about to consume through debug_checks.h, one thread per row, and the
// first violation is kept in a device word that infllmv2_debug_check reads
// and clears.  Without INFLLMV2_DEBUG nothing here is launched and
// infllmv2_debug_check reports that the checks are not compiled in.
#include "attn_common.h"
#include "debug_checks.h"

namespace infllmv2 {

__device__ int g_dbg_code;     // first violation's code (0: none)
__device__ int g_dbg_where;    // its row * h_kv + KV head, or the draft index

__device__ __forceinline__ void dbg_record(int code, int where) {
  if (code != kDbgOk && atomicCAS(&g_dbg_code, 0, code) == 0)
    atomicExch(&g_dbg_where, where);
}

constexpr int kDbgThreads = 256;

// mode 0 (prefill chunk): row r sits at n_k - n_q + r of an n_k-key sequence;
// mode 1 (decode): row r is sequence r at seqlens[r] - 1 (n_k = max_seqlen);
// mode 2 (tree): every row at n_k - 1 of the context.
__global__ __launch_bounds__(kDbgThreads) void debug_rows_kernel(
    const int32_t* block_idx, int rows, int h_kv, int topk, int B, int init, int local,
    int dense_len, int64_t n_k, int n_q, const int32_t* seqlens, int mode) {
  const int64_t u = (int64_t)blockIdx.x * kDbgThreads + threadIdx.x;
  if (u >= (int64_t)rows * h_kv) return;
  const int r = (int)(u / h_kv);
  int64_t L = n_k, pos = n_k - 1;
  if (mode == 0) pos = n_k - n_q + r;
  if (mode == 1) {
    L = seqlens[r];
    if (L < 1 || L > n_k) return;      // the decode kernel clamps such lengths
    pos = L - 1;
  }
  if (L < dense_len) return;           // dense: the row is not read
  dbg_record(check_block_row(block_idx + u * topk, topk, (int)(pos / B) + 1, init, local),
             (int)u);
}

__global__ __launch_bounds__(64) void debug_masks_kernel(const uint64_t* mask, int n_draft) {
  const int i = threadIdx.x;
  if (i < n_draft) dbg_record(check_tree_mask(mask[i], i, n_draft), i);
}

int debug_check_rows(const int32_t* block_idx, int rows, int h_kv, const Resolved& r,
                     int64_t n_k, int n_q, const int32_t* seqlens, int mode, hipStream_t st) {
  if (!block_idx || rows <= 0) return INFLLMV2_OK;
  const int64_t units = (int64_t)rows * h_kv;
  hipLaunchKernelGGL(debug_rows_kernel, dim3((unsigned)((units + kDbgThreads - 1) / kDbgThreads)),
                     dim3(kDbgThreads), 0, st, block_idx, rows, h_kv, r.topk, r.B, r.init, r.local,
                     r.dense_len, n_k, n_q, seqlens, mode);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

int debug_check_masks(const uint64_t* mask, int n_draft, hipStream_t st) {
  if (!mask || n_draft <= 0 || n_draft > 64) return INFLLMV2_OK;
  hipLaunchKernelGGL(debug_masks_kernel, dim3(1), dim3(64), 0, st, mask, n_draft);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

}  // namespace infllmv2

using namespace infllmv2;

extern "C" int infllmv2_debug_check(int* code, int* where, void* stream) {
#ifdef INFLLMV2_DEBUG
  if (!code || !where) return INFLLMV2_ERR_INVALID_ARG;
  const int zero = 0;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
      hipMemcpyFromSymbol(code, HIP_SYMBOL(g_dbg_code), sizeof(int)) != hipSuccess ||
      hipMemcpyFromSymbol(where, HIP_SYMBOL(g_dbg_where), sizeof(int)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_dbg_code), &zero, sizeof(int)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_dbg_where), &zero, sizeof(int)) != hipSuccess)
    return INFLLMV2_ERR_HIP;
  return INFLLMV2_OK;
#else
  (void)code;
  (void)where;
  (void)stream;
  return INFLLMV2_ERR_UNSUPPORTED;
#endif
}
