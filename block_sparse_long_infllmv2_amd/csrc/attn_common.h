// Arguments shared by the attention kernels (bf16 matrix-core path and the
// float32 vector path) and the host launchers.
#pragma once

#include "device_common.h"
#include "host_common.h"

namespace infllmv2 {

enum Mode { kPrefill = 0, kDecode = 1, kTree = 2 };

constexpr int kChunk = 64;                  // keys per staged unit
constexpr int kSortCap = 128;               // max topk handled by the union sort
constexpr int kEmptyBlock = 0x7fffffff;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_idx;   // [rows][h_kv][topk] or NULL (dense)
  const uint16_t* k_draft;    // tree: [h_kv][n_draft][D]
  const uint16_t* v_draft;
  const uint64_t* tree_mask;  // tree: [n_draft]
  const int32_t* seqlens;     // decode: [batch]
  const int32_t* union_blk;   // tree: [h_kv][union_cap] (from the planner)
  const uint64_t* union_mask; // tree: [h_kv][union_cap], bit = draft index
  const int32_t* union_len;   // tree: [h_kv]
  uint16_t* out;
  float* lse;
  float* ws;                  // split partials [rows][h_q][n_split][D+2]
  int64_t cap;                // tokens per (sequence, KV head) in the cache
  int64_t n_k;                // prefill: keys; tree: context length
  int n_rows;                 // prefill: n_q; decode: batch; tree: n_draft
  int h_q, h_kv, topk, B, dense_len, n_split, n_tiles, union_cap;
  int ring_min;               // prefill, 16-head groups: blocks kept by at least this
                              // many of a tile's tokens go through the shared ring,
                              // the others through each token's own pass (0: all ring)
  float scale_log2;           // softmax scale * log2(e)
  // decode / tree, 16-head groups, selection inside the attention kernel:
  const float* scores;        // [rows][h_kv][nb_cap] block scores
  int32_t* sel_out;           // [rows][h_kv][topk]: the selection, written by split 0
  int64_t nb_cap;
  int init, local;            // forced initial / local blocks
};


// Debug builds (-DINFLLMV2_DEBUG): checks of the kept-block rows / tree masks
// a call consumes (mode 0 prefill, 1 decode, 2 tree), queued before its
// attention kernels.
int debug_check_rows(const int32_t* block_idx, int rows, int h_kv, const Resolved& r,
                     int64_t n_k, int n_q, const int32_t* seqlens, int mode, hipStream_t st);
int debug_check_masks(const uint64_t* mask, int n_draft, hipStream_t st);

// float32 (vector ALU) attention: exact-precision path for float32 inputs.
int prefill_f32(const AttnArgs& a, int d, hipStream_t st);
int decode_f32(const AttnArgs& a, int d, hipStream_t st);
int tree_f32(const AttnArgs& a, int d, hipStream_t st);

}  // namespace infllmv2
