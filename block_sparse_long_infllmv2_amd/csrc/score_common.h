// Block-score definitions shared by the scoring kernels: arguments and the
// window <-> block overlap arithmetic.
// Source: "MiniCPM4: running LLMs on phones and PCs" (xugj520.cn), section 1.1
// InfLLM v2 (queries are scored against 32-token semantic kernels of stride
// 16, and blocks are chosen from those scores).
#pragma once

#include "device_common.h"

namespace infllmv2 {

constexpr int kScoreThreads = 256;
constexpr int kScoreMaxWindows = 1024;   // window scores held in LDS per chunk
constexpr int kMfmaMinRows = 64;         // fewer rows: the streaming kernel
// streaming kernel: workgroups aimed for, but at least kScoreMinBlocks blocks
// each.  Ragged batch of 8 up to 128K (flushed steps): 46.6 / 45.0 / 44.5 us at
// 512 / 1024 / 2048; 128K batch 1, batch 32 and the 16-draft tree unchanged.
constexpr int kScoreMinWgs = 2048;
constexpr int kScoreMinBlocks = 4;

struct ScoreArgs {
  const void* q;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const void* ck;
  const int32_t* seqlens;
  float* scores;
  int64_t nc_cap, nb_cap;
  int h_q, h_kv, B, ks, s, dense_len, blocks_per_wg, chunks_per_row, batch, max_pos, rows;
  bool vec_store;             // rows of `scores` are 16-byte aligned
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

// Blocks per workgroup of the streaming scorer: as many as keep a chunk's
// windows within the LDS buffer (a chunk of n blocks spans at most
// (n*B + ks - 2)/s + 2 windows), at most 64, and for few rows as few as
// still give about kScoreMinWgs workgroups (a decode row alone would
// otherwise leave most CUs without loads to issue), but at least
// kScoreMinBlocks.  0 if not even one block fits.
inline int stream_blocks_per_wg(int B, int ks, int s, int64_t nb_launch, int64_t rows,
                                int h_kv) {
  int bpw = (int)(((int64_t)(kScoreMaxWindows - 2) * s - ks + 2) / B);
  if (bpw > 64) bpw = 64;
  if (bpw < 1) return 0;
  const int64_t spread = (nb_launch * rows * h_kv + kScoreMinWgs - 1) / kScoreMinWgs;
  const int64_t want = spread < kScoreMinBlocks ? kScoreMinBlocks : spread;
  if (want < bpw) bpw = (int)want;
  return bpw;
}

}  // namespace infllmv2
