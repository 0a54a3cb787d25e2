// Checks of the kept-block lists and tree masks the attention calls consume,
// as plain functions that compile for the host (plain C++) and for the GPU
// (HIP).  Libraries built with -DINFLLMV2_DEBUG run them on every call's
// inputs before its attention kernels; the checks themselves are exercised
// on the host by the test suite.
//
// A kept-block row of a query whose eligible blocks are 0 .. n_elig-1 is what
// the top-k selection writes (xugj520.cn, section 1.1: the initial blocks and
// the sliding window are always kept; shadowrocket9.top, InfLLM v2 section:
// top-k blocks per query): min(topk, n_elig) strictly ascending block ids in
// [0, n_elig), the forced ones among them, then -1 padding.  The kernels
// guard against other rows (a list is cut at its first id out of range), so
// a malformed row gives a wrong result, not a fault; these checks say which.
//
// A tree mask row (xugj520.cn, section 1.1: uint64 mask for tree speculative
// decoding) names draft i's ancestors: bits below n_draft, none above i
// (drafts are stored parents first).  The kernels ignore bits at or above
// n_draft and always include draft i itself.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define INFLLMV2_HD __host__ __device__
#else
#define INFLLMV2_HD
#endif

namespace infllmv2 {

enum DebugCode {
  kDbgOk = 0,
  kDbgRange = 1,       // a kept-block id outside [0, n_elig)
  kDbgOrder = 2,       // ids not strictly ascending (a duplicate or a swap)
  kDbgPadding = 3,     // a -1 before a block id
  kDbgForced = 4,      // an initial or local-window block missing
  kDbgCount = 5,       // not min(topk, n_elig) ids
  kDbgMaskHigh = 6,    // a tree mask bit at or above n_draft
  kDbgMaskLater = 7,   // a tree mask bit naming a later draft
};

// Row of `topk` entries for a query whose own block is n_elig - 1.
INFLLMV2_HD inline int check_block_row(const int32_t* row, int topk, int n_elig, int init,
                                       int local) {
  int n = 0;
  int32_t prev = -1;
  bool pad = false;
  for (int i = 0; i < topk; ++i) {
    const int32_t b = row[i];
    if (b == -1) {
      pad = true;
      continue;
    }
    if (pad) return kDbgPadding;
    if (b < 0 || b >= n_elig) return kDbgRange;
    if (b <= prev) return kDbgOrder;
    prev = b;
    ++n;
  }
  const int want = topk < n_elig ? topk : n_elig;
  // forced blocks: [0, init) and [own - local + 1, own], the eligible ones
  const int own = n_elig - 1;
  auto kept = [&](int f) {
    for (int i = 0; i < n; ++i)
      if (row[i] == f) return true;
    return false;
  };
  for (int f = 0; f < init && f < n_elig; ++f)
    if (!kept(f)) return kDbgForced;
  for (int f = own - local + 1 > 0 ? own - local + 1 : 0; f <= own; ++f)
    if (!kept(f)) return kDbgForced;
  if (n != want) return kDbgCount;
  return kDbgOk;
}

// Mask row i of an n_draft-draft tree.
INFLLMV2_HD inline int check_tree_mask(uint64_t mask, int i, int n_draft) {
  const uint64_t below = n_draft >= 64 ? ~0ull : ((1ull << n_draft) - 1ull);
  if (mask & ~below) return kDbgMaskHigh;
  const uint64_t upto_i = i >= 63 ? ~0ull : ((2ull << i) - 1ull);
  if (mask & ~upto_i) return kDbgMaskLater;
  return kDbgOk;
}

}  // namespace infllmv2
