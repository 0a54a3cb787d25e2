// Host build of the kept-block and tree-mask checks (plain C++, no GPU):
// each case prints "<name> <code>" for the test suite to compare.
#include <cstdio>
#include <cstdint>

#include "../block_sparse_long_infllmv2_amd/csrc/debug_checks.h"

using namespace infllmv2;

static void row(const char* name, const int32_t* r, int topk, int n_elig, int init, int local) {
  std::printf("%s %d\n", name, check_block_row(r, topk, n_elig, init, local));
}

int main() {
  // topk 6, init 1, local 2, query in block 9 (eligible 0..9): forced 0, 8, 9
  const int32_t good[6] = {0, 3, 4, 7, 8, 9};
  const int32_t range[6] = {0, 3, 4, 7, 8, 10};
  const int32_t order[6] = {0, 4, 3, 7, 8, 9};
  const int32_t dup[6] = {0, 3, 3, 7, 8, 9};
  const int32_t pad[6] = {0, 3, -1, 7, 8, 9};
  const int32_t forced[6] = {1, 3, 4, 7, 8, 9};
  const int32_t local[6] = {0, 2, 3, 4, 7, 9};
  const int32_t count[6] = {0, 3, 8, 9, -1, -1};
  const int32_t neg[6] = {0, -2, 4, 7, 8, 9};
  row("good", good, 6, 10, 1, 2);
  row("range", range, 6, 10, 1, 2);
  row("order", order, 6, 10, 1, 2);
  row("duplicate", dup, 6, 10, 1, 2);
  row("padding", pad, 6, 10, 1, 2);
  row("forced_init", forced, 6, 10, 1, 2);
  row("forced_local", local, 6, 10, 1, 2);
  row("count", count, 6, 10, 1, 2);
  row("negative", neg, 6, 10, 1, 2);
  // fewer eligible blocks than topk: all of them, then padding
  const int32_t few[6] = {0, 1, 2, 3, -1, -1};
  const int32_t few_short[6] = {0, 1, 3, -1, -1, -1};
  row("few_good", few, 6, 4, 1, 2);
  row("few_short", few_short, 6, 4, 1, 2);
  // tree masks (n_draft 5): ancestors of draft 3 are 0, 1
  std::printf("mask_good %d\n", check_tree_mask(0b1011ull, 3, 5));
  std::printf("mask_no_self %d\n", check_tree_mask(0b0011ull, 3, 5));
  std::printf("mask_high %d\n", check_tree_mask((1ull << 5) | 1ull, 3, 5));
  std::printf("mask_later %d\n", check_tree_mask(0b10001ull, 3, 5));
  std::printf("mask_bit63 %d\n", check_tree_mask(1ull << 63, 63, 64));
  return 0;
}
