// One wave's top-k selection of one row (blocks ranked by score, ties to
// the lower index, forced initial and local blocks always kept), shared by
// the top-k kernel and the decode kernels that select their own rows.
// Sources: "MiniCPM 4.0" blog (shadowrocket9.top), InfLLM v2 section (each
// query keeps its top-k most relevant blocks, k = 64); "MiniCPM4: running
// LLMs on phones and PCs" (xugj520.cn), section 1.1 (initial tokens and a
// sliding window are always kept).
#pragma once

#include "topk_common.h"

namespace infllmv2 {

// ---------------------------------------------------------------------------
// One wave selects one (row, KV head) whose eligible blocks fit in registers
// (64 * KPL of them): lane l holds the scores of blocks b = l + 64 j
// (coalesced loads; ascending block order is (j, lane) order).  The top-k
// kernel runs four such waves per workgroup; the selecting decode kernels run
// it in each split's wave before its copies start.
//   1. Non-candidates (forced blocks, blocks past the row) become NaN, which
//      no comparison admits; only the 64-block pieces that reach them are
//      touched.
//   2. Lower bound lo: at least `need` lanes hold a score >= the need-th
//      largest lane maximum, so the threshold is >= it.  A bitwise search
//      over the 64 lane-maximum keys finds it.
//   3. Survivors (score >= lo, typically 100-260 of 2048) are compacted
//      into LDS as (score, block) in ascending block order, from ballots.
//   4. The threshold T (the need-th largest survivor key), the ranks of the
//      ties at T (lowest index first) and the output slots all come from
//      ballots over the survivors, at most kWaveSurvivors / 64 per lane.
// Rows where the bound is not finite (fewer than `need` finite lane maxima,
// or need > 64) or whose survivors overflow take a search over every key.
// Scores compare as floats in steps 1-3 (-0 == +0); keys are the
// order-preserving uint32 images, NaN candidates ranking below -inf.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float vmax3(float x, float y, float z) {
  // plain v_max3_f32: NaN operands are ignored, and no canonicalising
  // instructions are inserted for loaded values
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

constexpr int kWaveSurvivors = 512;   // per wave; a 2048-block row keeps ~100-260

// The k-th largest of one key per lane (1 <= k <= 64; hi = the largest).
// Close to either end (top-64 rows need the 61st largest = 4th smallest,
// top-6 rows the 3rd largest), a few wave extrema, each removing all lanes
// equal to it, find it; otherwise the bitwise search, whose early stop may
// land between two lane values, then the smallest lane value at or above.
__device__ __forceinline__ uint32_t kth_largest_of_lanes(uint32_t v, int k, uint32_t hi) {
  const bool from_top = k <= 32;
  int r = from_top ? k : 65 - k;         // rank from the nearer end
  if (r <= 8) {
    for (;;) {
      const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(from_top ? wave_max_u32(v) : wave_min_u32(v)));
      const int c = __popcll(__ballot(v == e));
      if (c >= r) return e;
      r -= c;
      v = v == e ? (from_top ? 0u : 0xffffffffu) : v;
    }
  }
  const uint32_t key[1] = {v};
  bool ex = false;
  const uint32_t t = threshold_search<1>(key, k, 0u, hi, &ex);
  return t == 0u ? 0u
                 : (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)wave_min_u32(v >= t ? v : 0xffffffffu));
}

// Step 4 over n_s survivors held as (score bits, block) in ascending block
// order, SPL per lane (n_s <= 64 SPL): the need-th largest key T, the ties
// at T taken lowest index first, the chosen blocks written to out[f_init ..
// f_init + need) in ascending order.
template <int SPL>
__device__ __forceinline__ void select_survivors(const int2* svw, int n_s, int need,
                                                 uint32_t lo_key, uint32_t hi_key, int f_init,
                                                 int32_t* out, int lane) {
  uint32_t sk[SPL];
  int32_t sbk[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int q = lane + 64 * i;
    const int2 e = svw[q];
    sk[i] = q < n_s ? orderable_key(__int_as_float(e.x)) : 0u;   // survivors: keys > 0
    sbk[i] = e.y;
  }
  bool exact = false;
  const uint32_t T = threshold_search<SPL>(sk, need, lo_key, hi_key, &exact);
  int take = 0;
  if (!exact) {
    int gt = 0;
#pragma unroll
    for (int i = 0; i < SPL; ++i) gt += __popcll(__ballot(sk[i] > T));
    take = need - gt;
  }
  // (i, lane) order is block order
  int slot = f_init, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    bool sel;
    if (exact) {
      sel = sk[i] >= T;
    } else {
      const uint64_t eqm = __ballot(sk[i] == T);
      const int rank = eq_seen + lanes_below(eqm);
      eq_seen += __popcll(eqm);
      sel = sk[i] > T || (sk[i] == T && rank < take);
    }
    const uint64_t selm = __ballot(sel);
    if (sel) out[slot + lanes_below(selm)] = sbk[i];
    slot += __popcll(selm);
  }
}

// The kept blocks of one row, chosen by one wave and written in ascending
// order to out[0, topk): the row's own block is b_own (b_own < nb_cap and
// b_own < 64 * KPL), its scores are S[0, nb_cap), and svw is the wave's LDS
// staging of kWaveSurvivors + 64 entries.  Rows with every eligible block
// inside the budget keep them all.
template <int KPL>
__device__ __forceinline__ void wave_select_row(const float* S, int64_t nb_cap, int b_own,
                                                int topk, int init, int local, int2* svw,
                                                int32_t* out, int lane) {
  const int n_elig = b_own + 1;
  if (n_elig <= topk) {
    for (int i = lane; i < topk; i += 64) out[i] = i < n_elig ? i : -1;
    return;
  }
  const int f_init = init < n_elig ? init : n_elig;
  const int f_lo = b_own - local + 1 > 0 ? b_own - local + 1 : 0;
  const int overlap = f_init > f_lo ? f_init - f_lo : 0;
  const int n_forced = f_init + (n_elig - f_lo) - overlap;
  const int need = topk - n_forced;

  // Here n_elig > topk >= init + local, so the forced blocks are the two
  // disjoint runs [0, f_init) and [f_lo, n_elig), and the candidates are
  // exactly the blocks in between: [f_init, f_lo).  The output is the first
  // run, the chosen candidates in ascending order, then the second run.
  // Entries past n_elig but inside the row (< nb_cap) are read as they are
  // and never become candidates, so a row of at least 64 * KPL entries needs
  // no index clamp.
  const uint32_t span = (uint32_t)(f_lo - f_init);
  auto is_cand = [&](int j) { return (uint32_t)(lane + 64 * j - f_init) < span; };
  float x[KPL];
  if (nb_cap >= 64 * KPL) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) x[j] = S[lane + 64 * j];
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int b = lane + 64 * j;
      x[j] = S[b < n_elig ? b : n_elig - 1];
    }
  }
  // the out slots: [0, f_init) init run, [f_init, lim) chosen, then the local run
  const int lim = f_init + (need > 0 ? need : 0);
  const int n_local = n_elig - f_lo;

  // fast path: steps 1-4 above
  bool done = need <= 0;
  if (need > 0 && need <= 64) {
    // in place: a candidate keeps its score (the full search below tests
    // is_cand itself and reads candidates only)
    // (on the vector ALU: the scalar unit carries this kernel's searches)
    const float qnan = __builtin_nanf("");
    const uint32_t c0 = (uint32_t)(lane - f_init);
#pragma unroll
    for (int j = 0; j < KPL; ++j) x[j] = c0 + 64u * j < span ? x[j] : qnan;
    float mx = x[0];
    int j0 = 1;
#pragma unroll
    for (; j0 + 1 < KPL; j0 += 2) mx = vmax3(mx, x[j0], x[j0 + 1]);
    if (j0 < KPL) mx = vmax3(mx, x[j0], x[j0]);
    // lane maximum key (NaN: no candidate -> 0) and the wave's largest
    const uint32_t mk[1] = {orderable_key(mx)};
    const uint32_t hk = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_max_u32(mk[0]));
    // the need-th largest lane maximum (0 if fewer than `need` lanes hold
    // one; empty lanes hold 0)
    const uint32_t lo_key = kth_largest_of_lanes(mk[0], need, hk);
    if (lo_key > orderable_key(-INFINITY)) {
      // lo as a float, by the inverse of the key map: y >= lo  <=>
      // key(y) >= lo_key for every non-NaN y (lo_key is a lane maximum's key,
      // at most key(+inf))
      const float lo = __uint_as_float((lo_key & 0x80000000u) ? (lo_key & 0x7fffffffu) : ~lo_key);
      // n_s only grows: once a piece does not fit, no later one does, and
      // n_s > kWaveSurvivors afterwards sends the row to the full search.
      // Lanes that keep nothing write a dummy slot (no branch per piece).
      int n_s = 0;                 // wave-uniform
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const bool keep = x[j] >= lo;
        const uint64_t m = __ballot(keep);
        const int c = __popcll(m);
        const bool ok = keep && n_s + c <= kWaveSurvivors;
        svw[ok ? n_s + lanes_below(m) : kWaveSurvivors + lane] =
            make_int2(__float_as_int(x[j]), lane + 64 * j);
        n_s += c;
      }
      if (n_s <= kWaveSurvivors) {
        __builtin_amdgcn_wave_barrier();
        if (n_s <= 256)
          select_survivors<4>(svw, n_s, need, lo_key, hk, f_init, out, lane);
        else
          select_survivors<kWaveSurvivors / 64>(svw, n_s, need, lo_key, hk, f_init, out, lane);
        done = true;
      }
    }
  }
  if (!done) {
    // every key: the bitwise search over all of them
    uint32_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const uint32_t k = orderable_key(x[j]);
      key[j] = is_cand(j) ? (k > 1u ? k : 1u) : 0u;
    }
    uint32_t hi = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) hi = key[j] > hi ? key[j] : hi;
    hi = wave_max_u32(hi);
    bool exact = false;
    const uint32_t T = threshold_search<KPL>(key, need, 0u, hi, &exact);
    int take = 0;
    if (!exact) {
      int gt = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) gt += __popcll(__ballot(key[j] > T));
      take = need - gt;
    }
    // chosen candidates go to slots f_init, f_init + 1, ... in ascending
    // order, staged in LDS
    int base = f_init, eq_seen = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      bool sel;
      if (exact) {
        sel = key[j] >= T;
      } else {
        const uint64_t eqm = __ballot(key[j] == T);
        const int rank = eq_seen + lanes_below(eqm);
        eq_seen += __popcll(eqm);
        sel = key[j] > T || (key[j] == T && rank < take);
      }
      const uint64_t selm = __ballot(sel);
      const int slot = base + lanes_below(selm);
      const int ok = (int)sel & (int)(slot < lim);           // no short-circuit branch
      svw[ok ? slot : kWaveSurvivors + lane].y = lane + 64 * j;
      base += __popcll(selm);
    }
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < topk; i += 64)
      if (i >= f_init && i < lim) out[i] = svw[i].y;
  }
  // the forced runs and the padding
  for (int i = lane; i < topk; i += 64) {
    if (i < f_init) out[i] = i;
    else if (i >= lim) out[i] = i < lim + n_local ? f_lo + (i - lim) : -1;
  }
}

}  // namespace infllmv2
