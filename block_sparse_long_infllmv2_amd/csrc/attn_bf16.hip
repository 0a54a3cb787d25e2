// Block-sparse causal attention over the kept blocks, bf16 inputs, float32
// accumulation, on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
// Sources: "MiniCPM4: running LLMs on phones and PCs" (xugj520.cn), section
// 1.1 (attention is computed on the selected blocks only; initial and local
// blocks always kept; uint64 tree mask); "MiniCPM 4.0" blog (shadowrocket9.top),
// InfLLM v2 section (64-token blocks, top-64, dense below 8192 tokens);
// pomoai.com CPM.cu article, sections 2 and 4 (tree verification inside the
// attention kernel, chunked prefill).
//
// Layout of the work inside a wave (64 lanes): the wave owns 32 query rows
// (32/G tokens x the G heads of one KV group, which share every selection).
// Scores are computed transposed, S^T = K Q^T, with K as the A operand
// (32 keys x 16 dims) and Q^T as the B operand held in registers, so each
// lane's accumulator column is ONE query row: the row max needs a single
// exchange between the two half-waves and the row sum none until the end.
// P^T then feeds the P.V product directly from the accumulator registers as
// the B operand of O^T = V^T P^T; V^T comes from LDS, where V is written
// transposed while it is staged.
//
// Work units are 64-key chunks of kept blocks.  A workgroup stages each chunk
// (K as [key][d], V as [d][key], both padded against bank conflicts) into a
// double-buffered LDS ring with one barrier per chunk; the next chunk is
// prefetched into registers while the current one is multiplied.
//   prefill: a workgroup owns TT consecutive query tokens of one KV head and
//            walks the union of their kept blocks (built in LDS by a bitonic
//            sort of the tokens' block lists); a wave skips chunks that none
//            of its tokens kept, and masks rows of tokens that did not keep it.
//   decode:  (sequence, KV head, split) workgroups walk a slice of the
//            sequence's kept blocks and write float32 partials (o, m, l).
//   tree:    (KV head, split) workgroups walk a slice of the union of all
//            drafts' kept blocks plus one chunk holding the draft tokens
//            (masked by the uint64 ancestor mask); partials as in decode.
//   combine: merges the split partials with their log-sum-exp weights.
#include <mutex>

#include "lds_tiles.h"
#include "topk_wave.h"

namespace infllmv2 {

template <int D>
struct Lds {
  static constexpr int kKStride = D + 8;         // bf16 elements per staged K row
  static constexpr int kVStride = kChunk + 8;    // bf16 elements per staged V^T row
  static constexpr int kKElems = kChunk * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kStageElems = kKElems + kVElems;
  static constexpr int kBytes = 2 * kStageElems * 2;   // double-buffered
};

// ---------------------------------------------------------------------------
// Staging of one 64-key chunk: keys [key0, key0 + nvalid) of a K/V row block.
// ---------------------------------------------------------------------------
// V^T rows hold the 64 keys of a chunk in a permuted order: key bits 2 and 3
// are swapped, so that the 8 keys one lane needs for a P.V k-step
// (16t + 4h + {0..3} and 16t + 8 + 4h + {0..3}) sit in 16 contiguous bytes.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D, int NT>
struct Stager {
  // K: thread t owns kKPer consecutive keys of one 16-byte column chunk:
  //    key = kKPer * (t / CPR) + i, chunk = t % CPR  (CPR = D/8 chunks per row).
  //    Its global pieces sit at immediate offsets 0, 2D, 4D, ... bytes.
  // V: thread t owns key pairs kp = t % 32 for chunks c = t / 32 + (NT/32) * i,
  //    i.e. rows 2kp and 2kp+1 of kVPer chunks (again immediate offsets).
  static constexpr int CPR = D / 8;
  static constexpr int kKPer = kChunk * CPR / NT;
  static constexpr int kVJobs = (kChunk / 2) * CPR;
  static constexpr int kVPer = (kVJobs + NT - 1) / NT;
  static_assert(kKPer >= 1 && (kChunk * CPR) % NT == 0, "K staging shape");
  u32x4 kr[kKPer];
  u32x4 vr[kVPer][2];

  __device__ static __forceinline__ int k_key0(int tid) { return kKPer * (tid / CPR); }
  __device__ static __forceinline__ int k_chunk(int tid) { return tid % CPR; }
  __device__ static __forceinline__ int v_pair(int tid) { return tid % (kChunk / 2); }
  __device__ static __forceinline__ int v_chunk(int tid, int i) {
    return tid / (kChunk / 2) + (NT / (kChunk / 2)) * i;
  }

  // kbase/vbase point at key 0 of the chunk (or at any valid row when
  // nvalid == 0); keys >= nvalid are zero-filled so that masked lanes never
  // multiply garbage.  Full chunks take the branch-free path.
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase,
                                       int nvalid, int tid) {
    const int kk0 = k_key0(tid), kc = k_chunk(tid);
    const int vk0 = 2 * v_pair(tid);
    if (nvalid == kChunk) {
      const uint16_t* kp = kbase + kk0 * D + kc * 8;
#pragma unroll
      for (int i = 0; i < kKPer; ++i) kr[i] = ldg16(kp + i * D);
      const uint16_t* vp = vbase + vk0 * D;
#pragma unroll
      for (int i = 0; i < kVPer; ++i) {
        const int c = v_chunk(tid, i);
        if (kVJobs % NT != 0 && c >= CPR) break;
        vr[i][0] = ldg16(vp + c * 8);
        vr[i][1] = ldg16(vp + D + c * 8);
      }
      return;
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int key = kk0 + i;
      const bool ok = key < nvalid;
      const u32x4 x = ldg16(kbase + (ok ? key : 0) * D + kc * 8);
      kr[i] = ok ? x : z;
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int c = v_chunk(tid, i);
      const bool in = c < CPR;
      const bool ok0 = in && vk0 < nvalid, ok1 = in && vk0 + 1 < nvalid;
      const u32x4 x0 = ldg16(vbase + (ok0 ? vk0 : 0) * D + (in ? c : 0) * 8);
      const u32x4 x1 = ldg16(vbase + (ok1 ? vk0 + 1 : 0) * D + (in ? c : 0) * 8);
      vr[i][0] = ok0 ? x0 : z;
      vr[i][1] = ok1 ? x1 : z;
    }
  }

  __device__ __forceinline__ void store(uint16_t* stage, int tid) const {
    uint16_t* Ks = stage + k_key0(tid) * Lds<D>::kKStride + k_chunk(tid) * 8;
#pragma unroll
    for (int i = 0; i < kKPer; ++i)
      *reinterpret_cast<u32x4*>(Ks + i * Lds<D>::kKStride) = kr[i];
    // keys 2kp, 2kp+1 stay adjacent in the permuted V^T row order
    uint16_t* Vt = stage + Lds<D>::kKElems + vt_pos(2 * v_pair(tid));
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int c = v_chunk(tid, i);
      if (kVJobs % NT != 0 && c >= CPR) break;
      const uint32_t a[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
      const uint32_t b[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims c*8 + 2e (low halves) and c*8 + 2e + 1 (high halves)
        const uint32_t lo = __builtin_amdgcn_perm(b[e], a[e], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(b[e], a[e], 0x07060302u);
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + 2 * e) * Lds<D>::kVStride) = lo;
        *reinterpret_cast<uint32_t*>(Vt + (c * 8 + 2 * e + 1) * Lds<D>::kVStride) = hi;
      }
    }
  }
};


// Per-lane fragment addresses inside a swizzled tile.
//   K, A operand of S^T = K Q^T: lane (col, half), k-step ks reads row
//     32 kt + col, logical chunk 2 ks + half (kt adds 32 rows).
//   V^T A operand of O^T = V^T P^T, d-tile dt: element e of half h is key
//     16 t + 8 (e/4) + 4 h + e%4 of tile kt, at d = 32 dt + col.  Two
//     transposing reads (e/4 = 0, 1) each give 4 keys; lane L addresses key
//     8 c' + 4 h + (L%16)/4 (+ 32 kt + 16 t) and d = 32 dt + 16 ((L/16)%2) + 4 (L%4).
// Position bits of a chunk (bits 4.. of the byte offset inside a row) never
// overlap the row bits, so k-step ks and d-tile dt enter as XOR masks:
//   K:  (2 ks + half) ^ f = 2 ks ^ (half ^ f)  ->  k0 ^ (32 ks)
//   V:  (4 dt + 2 g + q/2) ^ f = 4 dt ^ (...)  ->  v0[c'] ^ (64 dt)
template <int D>
struct FragAddr {
  uint32_t k0;
  uint32_t v0[2];
  __device__ __forceinline__ void init(int lane) {
    constexpr int RB = Swz<D>::RB;
    const int col = lane & 31, half = lane >> 5;
    k0 = (uint32_t)(col * RB + ((half ^ Swz<D>::f(col)) * 16));
    const int g = (lane >> 4) & 1, j = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 8 * c + 4 * half + j;
      v0[c] = (uint32_t)(row * RB + (((2 * g + (q >> 1)) ^ Swz<D>::f(row)) * 16) + 8 * (q & 1));
    }
  }
  __device__ __forceinline__ uint32_t k(int ks) const { return k0 ^ (uint32_t)(32 * ks); }
  __device__ __forceinline__ uint32_t v(int dt, int c) const { return v0[c] ^ (uint32_t)(64 * dt); }
};

// ---------------------------------------------------------------------------
// Per-wave online-softmax state for 32 query rows (one row per lane column).
// The running max m is only raised when a block's max exceeds it by more
// than kRescaleSlack (log2 units): exponentials then stay below 2^slack, which
// float32 sums and bf16 P fragments hold without loss, and the O rescale runs
// rarely.  The result is unchanged: numerator and denominator use the same m.
// ---------------------------------------------------------------------------
constexpr float kRescaleSlack = 8.0f;
template <int D>
struct RowState {
  bf16x8 q[D / 16];      // Q^T B-operand fragments (row = lane % 32)
  f32x16 o[D / 32];      // O^T accumulators: rows d = 32*dt + 8*(v/4) + 4*half + v%4
  float m, l;            // running max (log2 domain) and this half's sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] = 0.0f;
    m = kNoMax;
    l = 0.0f;
  }

  // One staged 64-key chunk.  `lim` = largest valid key offset (0..63) inside
  // the chunk for this lane's row, or -1 if the row keeps none of it.
  // `draft_bits` (tree chunk) restricts the valid offsets further.
  // P^T fragments of one chunk: k-step t of key tile kt.
  struct PFrag { bf16x8 f[2][2]; };

  // S^T = K Q^T for one staged chunk, masked online softmax; returns the
  // P^T fragments (and rescales O when the running max moves).
  // kfrag(kt, ks): this lane's A fragment of key tile kt, k-step ks.
  // LA > 0: software pipeline, LA fragments read ahead of the MFMA that uses
  // them (the two key tiles' accumulation chains alternate).
  template <int LA = 0, class KFrag>
  __device__ __forceinline__ PFrag scores(KFrag kfrag, int lim, bool use_bits,
                                          uint64_t draft_bits, float scale_log2) {
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = 0.0f;
    if constexpr (LA > 0) {
      constexpr int NM = 2 * (D / 16);
      static_assert(LA < NM, "lookahead");
      bf16x8 a[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) a[m] = kfrag(m & 1, m >> 1);
#pragma unroll
      for (int m = 0; m < NM; ++m)
        s[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], q[m >> 1], s[m & 1], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);        // LDS reads
#pragma unroll
      for (int m = 0; m < NM - LA; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 a[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) a[ks] = kfrag(kt, ks);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], q[ks], s[kt], 0, 0, 0);
      }
    }
    // Scale into the log2 domain, mask, row max, exponentials.  Common case
    // (every row of the wave keeps all 64 keys or none of them): no per-key
    // masking -- rows that keep nothing subtract +inf, so their p is 0.
    const bool partial = (lim >= 0 && lim < kChunk - 1) || use_bits;
    const bool keep = lim >= 0;
    float m_new, alpha, psum = 0.0f;
    if (!__ballot(partial)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
      mx = keep ? mx * scale_log2 : -INFINITY;
      mx = fmaxf(mx, swap_halves(mx));
      m_new = mx > m + kRescaleSlack ? mx : m;
      alpha = fast_exp2(m - m_new);
      const float msub = keep ? m_new : INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(s[kt][v], scale_log2, -msub));
          s[kt][v] = p;
          psum += p;
        }
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = 32 * kt + 8 * (v >> 2) + 4 * half + (v & 3);
          bool ok = off <= lim;
          if (use_bits) ok = ok && ((draft_bits >> off) & 1ull);
          const float x = ok ? s[kt][v] * scale_log2 : -INFINITY;
          s[kt][v] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, swap_halves(mx));
      m_new = mx > m + kRescaleSlack ? mx : m;
      alpha = fast_exp2(m - m_new);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(s[kt][v] - m_new);
          s[kt][v] = p;
          psum += p;
        }
    }
    m = m_new;
    l = l * alpha + psum;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
    }
    // P^T fragments: k-step t of key tile kt uses accumulator entries 8t..8t+7
    PFrag pf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf.f[kt][t][e] = (__bf16)s[kt][8 * t + e];
    return pf;
  }

  // O^T += V^T P^T; A-operand element e of half h <-> key 16t + 8(e/4) + 4h + e%4.
  // Run for every staged chunk (with zero P when the wave keeps none of it),
  // so that O flows through the same instructions on every iteration.
  // vfrag(dt, kt, t): this lane's A fragment of V^T rows 32 dt.., k-step t of
  // key tile kt.
  // LA > 0: k-step outer, d-tile inner (consecutive MFMAs are independent),
  // LA fragments (2 LDS reads each) read ahead of their MFMA.
  template <int LA = 0, class VFrag>
  __device__ __forceinline__ void pv(VFrag vfrag, const PFrag& pf) {
    const auto& pb = pf.f;
    if constexpr (LA > 0) {
      constexpr int NDT = D / 32, NF = 4 * NDT;
      static_assert(LA < NF, "lookahead");
      bf16x8 b[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) b[f] = vfrag(f % NDT, f / NDT / 2, (f / NDT) & 1);
#pragma unroll
      for (int f = 0; f < NF; ++f)
        o[f % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[f], pb[f / NDT / 2][(f / NDT) & 1],
                                                             o[f % NDT], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
      for (int f = 0; f < NF - LA; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
      return;
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      bf16x8 a[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t) a[kt][t] = vfrag(dt, kt, t);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kt][t], pb[kt][t], o[dt], 0, 0, 0);
    }
  }

  // ---- split form for the software-pipelined loop ------------------------
  // S^T = K Q^T only (LA fragments read ahead of their MFMA).
  template <int LA, class KFrag>
  __device__ __forceinline__ void qk(KFrag kfrag, f32x16 (&s)[2]) const {
    constexpr int NM = 2 * (D / 16);
    static_assert(LA > 0 && LA < NM, "lookahead");
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = 0.0f;
    bf16x8 a[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) a[m] = kfrag(m & 1, m >> 1);
#pragma unroll
    for (int m = 0; m < NM; ++m)
      s[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], q[m >> 1], s[m & 1], 0, 0, 0);
  }

  // Online softmax of one chunk's S^T (this lane's row), without the O
  // rescale: returns P^T and sets alpha = 2^(m_old - m_new) (1 when the
  // running max stays).  MASKED: per-key limit `lim` and draft bits;
  // otherwise every row keeps all 64 keys (lim = 63) or none (lim = -1).
  template <bool MASKED>
  __device__ __forceinline__ PFrag softmax(f32x16 (&s)[2], int lim, bool use_bits,
                                           uint64_t draft_bits, float scale_log2,
                                           float& alpha) {
    const int half = (threadIdx.x & 63) >> 5;
    const bool keep = lim >= 0;
    float mx = -INFINITY;
    if constexpr (!MASKED) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
      mx = keep ? mx * scale_log2 : -INFINITY;
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = 32 * kt + 8 * (v >> 2) + 4 * half + (v & 3);
          bool ok = off <= lim;
          if (use_bits) ok = ok && ((draft_bits >> off) & 1ull);
          const float x = ok ? s[kt][v] * scale_log2 : -INFINITY;
          s[kt][v] = x;
          mx = fmaxf(mx, x);
        }
    }
    // the other half-wave holds the other 32 keys of this row
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float m_new = mx > m + kRescaleSlack ? mx : m;
    alpha = fast_exp2(m - m_new);
    float psum = 0.0f;
    if constexpr (!MASKED) {
      const float msub = keep ? m_new : INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(s[kt][v], scale_log2, -msub));
          s[kt][v] = p;
          psum += p;
        }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(s[kt][v] - m_new);
          s[kt][v] = p;
          psum += p;
        }
    }
    m = m_new;
    l = l * alpha + psum;
    PFrag pf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf.f[kt][t][e] = (__bf16)s[kt][8 * t + e];
    return pf;
  }

  // Partial chunk: scores of keys past `lim` (or outside the draft bits) ->
  // -inf, after which the unmasked softmax gives them p = 0.
  __device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int lim, bool use_bits,
                                              uint64_t draft_bits) const {
    const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = 32 * kt + 8 * (v >> 2) + 4 * half + (v & 3);
        bool ok = off <= lim;
        if (use_bits) ok = ok && ((draft_bits >> off) & 1ull);
        s[kt][v] = ok ? s[kt][v] : -INFINITY;
      }
  }

  __device__ __forceinline__ void rescale(float alpha) {
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
    }
  }
};

// Load this lane's Q^T fragments: row `qrow` (NULL -> zeros).
template <int D>
__device__ __forceinline__ void load_q(RowState<D>& st, const uint16_t* qrow) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow) w = ldg16(qrow + 16 * ks + 8 * half);
    st.q[ks] = *reinterpret_cast<const bf16x8*>(&w);
  }
}


// Entries a split workgroup may hold in LDS (host keeps units per split below).
constexpr int kSplitEntryCap = 64;


// Instruction order for a block holding NM QK MFMAs and their NM fragment
// reads (and, with VALU > 0, another chunk's softmax): LA reads first, then
// each MFMA followed by the next read and up to VALU vector instructions.
template <int NM, int LA, int VALU>
__device__ __forceinline__ void sched_qk() {
  __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);          // LDS reads
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    if (m + LA < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (VALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);
  }
}
// fragments read ahead of their MFMA in the directly staged loop
#ifndef INFLLMV2_LOOKAHEAD
#define INFLLMV2_LOOKAHEAD 2
#endif
constexpr int kLookahead = INFLLMV2_LOOKAHEAD;
// vector instructions placed after each QK MFMA when a softmax runs beside it
#ifndef INFLLMV2_VALU_PER_MFMA
#define INFLLMV2_VALU_PER_MFMA 4
#endif
constexpr int kValuPerMfma = INFLLMV2_VALU_PER_MFMA;

// ---------------------------------------------------------------------------
// The attention kernel.
//   W waves, each 32 rows = TPW tokens x G heads; TT = W * TPW tokens.
// Indices are 32-bit inside the kernel: the host rejects caches with more
// than 2^31 - 1 tokens per (sequence, KV head).
// ---------------------------------------------------------------------------
template <int D, int G, int W, int MODE, int PF = 1>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = W * 64;
  constexpr int TPW = 32 / G;
  constexpr int TT = (MODE == kDecode) ? 1 : W * TPW;
  static_assert(TT <= 32, "token bitmask is 32 bits");
  static_assert(MODE != kPrefill || TT > 1, "prefill tiles hold several tokens");
  constexpr int SORT_N = (MODE == kPrefill) ? TT * kSortCap : 0;
  constexpr int ECAP = (MODE == kPrefill) ? TT * kSortCap : kSplitEntryCap;
  // PF 1/2: two padded K + V^T stages; PF 3/4: K0 K1 V0 V1 swizzled tiles
  constexpr int STAGE_ELEMS = PF >= 3 ? 2 * Swz<D>::TILE : 2 * Lds<D>::kStageElems;
  __shared__ __attribute__((aligned(16))) uint16_t stage[STAGE_ELEMS];
  __shared__ int2 ents[ECAP];
  __shared__ int scan_lds[NT / 64];
  static_assert(SORT_N * 4 <= (int)sizeof(stage), "sort buffer aliases the staging ring");

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;

  // ---- work item ---------------------------------------------------------
  int g, tile = 0, seq = 0, split = 0;
  if constexpr (MODE == kPrefill) {
    const int w = xcd_contiguous_index(blockIdx.x, gridDim.x);
    g = w / a.n_tiles;
    tile = w % a.n_tiles;
  } else {
    split = blockIdx.x;
    g = blockIdx.y;
    if constexpr (MODE == kDecode) seq = blockIdx.z; else tile = blockIdx.z;
  }

  // tokens of this workgroup and their query positions
  int n_keys, tok0, n_tok;
  if constexpr (MODE == kDecode) {
    // lengths outside [1, max_seqlen] are clamped: wrong input, no fault
    const int L = a.seqlens[seq];
    n_keys = L < 1 ? 1 : (L > (int)a.n_k ? (int)a.n_k : L);
    tok0 = seq;
    n_tok = 1;
  } else {
    n_keys = (int)a.n_k;
    tok0 = tile * TT;
    n_tok = min(TT, a.n_rows - tok0);
  }
  const bool dense = n_keys < a.dense_len || a.block_idx == nullptr;
  const int n_b = (n_keys + a.B - 1) / a.B;
  const int cpb = (a.B + kChunk - 1) / kChunk;            // chunks per block
  const uint32_t full_mask = n_tok >= 32 ? 0xffffffffu : ((1u << n_tok) - 1u);
  // first query position of the tile (prefill: consecutive positions)
  const int p0 = (MODE == kPrefill) ? (int)a.n_k - a.n_rows + tok0 : n_keys - 1;

  // this lane's row
  const int t_in_wave = col / G, head_in_group = col % G;
  const int my_t = (MODE == kDecode) ? (wave == 0 && t_in_wave == 0 ? 0 : 32)
                                     : wave * TPW + t_in_wave;   // 32 = none
  const bool row_ok = my_t < n_tok;
  const int my_row = tok0 + (row_ok ? my_t : 0);
  const int my_head = g * G + head_in_group;
  const int my_pos = (MODE == kPrefill) ? p0 + (row_ok ? my_t : 0) : n_keys - 1;

  // ---- entries (kept blocks with token masks) and this workgroup's units ---
  const bool has_draft = MODE == kTree;
  int n_entries;
  if constexpr (MODE == kPrefill) {
    if (dense) {
      n_entries = (p0 + n_tok - 1) / a.B + 1;
    } else {
      int N = 1;
      while (N < TT * a.topk) N <<= 1;
      n_entries = build_union<NT, TT>(a.block_idx, tok0, a.h_kv, g, n_tok, a.topk, n_b,
                                      reinterpret_cast<uint32_t*>(stage), N, ents, scan_lds);
    }
  } else if constexpr (MODE == kDecode) {
    if (dense) {
      n_entries = n_b;
    } else {
      // kept blocks = the leading valid entries of the list (topk <= 128)
      const int32_t* lst = a.block_idx + ((int64_t)seq * a.h_kv + g) * a.topk;
      int nn = a.topk;
#pragma unroll
      for (int hf = 1; hf >= 0; --hf) {
        const int i = 64 * hf + lane;
        const int32_t b = i < a.topk ? lst[i] : -1;
        const uint64_t bad = __ballot(i < a.topk && !(b >= 0 && b < n_b));
        if (bad) nn = 64 * hf + (int)__builtin_ctzll(bad);
      }
      n_entries = nn;
    }
  } else {
    n_entries = dense ? n_b : a.union_len[g];
  }
  const int n_units_total = n_entries * cpb + (has_draft ? 1 : 0);
  int u_begin = 0, u_end = n_units_total;
  if constexpr (MODE != kPrefill) {
    // balanced contiguous slices of this row's units over the n_split splits
    const int per = (n_units_total + a.n_split - 1) / a.n_split;
    u_begin = min(n_units_total, split * per);
    u_end = min(n_units_total, u_begin + per);
  }
  // split modes: copy this slice's entries into LDS (entry e -> ents[e - e_base])
  int e_base = 0;
  if constexpr (MODE != kPrefill) {
    if (!dense) {
      e_base = u_begin / cpb;
      const int e_end = min(n_entries, (u_end + cpb - 1) / cpb);
      for (int e = e_base + tid; e < e_end && e - e_base < kSplitEntryCap; e += NT) {
        if constexpr (MODE == kDecode) {
          ents[e - e_base] = make_int2(a.block_idx[((int64_t)seq * a.h_kv + g) * a.topk + e], 1);
        } else {
          const int64_t ix = (int64_t)g * a.union_cap + e;
          ents[e - e_base] = make_int2(a.union_blk[ix], (int)(uint32_t)(a.union_mask[ix] >> tok0));
        }
      }
      __syncthreads();
    }
  }

  // unit -> first key, #valid keys, token mask, draft flag
  struct UnitInfo { int key0, nv; uint32_t tm; bool isd; };
  // per-lane form (u may differ between lanes; u < n_units_total)
  auto unit_info_lane = [&](int u) -> UnitInfo {
    UnitInfo r;
    r.isd = has_draft && u == n_entries * cpb;
    if (r.isd) {
      r.key0 = 0; r.nv = a.n_rows; r.tm = full_mask;
      return r;
    }
    int e = u, c = 0;
    if (cpb != 1) { e = u / cpb; c = u - e * cpb; }
    int b;
    if (dense) {
      b = e;
      if constexpr (MODE == kPrefill) {
        // token t keeps block b iff b <= (p0 + t) / B, i.e. t >= b*B - p0
        const int t_min = b * a.B - p0;
        r.tm = t_min <= 0 ? full_mask : (t_min >= 32 ? 0u : (full_mask & (0xffffffffu << t_min)));
      } else {
        r.tm = full_mask;
      }
    } else {
      const int2 en = ents[e - e_base];
      b = en.x;
      r.tm = (uint32_t)en.y;
    }
    r.key0 = b * a.B + c * kChunk;
    const int blk_end = min((b + 1) * a.B, n_keys);
    r.nv = max(0, min(kChunk, blk_end - r.key0));
    return r;
  };
  auto unit_info = [&](int u) -> UnitInfo {
    UnitInfo r = unit_info_lane(u);
    // identical in every lane: keep them in scalar registers
    r.key0 = __builtin_amdgcn_readfirstlane(r.key0);
    r.nv = __builtin_amdgcn_readfirstlane(r.nv);
    r.tm = __builtin_amdgcn_readfirstlane(r.tm);
    return r;
  };

  const int64_t kv_head_off = (MODE == kDecode ? ((int64_t)seq * a.h_kv + g) : (int64_t)g) *
                              a.cap * D;
  const uint16_t* kbase_seq = a.k + kv_head_off;
  const uint16_t* vbase_seq = a.v + kv_head_off;
  const uint16_t* kdraft = has_draft ? a.k_draft + (int64_t)g * a.n_rows * D : nullptr;
  const uint16_t* vdraft = has_draft ? a.v_draft + (int64_t)g * a.n_rows * D : nullptr;
  auto kptr = [&](const UnitInfo& ui) {
    return ui.isd ? kdraft : kbase_seq + (ui.nv > 0 ? (int64_t)ui.key0 * D : 0);
  };
  auto vptr = [&](const UnitInfo& ui) {
    return ui.isd ? vdraft : vbase_seq + (ui.nv > 0 ? (int64_t)ui.key0 * D : 0);
  };

  RowState<D> st;
  st.init();
  load_q<D>(st, row_ok ? a.q + ((int64_t)my_row * a.h_q + my_head) * D : nullptr);
  uint64_t my_bits = 0;
  if (has_draft && row_ok) {
    const uint64_t full = a.n_rows >= 64 ? ~0ull : ((1ull << a.n_rows) - 1ull);
    my_bits = (a.tree_mask[my_row] & full) | (1ull << my_row);
  }

  // one staged chunk: largest key offset my row uses, -1 if none
  auto chunk_lim = [&](const UnitInfo& ui) {
    int lim = -1;
    if (row_ok && ((ui.tm >> my_t) & 1u)) {
      const int last = (ui.isd ? ui.nv - 1 : min(my_pos - ui.key0, ui.nv - 1));
      lim = last < 0 ? -1 : last;
    }
    return lim;
  };
  // scores + softmax when any row of the wave uses the chunk, else zero P
  auto chunk_scores = [&](auto kfrag, const UnitInfo& ui, int lim) {
    typename RowState<D>::PFrag pf;
    if (__ballot(lim >= 0)) {
      pf = st.scores(kfrag, lim, ui.isd, my_bits, a.scale_log2);
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf.f[kt][t][e] = (__bf16)0.0f;
    }
    return pf;
  };
  // padded layout (PF 1/2): K rows of kKStride, V^T rows of kVStride
  auto compute_chunk = [&](const uint16_t* buf, const UnitInfo& ui) {
    const uint16_t* krow = buf + col * Lds<D>::kKStride + 8 * half;
    const uint16_t* vrow = buf + Lds<D>::kKElems + col * Lds<D>::kVStride + 8 * half;
    auto kfrag = [&](int kt, int ks) {
      return *reinterpret_cast<const bf16x8*>(krow + 32 * kt * Lds<D>::kKStride + 16 * ks);
    };
    // keys 16t + 4h + {0..3} and 16t + 8 + 4h + {0..3}: the permuted V^T
    // rows put them at positions 16t + 8h .. +8
    auto vfrag = [&](int dt, int kt, int t) {
      return *reinterpret_cast<const bf16x8*>(vrow + 32 * dt * Lds<D>::kVStride + 32 * kt + 16 * t);
    };
    const typename RowState<D>::PFrag pf = chunk_scores(kfrag, ui, chunk_lim(ui));
    st.pv(vfrag, pf);
  };

  if constexpr (PF == 4) {
    // Direct staging with a software pipeline inside each wave: while the
    // matrix cores compute S^T = K Q^T of chunk i+1, the vector ALU runs the
    // softmax of chunk i (same basic block, so the scheduler interleaves
    // them); then O^T += V^T P^T of chunk i.  Chunk i sits in K[i&1], V[i&1].
    // One barrier per iteration, X_i: K(i+1) and V(i) have landed and every
    // wave is done with iteration i-1, so K(i+2) -> K[i&1] (read by QK(i)
    // in iteration i-1) and V(i+1) -> V[(i+1)&1] (read by PV(i-1)) are
    // issued right after it and have one iteration to arrive.
    __builtin_amdgcn_s_waitcnt(0x0f70);   // Q and draft mask loads: vmcnt(0)
    using DT = DmaTile<D, NT>;
    constexpr int TILE = Swz<D>::TILE;
    DT dma;
    dma.init(tid);
    FragAddr<D> fa;
    fa.init(lane);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)stage;
    const int n = u_end - u_begin;
    const UnitInfo none = {0, 0, 0u, false};
    // Metadata of 64 consecutive units, one unit per lane; unit u is taken
    // from lane u - wb with readlane (units are visited in increasing order,
    // so the window only moves forward).
    int wb = u_begin;
    UnitInfo wl = none;
    auto load_window = [&]() {
      const int uu = wb + lane;
      wl = uu < u_end ? unit_info_lane(uu) : none;
    };
    load_window();
    auto info = [&](int u) -> UnitInfo {
      if (u >= u_end) return none;
      if (u >= wb + 64) {
        wb += 64;
        load_window();
      }
      UnitInfo r;
      const int ln = u - wb;
      r.key0 = __builtin_amdgcn_readlane(wl.key0, ln);
      r.nv = __builtin_amdgcn_readlane(wl.nv, ln);
      r.tm = (uint32_t)__builtin_amdgcn_readlane((int)wl.tm, ln);
      r.isd = has_draft && u == n_entries * cpb;
      return r;
    };
    auto kfrag_at = [&](uint32_t kb) {
      return [=, &fa](int kt, int ks) {
        return lds_read16(kb + fa.k(ks) + kt * 32 * Swz<D>::RB);
      };
    };
    auto vfrag_at = [&](uint32_t vb) {
      return [=, &fa](int dt, int kt, int t) {
        const uint32_t off = vb + (32 * kt + 16 * t) * Swz<D>::RB;
        const bf16x4 lo = lds_read_tr8(off + fa.v(dt, 0));
        const bf16x4 hi = lds_read_tr8(off + fa.v(dt, 1));
        return (bf16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
    };
    UnitInfo I0 = info(u_begin), I1 = info(u_begin + 1), I2 = info(u_begin + 2);
    if (n > 0) {
      dma.issue(lds0, kptr(I0), I0.nv, tid, wave_u);
      dma.issue(lds0 + 2 * TILE, vptr(I0), I0.nv, tid, wave_u);
    }
    if (n > 1) dma.issue(lds0 + TILE, kptr(I1), I1.nv, tid, wave_u);
    wait_vm_barrier<0>();
    f32x16 sA[2], sB[2];
    int lim0 = n > 0 ? chunk_lim(I0) : -1;
    bool use0 = __ballot(lim0 >= 0) != 0;
    if (use0) st.template qk<kLookahead>(kfrag_at(lds0), sA);

    // iteration i: scores of chunk i in `sc`, chunk i+1's go to `sn`
    auto iter = [&](int i, auto stage_tag, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      constexpr int S = decltype(stage_tag)::value;
      const int u = u_begin + i;
      wait_vm_barrier<0>();
      if (i + 2 < n) dma.issue(lds0 + S * TILE, kptr(I2), I2.nv, tid, wave_u);
      if (i + 1 < n) dma.issue(lds0 + (3 - S) * TILE, vptr(I1), I1.nv, tid, wave_u);
      const int lim1 = i + 1 < n ? chunk_lim(I1) : -1;
      const bool use1 = __ballot(lim1 >= 0) != 0;
      const bool part0 = __ballot((lim0 >= 0 && lim0 < kChunk - 1) || I0.isd) != 0;
      // One straight-line block (variants of it would each need their own
      // register assignment): QK of chunk i+1, computed whether or not a row
      // of the wave uses it, beside the softmax of chunk i (p = 0 in rows
      // that do not use it; masked keys were set to -inf just before).
      if (part0) st.mask_scores(sc, lim0, I0.isd, my_bits);
      float alpha;
      st.template qk<kLookahead>(kfrag_at(lds0 + (1 - S) * TILE), sn);
      const typename RowState<D>::PFrag pf =
          st.template softmax<false>(sc, lim0, false, 0ull, a.scale_log2, alpha);
      sched_qk<2 * (D / 16), kLookahead, kValuPerMfma>();
      (void)use1;
      if (use0) {
        st.rescale(alpha);
        st.template pv<kLookahead>(vfrag_at(lds0 + (2 + S) * TILE), pf);
      }
      (void)u;
      lim0 = lim1;
      use0 = use1;
      I0 = I1;
      I1 = I2;
      I2 = info(u + 3);
    };
    for (int i = 0; i < n; i += 2) {
      iter(i, StageTag<0>(), sA, sB);
      if (i + 1 < n) iter(i + 1, StageTag<1>(), sB, sA);
    }
  } else if constexpr (PF == 3) {
    // Direct staging, two K and two V tiles.  Chunk i is read from K[i&1],
    // V[i&1].  Issue order: K0 V0 K1 | A0 V1 B0 K2 | A1 V2 B1 K3 | ...
    //   barrier A_i (K(i) has landed):  V(i+1) -> V[(i+1)&1], which PV(i-1)
    //                                  finished reading before A_i;
    //   S^T = K Q^T and the softmax of chunk i;
    //   barrier B_i (V(i) has landed):  K(i+2) -> K[i&1], free after QK(i);
    //   O^T += V^T P^T.
    // Every tile thus has about one and a half iterations to arrive.  At A_i
    // the loads issued after K(i) are V(i) and K(i+1) (if it exists); at B_i
    // those after V(i) are K(i+1) and V(i+1) (both exist iff i+1 < n).
    // Q (and the draft mask) must have arrived before the loop: the compiler
    // would otherwise wait for them inside it with vmcnt counts that do not
    // know about the direct loads, i.e. wait for those too.
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    using DT = DmaTile<D, NT>;
    constexpr int TILE = Swz<D>::TILE;
    constexpr int KL = DT::kLoads;
    DT dma;
    dma.init(tid);
    FragAddr<D> fa;
    fa.init(lane);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)stage;
    auto issue_k = [&](int u, int sidx) {
      const UnitInfo ui = unit_info(u);
      dma.issue(lds0 + sidx * TILE, kptr(ui), ui.nv, tid, wave_u);
    };
    auto issue_v = [&](int u, int sidx) {
      const UnitInfo ui = unit_info(u);
      dma.issue(lds0 + (2 + sidx) * TILE, vptr(ui), ui.nv, tid, wave_u);
    };
    const int n = u_end - u_begin;
    if (n > 0) { issue_k(u_begin, 0); issue_v(u_begin, 0); }
    if (n > 1) issue_k(u_begin + 1, 1);
    auto iter = [&](int i, auto stage_tag) {
      constexpr int S = decltype(stage_tag)::value;
      const int u = u_begin + i;
      const bool more = i + 1 < n;
      if (more) wait_vm_barrier<2 * KL>(); else wait_vm_barrier<KL>();
      if (more) issue_v(u + 1, S ^ 1);
      const UnitInfo ui = unit_info(u);
      const uint32_t kb = lds0 + S * TILE, vb = lds0 + (2 + S) * TILE;
      auto kfrag = [&](int kt, int ks) {
        return lds_read16(kb + fa.k(ks) + kt * 32 * Swz<D>::RB);
      };
      auto vfrag = [&](int dt, int kt, int t) {
        const uint32_t off = vb + (32 * kt + 16 * t) * Swz<D>::RB;
        const bf16x4 lo = lds_read_tr8(off + fa.v(dt, 0));
        const bf16x4 hi = lds_read_tr8(off + fa.v(dt, 1));
        return (bf16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      const int lim = chunk_lim(ui);
      const bool use = __ballot(lim >= 0) != 0;
      typename RowState<D>::PFrag pf;
      if (use) pf = st.template scores<kLookahead>(kfrag, lim, ui.isd, my_bits, a.scale_log2);
      if (more) wait_vm_barrier<2 * KL>(); else wait_vm_barrier<0>();
      if (i + 2 < n) issue_k(u + 2, S);
      if (use) st.template pv<kLookahead>(vfrag, pf);
    };
    for (int i = 0; i < n; i += 2) {
      iter(i, StageTag<0>());
      if (i + 1 < n) iter(i + 1, StageTag<1>());
    }
  } else if constexpr (PF == 1) {
    // register prefetch one chunk ahead; store -> barrier -> prefetch -> compute
    Stager<D, NT> sg;
    UnitInfo cur = {0, 0, 0u, false};
    if (u_begin < u_end) {
      cur = unit_info(u_begin);
      sg.load(kptr(cur), vptr(cur), cur.nv, tid);
    }
    for (int u = u_begin; u < u_end; ++u) {
      uint16_t* buf = stage + ((u - u_begin) & 1) * Lds<D>::kStageElems;
      sg.store(buf, tid);
      __syncthreads();
      UnitInfo nxt = cur;
      if (u + 1 < u_end) {
        nxt = unit_info(u + 1);
        sg.load(kptr(nxt), vptr(nxt), nxt.nv, tid);
      }
      compute_chunk(buf, cur);
      cur = nxt;
    }
  } else {
    // two register sets: chunk u+1 is stored while chunk u is multiplied,
    // and the loads of chunk u+3 go out into the set just stored, so every
    // chunk has two iterations to arrive.  Iteration i (u = u_begin + i):
    //   barrier; store set[(i+1)&1] -> stage[(i+1)&1]; load u+3 -> that set;
    //   compute stage[i&1].
    Stager<D, NT> sgA, sgB;
    auto fetch = [&](Stager<D, NT>& sg, int u) {
      if (u < u_end) {
        const UnitInfo ui = unit_info(u);
        sg.load(kptr(ui), vptr(ui), ui.nv, tid);
      }
    };
    fetch(sgA, u_begin);
    fetch(sgB, u_begin + 1);
    if (u_begin < u_end) sgA.store(stage, tid);
    fetch(sgA, u_begin + 2);
    auto iter = [&](int i, Stager<D, NT>& nxt_set) {
      const int u = u_begin + i;
      __syncthreads();
      if (u + 1 < u_end) {
        nxt_set.store(stage + ((i + 1) & 1) * Lds<D>::kStageElems, tid);
        fetch(nxt_set, u + 3);
      }
      compute_chunk(stage + (i & 1) * Lds<D>::kStageElems, unit_info(u));
    };
    const int n = u_end - u_begin;
    for (int i = 0; i < n; i += 2) {
      iter(i, sgB);                       // stores chunk u+1 from set B
      if (i + 1 < n) iter(i + 1, sgA);    // stores chunk u+2 from set A
    }
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = st.l + swap_halves(st.l);
  if constexpr (MODE == kPrefill) {
    if (row_ok) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      uint16_t* orow = a.out + ((int64_t)my_row * a.h_q + my_head) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int d0 = 32 * dt + 8 * qd + 4 * half;
          u32x2 w;
          w.x = pack_bf16x2(st.o[dt][4 * qd + 0] * inv, st.o[dt][4 * qd + 1] * inv);
          w.y = pack_bf16x2(st.o[dt][4 * qd + 2] * inv, st.o[dt][4 * qd + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      if (a.lse && half == 0)
        a.lse[(int64_t)my_row * a.h_q + my_head] = (st.m + __log2f(l_tot)) * kLn2;
    }
  } else {
    if (row_ok) {
      float* part = a.ws + (((int64_t)my_row * a.h_q + my_head) * a.n_split + split) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int d0 = 32 * dt + 8 * qd + 4 * half;
          f32x4 w = {st.o[dt][4 * qd + 0], st.o[dt][4 * qd + 1], st.o[dt][4 * qd + 2],
                     st.o[dt][4 * qd + 3]};
          *reinterpret_cast<f32x4*>(part + d0) = w;
        }
      if (half == 0) {
        part[D] = st.m;
        part[D + 1] = l_tot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill with 16 query rows per wave: one token's 16 heads of a KV group, on
// v_mfma_f32_16x16x32_bf16.  Operand layouts (lane l = j + 16 h):
//   A[i][k]: lane i + 16 (k/8), element k%8     (16 x 32)
//   B[k][j]: lane j + 16 (k/8), element k%8     (32 x 16)
//   D[i][j]: lane j + 16 (i/4), register i%4    (16 x 16, float32)
// As in the 32-row kernel the products are transposed: S^T = K Q^T (A = 16
// keys of K, B = Q^T) and O^T = V^T P^T, so lane (j, h) owns query row j:
// its S^T registers hold keys 16 kt + 4 h + r of key tile kt, and the P^T
// B operand of k-step s is built from its own registers, element e <-> key
// 16 (2 s + e/4) + 4 h + e%4.  V^T fragments come from transposing LDS reads.
// A wave computes exactly the chunks its token kept: a workgroup of 8 waves
// stages the union of its 8 tokens' blocks and each wave skips the others.
// Per-wave state is half that of the 32-row kernel, so four waves share a
// SIMD and hide each other's barrier and staging waits.
// ---------------------------------------------------------------------------

template <int D>
struct Row16 {
  static constexpr int NKS = D / 32;       // QK k-steps of 32 dims
  static constexpr int NDT = D / 16;       // O^T d-tiles of 16
  static constexpr int RB = Swz16<D>::RB;
  static constexpr int CPR_ = D / 8;        // 16-byte chunks per K/V row
  bf16x8 q[NKS];                           // lane (j, h): Q[row j][32 ks + 8 h .. +8]
  f32x4 o[NDT];                            // lane (j, h): O[row j][16 dt + 4 h + r]
  float m, l;
  uint32_t k0, v0;                         // fragment addresses inside a tile
  struct PFrag { bf16x8 f[2]; };

  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    m = kNoMax;
    l = 0.0f;
    const int i = lane & 15, h = lane >> 4;
    // K A operand, key tile kt, k-step ks: row 16 kt + i, logical chunk 4 ks + h
    k0 = (uint32_t)(i * RB + ((h ^ Swz16K<D>::f(i)) * 16));
    // V^T A operand, d-tile dt, k-step s, half c: this lane addresses row
    // 16 (2 s + c) + 4 h + i/4 at d = 16 dt + 4 (i%4) (8 bytes)
    const int row = 4 * h + (i >> 2), qd = i & 3;
    v0 = (uint32_t)(row * RB + (((qd >> 1) ^ Swz16V<D>::f(row)) * 16) + 8 * (qd & 1));
  }
  __device__ __forceinline__ uint32_t kaddr(int kt, int ks) const {
    return (k0 ^ (uint32_t)(64 * ks)) + (uint32_t)(16 * kt * RB);
  }
  __device__ __forceinline__ uint32_t vaddr(int dt, int s, int c) const {
    return (v0 ^ (uint32_t)(32 * dt)) + (uint32_t)(16 * (2 * s + c) * RB);
  }

  // S^T for the 64 keys of the tile at kb: 4 independent accumulation chains
  __device__ __forceinline__ void qk(uint32_t kb, f32x4 (&s)[4]) const {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_read16(kb + kaddr(kt, ks)), q[ks],
                                                        s[kt], 0, 0, 0);
  }

  // keys past `lim` -> -inf (partial chunks); NKT 16-key tiles
  template <int NKT>
  __device__ __forceinline__ void mask(f32x4 (&s)[NKT], int lim) const {
    const int h = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s[kt][r] = 16 * kt + 4 * h + r <= lim ? s[kt][r] : -INFINITY;
  }

  // keys whose bit is clear in `bits` -> -inf (the chunk of draft tokens)
  __device__ __forceinline__ void mask_bits(f32x4 (&s)[4], uint64_t bits) const {
    const int h = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s[kt][r] = ((bits >> (16 * kt + 4 * h + r)) & 1ull) ? s[kt][r] : -INFINITY;
  }

  // online softmax (log2 domain, lazy rescale as in the 32-row kernel); rows
  // with keep == false get p = 0 and leave m, l unchanged.  NKT 16-key tiles
  // (4: a 64-key chunk, 2: a 32-key half) give NKT / 2 B operands.
  template <int NKT>
  struct PFragN { bf16x8 f[NKT / 2]; };
  template <bool SKIP = true>
  __device__ __forceinline__ PFrag softmax(f32x4 (&s)[4], bool keep, float scale_log2) {
    const PFragN<4> r = softmax_n<4, SKIP>(s, keep, scale_log2);
    PFrag pf;
    pf.f[0] = r.f[0];
    pf.f[1] = r.f[1];
    return pf;
  }
  // maximum over a row's four lanes: its other 48 keys sit in lanes j + 16,
  // j + 32, j + 48
  __device__ __forceinline__ static float row_max(float mx) {
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
    mx = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
    return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  }
  template <int NKT>
  __device__ __forceinline__ PFragN<NKT> pack(const f32x4 (&s)[NKT]) const {
    PFragN<NKT> pf;
#pragma unroll
    for (int sidx = 0; sidx < NKT / 2; ++sidx)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.f[sidx][e] = (__bf16)s[2 * sidx + (e >> 2)][e & 3];
    return pf;
  }
  // SKIP: the row maximum is only formed when some lane's own maximum clears
  // the slack.  Otherwise no row's maximum does, so every row keeps m with
  // alpha = 1 and O untouched, exactly what the full step gives, and the
  // cross-lane reduction and the rescale exponential are saved.  That pays
  // on most chunks of the prefill loops; the decode loop, bound by latency,
  // is faster with the straight-line step (SKIP = false).
  template <int NKT, bool SKIP = true>
  __device__ __forceinline__ PFragN<NKT> softmax_n(f32x4 (&s)[NKT], bool keep,
                                                   float scale_log2) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = keep ? mx * scale_log2 : -INFINITY;
    if constexpr (SKIP) {
      float alpha = 1.0f;
      if (__ballot(mx > m + kRescaleSlack)) {
        mx = row_max(mx);
        const float m_new = mx > m + kRescaleSlack ? mx : m;
        alpha = fast_exp2(m - m_new);
        m = m_new;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        }
      }
      const float msub = keep ? m : INFINITY;
      float psum;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kt][r], scale_log2, -msub));
          s[kt][r] = p;
          psum = kt == 0 && r == 0 ? p : psum + p;   // p >= 0: the same sum as from 0
        }
      l = l * alpha + psum;
    } else {
      mx = row_max(mx);
      const float m_new = mx > m + kRescaleSlack ? mx : m;
      const float alpha = fast_exp2(m - m_new);
      const float msub = keep ? m_new : INFINITY;
      float psum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kt][r], scale_log2, -msub));
          s[kt][r] = p;
          psum += p;
        }
      m = m_new;
      l = l * alpha + psum;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      }
    }
    return pack(s);
  }

  // O^T += V^T P^T for the tile at vb; k-step outer, d-tile inner
  __device__ __forceinline__ void pv(uint32_t vb, const PFrag& pf) {
    PFragN<4> r;
    r.f[0] = pf.f[0];
    r.f[1] = pf.f[1];
    pv_n<4>(vb, r);
  }
  template <int NKT>
  __device__ __forceinline__ void pv_n(uint32_t vb, const PFragN<NKT>& pf) {
#pragma unroll
    for (int sidx = 0; sidx < NKT / 2; ++sidx)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x4 lo = lds_read_tr8(vb + vaddr(dt, sidx, 0));
        const bf16x4 hi = lds_read_tr8(vb + vaddr(dt, sidx, 1));
        const bf16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pf.f[sidx], o[dt], 0, 0, 0);
      }
  }
};

// Two tokens in one wave (32 rows): every K and V^T fragment read from LDS
// feeds the MFMA of each of the two tokens' 16-row tiles.
template <int D>
__device__ __forceinline__ void qk_pair(uint32_t kb, const Row16<D>& x, const Row16<D>& y,
                                        f32x4 (&sx)[4], f32x4 (&sy)[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    sx[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    sy[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int ks = 0; ks < Row16<D>::NKS; ++ks)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const bf16x8 kf = lds_read16(kb + x.kaddr(kt, ks));
      sx[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, x.q[ks], sx[kt], 0, 0, 0);
      sy[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, y.q[ks], sy[kt], 0, 0, 0);
    }
}
template <int D>
__device__ __forceinline__ void pv_pair(uint32_t vb, Row16<D>& x,
                                        const typename Row16<D>::PFrag& px, Row16<D>& y,
                                        const typename Row16<D>::PFrag& py) {
#pragma unroll
  for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
    for (int dt = 0; dt < Row16<D>::NDT; ++dt) {
      const bf16x4 lo = lds_read_tr8(vb + x.vaddr(dt, sidx, 0));
      const bf16x4 hi = lds_read_tr8(vb + x.vaddr(dt, sidx, 1));
      const bf16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      x.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, px.f[sidx], x.o[dt], 0, 0, 0);
      y.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, py.f[sidx], y.o[dt], 0, 0, 0);
    }
}

// W waves of TPW tokens each per workgroup, NS staging slots of one K and
// one V tile.  SPLIT (one token per wave): blocks kept by fewer than
// a.ring_min of the tile's tokens go through each token's own pass.
template <int D, int W, int NS, int TPW, bool SPLIT = false>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(TPW == 1 ? 4 : 2)))
void attn16_prefill_kernel(AttnArgs a) {
  constexpr int G = 16, NT = W * 64;
  constexpr int TT = W * TPW;
  static_assert(TPW == 1 || TPW == 2, "tokens per wave");
  static_assert(TT <= 32, "token bitmask is 32 bits");
  constexpr int TILE = Swz16<D>::TILE;
  constexpr int SORT_N = TT * kSortCap;
  constexpr int ECAP = TT * kSortCap;
  __shared__ __attribute__((aligned(16))) uint16_t stage[NS * TILE];   // K[0..NS) V[0..NS)
  __shared__ int2 ents[ECAP];
  __shared__ int scan_lds[NT / 64];
  static_assert(SORT_N * 4 <= (int)sizeof(stage), "sort buffer aliases the staging ring");

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int w = xcd_contiguous_index(blockIdx.x, gridDim.x);
  const int g = w / a.n_tiles, tile = w % a.n_tiles;
  const int n_keys = (int)a.n_k;
  const int tok0 = tile * TT;
  const int n_tok = min(TT, a.n_rows - tok0);
  const bool dense = n_keys < a.dense_len || a.block_idx == nullptr;
  const int n_b = (n_keys + a.B - 1) / a.B;
  const int cpb = (a.B + kChunk - 1) / kChunk;
  const uint32_t full_mask = n_tok >= 32 ? 0xffffffffu : ((1u << n_tok) - 1u);
  const int p0 = (int)a.n_k - a.n_rows + tok0;   // query position of the tile's first token

  // this wave's tokens: TPW consecutive ones (a scalar, so the per-chunk
  // token tests stay on the scalar unit)
  const int my_head = g * G + (lane & 15);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto tok_of = [&](int j) { return wave_u * TPW + j; };

  int n_entries;
  if (dense) {
    n_entries = (p0 + n_tok - 1) / a.B + 1;
  } else {
    int N = 1;
    while (N < TT * a.topk) N <<= 1;
    n_entries = build_union<NT, TT>(a.block_idx, tok0, a.h_kv, g, n_tok, a.topk, n_b,
                                    reinterpret_cast<uint32_t*>(stage), N, ents, scan_lds);
  }
  // Split of the union (one token per wave only): blocks kept by at least
  // ring_min of the tile's tokens stay on the shared ring; each token's
  // other blocks go through its own pass afterwards, with no barrier, so
  // waves that do not keep a block do not wait for it.  A stable partition
  // puts the ring entries first (ascending), then the others (ascending).
  static_assert(!SPLIT || TPW == 1, "the split takes one token per wave");
  const bool split = SPLIT && !dense && a.ring_min > 1;
  int n_ring_e = n_entries;
  if (SPLIT && split) {
    static_assert(ECAP <= 2 * NT, "two entries per thread");
    int2 ev[2];
    int fl[2], base[2], tot[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + k * NT;
      ev[k] = e < n_entries ? ents[e] : make_int2(0, 0);
      fl[k] = e < n_entries && __popc((uint32_t)ev[k].y) >= a.ring_min;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) base[k] = block_excl_scan<NT>(fl[k], &tot[k], scan_lds);
    n_ring_e = tot[0] + tot[1];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + k * NT;
      if (e < n_entries) {
        const int ring_before = (k ? tot[0] : 0) + base[k];   // ring entries before e
        ents[fl[k] ? ring_before : n_ring_e + (e - ring_before)] = ev[k];
      }
    }
    __syncthreads();
  }
  const int n = __builtin_amdgcn_readfirstlane(n_ring_e * cpb);   // same in every lane

  // unit u -> first key, valid keys, mask of the tile's tokens that use it
  struct Unit { int key0, nv; uint32_t tm; };
  auto unit_lane = [&](int u) -> Unit {
    Unit r;
    int e = u, c = 0;
    if (cpb != 1) { e = u / cpb; c = u - e * cpb; }
    int b;
    if (dense) {
      b = e;
      const int t_min = b * a.B - p0;      // token t keeps block b iff t >= b*B - p0
      r.tm = t_min <= 0 ? full_mask : (t_min >= 32 ? 0u : (full_mask & (0xffffffffu << t_min)));
    } else {
      const int2 en = ents[e];
      b = en.x;
      r.tm = (uint32_t)en.y;
    }
    r.key0 = b * a.B + c * kChunk;
    r.nv = max(0, min(kChunk, min((b + 1) * a.B, n_keys) - r.key0));
    return r;
  };
  // metadata of 64 consecutive units, one per lane, read with readlane
  int wb = 0;
  Unit wl = {0, 0, 0u};
  auto load_window = [&]() {
    const int uu = wb + lane;
    if (uu < n) wl = unit_lane(uu); else wl = Unit{0, 0, 0u};
  };
  load_window();
  auto info = [&](int u) -> Unit {
    if (u >= n) return Unit{0, 0, 0u};
    if (u >= wb + 64) {
      wb += 64;
      load_window();
    }
    const int ln = u - wb;
    return Unit{__builtin_amdgcn_readlane(wl.key0, ln), __builtin_amdgcn_readlane(wl.nv, ln),
                (uint32_t)__builtin_amdgcn_readlane((int)wl.tm, ln)};
  };

  const uint16_t* kseq = a.k + (int64_t)g * a.cap * D;
  const uint16_t* vseq = a.v + (int64_t)g * a.cap * D;
  auto kp = [&](const Unit& un) { return kseq + (un.nv > 0 ? (int64_t)un.key0 * D : 0); };
  auto vp = [&](const Unit& un) { return vseq + (un.nv > 0 ? (int64_t)un.key0 * D : 0); };

  Row16<D> st[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    st[j].init(lane);
    const bool ok = tok_of(j) < n_tok;
    const int row = tok0 + (ok ? tok_of(j) : 0);
    const uint16_t* qrow = a.q + ((int64_t)row * a.h_q + my_head) * D + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < Row16<D>::NKS; ++ks) {
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (ok) wv = ldg16(qrow + 32 * ks);
      st[j].q[ks] = *reinterpret_cast<const bf16x8*>(&wv);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);   // Q has arrived before the direct loads start

  using DTK = DmaTile<D, NT, Swz16K<D>>;
  using DTV = DmaTile<D, NT, Swz16V<D>>;
  constexpr int KL = DTK::kLoads;
  static_assert(DTV::kLoads == KL, "K and V copies are the same size");
  static_assert(2 * KL * (NS - 1) <= 63, "vmcnt range");
  DTK dmak;
  DTV dmav;
  dmak.init(tid);
  dmav.init(tid);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)stage;
  // Chunk i sits in slot i % NS: K at lds0 + slot TILE, V at lds0 + (NS + slot) TILE.
  // Iteration i: barrier (chunk i landed, iteration i-1 done everywhere, so
  // slot (i-1) % NS is free), copy chunk i + NS - 1 into it, compute chunk i.
  // At the barrier the copies issued after chunk i's are those of chunks
  // i+1 .. i+NS-2, the ones that exist.
  auto issue = [&](const Unit& un, int slot) {
    dmak.issue(lds0 + slot * TILE, kp(un), un.nv, tid, wave_u);
    dmav.issue(lds0 + (NS + slot) * TILE, vp(un), un.nv, tid, wave_u);
  };
  Unit cur = info(0);
  Unit ahead[NS > 2 ? NS - 2 : 1];       // chunks i+1 .. i+NS-2 (already issued)
#pragma unroll
  for (int j = 0; j + 1 < NS; ++j) {
    const Unit un = j == 0 ? cur : info(j);
    if (j < n) issue(un, j);
    if (j >= 1 && j - 1 < NS - 2) ahead[j - 1] = un;
  }
  auto iter = [&](int i, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    // in flight after chunk i: chunks i+1 .. min(i+NS-2, n-1)
    const int after = min(NS - 2, n - 1 - i);
    if constexpr (NS == 2) {
      wait_vm_barrier<0>();
    } else {
      if (after >= NS - 2) wait_vm_barrier<2 * KL * (NS - 2)>();
      else if (NS > 3 && after >= 1) wait_vm_barrier<2 * KL>();
      else wait_vm_barrier<0>();
    }
    const Unit far = info(i + NS - 1);
    if (i + NS - 1 < n) issue(far, (S + NS - 1) % NS);
    // per token: largest key offset it uses in this chunk, -1 if none (the
    // same in every lane of the wave: scalar branches)
    int lim[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = tok_of(j);
      int l = -1;
      if (t < n_tok && ((cur.tm >> t) & 1u)) l = min(p0 + t - cur.key0, cur.nv - 1);
      lim[j] = __builtin_amdgcn_readfirstlane(l);
    }
    const uint32_t kb = lds0 + S * TILE, vb = lds0 + (NS + S) * TILE;
    auto one = [&](Row16<D>& r, int l) {
      f32x4 sc[4];
      r.qk(kb, sc);
      if (l < kChunk - 1) r.mask(sc, l);
      const typename Row16<D>::PFrag pf = r.softmax(sc, true, a.scale_log2);
      r.pv(vb, pf);
    };
    if constexpr (TPW == 1) {
      if (lim[0] >= 0) one(st[0], lim[0]);
    } else {
      if (lim[0] >= 0 && lim[1] >= 0) {
        f32x4 sx[4], sy[4];
        qk_pair<D>(kb, st[0], st[1], sx, sy);
        if (lim[0] < kChunk - 1) st[0].mask(sx, lim[0]);
        if (lim[1] < kChunk - 1) st[1].mask(sy, lim[1]);
        const typename Row16<D>::PFrag px = st[0].softmax(sx, true, a.scale_log2);
        const typename Row16<D>::PFrag py = st[1].softmax(sy, true, a.scale_log2);
        pv_pair<D>(vb, st[0], px, st[1], py);
      } else if (lim[0] >= 0) {
        one(st[0], lim[0]);
      } else if (lim[1] >= 0) {
        one(st[1], lim[1]);
      }
    }
    if constexpr (NS == 2) {
      cur = far;
    } else {
      cur = ahead[0];
#pragma unroll
      for (int j = 0; j + 1 < NS - 2; ++j) ahead[j] = ahead[j + 1];
      ahead[NS - 3] = far;
    }
  };
  static_assert(NS == 2 || NS == 3, "staging depth");
  if constexpr (NS == 2) {
    for (int i = 0; i < n; i += 2) {
      iter(i, StageTag<0>());
      if (i + 1 < n) iter(i + 1, StageTag<1>());
    }
  } else {
    for (int i = 0; i < n; i += 3) {
      iter(i, StageTag<0>());
      if (i + 1 < n) iter(i + 1, StageTag<1>());
      if (i + 2 < n) iter(i + 2, StageTag<2>());
    }
  }

  // Each token's own pass over its blocks kept by fewer than ring_min of the
  // tile's tokens, 32 keys at a time: K fragments straight from global memory
  // into registers (A operands), V through the wave's own 8 KB of the ring's
  // LDS (swizzled rows for the transposing reads), no barrier.
  if constexpr (SPLIT) {
    if (split) {
      __syncthreads();                       // every wave is done with the ring
      const int t = tok_of(0);
      constexpr int kHalf = 32;
      constexpr int kSlotBytes = kHalf * Row16<D>::RB;
      static_assert(W * kSlotBytes <= NS * 2 * TILE, "per-wave slots fit the ring");
      const uint32_t vslot = lds0 + (uint32_t)(wave_u * kSlotBytes);
      const int i16 = lane & 15, h4 = lane >> 4;
      auto half_pass = [&](int key0, int nv, int lim) {
        // V rows -> LDS: instruction i, lane l -> slot 64 i + l: row r = slot / 16,
        // stored chunk position slot % 16, holding logical chunk pos ^ f(r)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // last half's V reads done
        const uint16_t* vsrc = vseq + (int64_t)key0 * D;
#pragma unroll
        for (int i = 0; i < kSlotBytes / 1024; ++i) {
          const int sl = 64 * i + lane, r = sl / Row16<D>::CPR_, cp = sl % Row16<D>::CPR_;
          const int rr = r < nv ? r : nv - 1;
          lds_dma16(vslot + (uint32_t)(1024 * i), vsrc,
                    (uint32_t)(rr * Row16<D>::RB + ((cp ^ Swz16V<D>::f(r)) * 16)));
        }
        // K fragments (key 16 kt + i16, dims 32 ks + 8 h4), one 16-key tile
        // at a time
        f32x4 sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int row = min(16 * kt + i16, nv - 1);
          const uint16_t* kr = kseq + (int64_t)(key0 + row) * D + 8 * h4;
          bf16x8 kf[Row16<D>::NKS];
#pragma unroll
          for (int ks = 0; ks < Row16<D>::NKS; ++ks) {
            const u32x4 w = ldg16(kr + 32 * ks);
            kf[ks] = *reinterpret_cast<const bf16x8*>(&w);
          }
          sc[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < Row16<D>::NKS; ++ks)
            sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], st[0].q[ks], sc[kt], 0, 0, 0);
        }
        if (lim < kHalf - 1) st[0].mask(sc, lim);
        const auto pf = st[0].template softmax_n<2>(sc, true, a.scale_log2);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this half's V has landed
        st[0].template pv_n<2>(vslot, pf);
      };
      if (t < n_tok) {
        const uint32_t my_bit = 1u << t;
        for (int e0 = n_ring_e; e0 < n_entries; e0 += 64) {
          const int e = e0 + lane;
          const int2 en = e < n_entries ? ents[e] : make_int2(0, 0);
          uint64_t mine = __ballot(((uint32_t)en.y & my_bit) != 0u);
          while (mine) {
            const int ln = (int)__builtin_ctzll(mine);
            mine &= mine - 1;
            const int b = __builtin_amdgcn_readlane(en.x, ln);
            for (int c = 0; c < 2 * cpb; ++c) {
              const int key0 = b * a.B + c * kHalf;
              const int nv = max(0, min(kHalf, min((b + 1) * a.B, n_keys) - key0));
              const int lim = min(p0 + t - key0, nv - 1);
              if (lim >= 0) half_pass(key0, nv, lim);
            }
          }
        }
      }
    }
  }

  // row sum over the four lanes of the row, then normalise and store
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    float lt = st[j].l;
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lt), __float_as_uint(lt),
                                                      false, false);
    lt = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt),
                                                      false, false);
    lt = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    if (tok_of(j) < n_tok) {
      const int row = tok0 + tok_of(j);
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      const int h = lane >> 4;
      uint16_t* orow = a.out + ((int64_t)row * a.h_q + my_head) * D;
#pragma unroll
      for (int dt = 0; dt < Row16<D>::NDT; ++dt) {
        u32x2 wv;
        wv.x = pack_bf16x2(st[j].o[dt][0] * inv, st[j].o[dt][1] * inv);
        wv.y = pack_bf16x2(st[j].o[dt][2] * inv, st[j].o[dt][3] * inv);
        *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * h) = wv;
      }
      if (a.lse && h == 0)
        a.lse[(int64_t)row * a.h_q + my_head] = (st[j].m + __log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode with one wave per (sequence, KV head, split): the decode token's 16
// heads of the group are one 16-row tile of v_mfma_f32_16x16x32_bf16.  The
// wave copies its chunks straight into a two-slot LDS ring, the second copy
// issued before the first chunk is used, so a split's loads overlap each
// other and those of every other split on the GPU.  Writes float32 partials
// (o, m, l) that the combine kernel merges.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

//
// TREE: the rows are the draft tokens of a tree over one shared context cache
// (row = draft, all at context position n_ctx - 1, each with its own kept
// blocks); every row has one more unit after its context units: the chunk of
// draft tokens, of which it sees those set in its ancestor mask (and itself).
//
// KPL > 0: the wave selects its row's kept blocks itself from the block
// scores (the top-k selection of topk_wave.h over rows of up to 64 * KPL
// blocks, the same result as the top-k kernel), every split redundantly, and
// split 0 writes the selection out; the wave's staging LDS holds the
// selection's survivors before the copies start.
template <int D, bool TREE, int KPL = 0>
__global__ __launch_bounds__(64) void attn16_decode_kernel(AttnArgs a) {
  constexpr int NS = 2;
  constexpr int TILE = Swz16<D>::TILE;
  __shared__ __attribute__((aligned(16))) uint16_t stage[NS * TILE];   // K0 K1 V0 V1
  static_assert(KPL == 0 || (kWaveSurvivors + 64) * 8 + kMaxTopk * 4 <= NS * TILE * 2,
                "the selection's staging fits the copy staging");
  const int lane = threadIdx.x;
  const int split = blockIdx.x, g = blockIdx.y, seq = blockIdx.z;    // seq: the row
  // The sequence length, the whole kept-block list (topk <= 128: two entries
  // per lane) and the query are loaded together: the copies then wait for
  // one memory round trip instead of a chain of dependent ones.
  int Lr = (int)a.n_k;
  if constexpr (!TREE) Lr = a.seqlens[seq];
  const int32_t* lst = KPL == 0 && a.block_idx
                           ? a.block_idx + ((int64_t)seq * a.h_kv + g) * a.topk
                           : nullptr;
  int32_t lst0 = -1, lst1 = -1;                 // entries lane and 64 + lane
  if (lst) {
    if (lane < a.topk) lst0 = lst[lane];
    if (64 + lane < a.topk) lst1 = lst[64 + lane];
  }
  const int head = g * 16 + (lane & 15);
  Row16<D> st;
  st.init(lane);
  {
    const uint16_t* qrow = a.q + ((int64_t)seq * a.h_q + head) * D + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < Row16<D>::NKS; ++ks) {
      const u32x4 wv = ldg16(qrow + 32 * ks);
      st.q[ks] = *reinterpret_cast<const bf16x8*>(&wv);
    }
  }
  // lengths outside [1, max_seqlen] are clamped: wrong input, no fault
  const int L = TREE ? Lr : (Lr < 1 ? 1 : (Lr > (int)a.n_k ? (int)a.n_k : Lr));
  const bool dense =
      L < a.dense_len || (KPL > 0 ? a.scores == nullptr : a.block_idx == nullptr);
  const int n_b = (L + a.B - 1) / a.B;
  const int cpb = (a.B + kChunk - 1) / kChunk;
  if constexpr (KPL > 0) {
    int32_t* sel = reinterpret_cast<int32_t*>(stage) + 2 * (kWaveSurvivors + 64);
    if (!dense) {
      wave_select_row<KPL>(a.scores + ((int64_t)seq * a.h_kv + g) * a.nb_cap, a.nb_cap,
                           (L - 1) / a.B, a.topk, a.init, a.local,
                           reinterpret_cast<int2*>(stage), sel, lane);
      __builtin_amdgcn_wave_barrier();
      if (lane < a.topk) lst0 = sel[lane];
      if (64 + lane < a.topk) lst1 = sel[64 + lane];
    }
    if (split == 0) {                 // dense rows: nothing selected
      int32_t* so = a.sel_out + ((int64_t)seq * a.h_kv + g) * a.topk;
      if (lane < a.topk) so[lane] = lst0;
      if (64 + lane < a.topk) so[64 + lane] = lst1;
    }
    // the staging is free for the copies once the list has been read
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  int n_entries = n_b;
  if (!dense) {
    // kept blocks = the leading valid entries of the list
    n_entries = a.topk;
#pragma unroll
    for (int half = 1; half >= 0; --half) {
      const int i = 64 * half + lane;
      const int32_t b = half ? lst1 : lst0;
      const uint64_t bad = __ballot(i < a.topk && !(b >= 0 && b < n_b));
      if (bad) n_entries = 64 * half + (int)__builtin_ctzll(bad);
    }
  }
  const int ctx_units = n_entries * cpb;
  const int units = ctx_units + (TREE ? 1 : 0);          // + the draft chunk
  const int per = (units + a.n_split - 1) / a.n_split;
  const int u_begin = min(units, split * per);
  const int n = min(units, u_begin + per) - u_begin;
  // this split's block ids, one per lane (a split spans at most 64 entries),
  // taken from the loaded list with cross-lane reads
  const int e_base = u_begin / cpb;
  int blk_lane = e_base + lane;
  if (!dense) {
    const int e = e_base + lane;                // < n_entries <= 128 where used
    const int32_t v0 = __shfl(lst0, e & 63, 64), v1 = __shfl(lst1, e & 63, 64);
    blk_lane = e < n_entries ? (e < 64 ? v0 : v1) : 0;
  }
  struct Unit { int key0, nv; };
  auto unit = [&](int u) -> Unit {
    if (TREE && u == ctx_units) return Unit{0, (int)a.n_rows};   // the draft chunk
    int e = u, c = 0;
    if (cpb != 1) { e = u / cpb; c = u - e * cpb; }
    const int b = __builtin_amdgcn_readlane(blk_lane, e - e_base);
    Unit r;
    r.key0 = b * a.B + c * kChunk;
    r.nv = max(0, min(kChunk, min((b + 1) * a.B, L) - r.key0));
    r.key0 = __builtin_amdgcn_readfirstlane(r.key0);
    r.nv = __builtin_amdgcn_readfirstlane(r.nv);
    return r;
  };
  const int64_t kv_off = ((int64_t)(TREE ? 0 : seq) * a.h_kv + g) * a.cap * D;
  const uint16_t* kseq = a.k + kv_off;
  const uint16_t* vseq = a.v + kv_off;
  // the draft chunk is unit ctx_units (its Unit has key0 0, nv = drafts)
  const uint16_t* kdr = TREE ? a.k_draft + (int64_t)g * a.n_rows * D : nullptr;
  const uint16_t* vdr = TREE ? a.v_draft + (int64_t)g * a.n_rows * D : nullptr;
  uint64_t dbits = 0ull;
  if constexpr (TREE) {
    const uint64_t full = a.n_rows >= 64 ? ~0ull : ((1ull << a.n_rows) - 1ull);
    dbits = (a.tree_mask[seq] & full) | (1ull << seq);
  }
  auto kp = [&](const Unit& un, bool isd) {
    return isd ? kdr : kseq + (un.nv > 0 ? (int64_t)un.key0 * D : 0);
  };
  auto vp = [&](const Unit& un, bool isd) {
    return isd ? vdr : vseq + (un.nv > 0 ? (int64_t)un.key0 * D : 0);
  };

  __builtin_amdgcn_s_waitcnt(0x0f70);   // Q has arrived before the direct loads start

  using DTK = DmaTile<D, 64, Swz16K<D>>;
  using DTV = DmaTile<D, 64, Swz16V<D>>;
  constexpr int KL = DTK::kLoads;
  DTK dmak;
  DTV dmav;
  dmak.init(lane);
  dmav.init(lane);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)stage;
  auto is_draft = [&](int u) { return TREE && u == ctx_units; };
  auto issue = [&](const Unit& un, int slot, bool isd) {
    dmak.issue(lds0 + slot * TILE, kp(un, isd), un.nv, lane, 0);
    dmav.issue(lds0 + (NS + slot) * TILE, vp(un, isd), un.nv, lane, 0);
  };
  Unit cur = {0, 0}, nxt = {0, 0};
  if (n > 0) { cur = unit(u_begin); issue(cur, 0, is_draft(u_begin)); }
  if (n > 1) { nxt = unit(u_begin + 1); issue(nxt, 1, is_draft(u_begin + 1)); }
  const int pos = L - 1;
  auto step = [&](int i, auto slot_tag) {
    constexpr int S = decltype(slot_tag)::value;
    // the copy of chunk i+1 (if any) was issued after chunk i's
    if (i + 1 < n) wait_vm<2 * KL>(); else wait_vm<0>();
    const bool isd = is_draft(u_begin + i);
    const int lim = isd ? cur.nv - 1 : min(pos - cur.key0, cur.nv - 1);
    if (lim >= 0) {
      f32x4 sc[4];
      st.qk(lds0 + S * TILE, sc);
      if (isd) st.mask_bits(sc, dbits);
      else if (lim < kChunk - 1) st.mask(sc, lim);
      const typename Row16<D>::PFrag pf = st.template softmax<false>(sc, true, a.scale_log2);
      st.pv(lds0 + (NS + S) * TILE, pf);
    }
    if (i + 2 < n) {
      // slot S is free once this wave's reads of it have returned
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const Unit far = unit(u_begin + i + 2);
      issue(far, S, is_draft(u_begin + i + 2));
      cur = nxt;
      nxt = far;
    } else {
      cur = nxt;
    }
  };
  for (int i = 0; i < n; i += 2) {
    step(i, StageTag<0>());
    if (i + 1 < n) step(i + 1, StageTag<1>());
  }

  // partials: lane (j, h) holds O[row j][16 dt + 4 h + r]; m is per row, l per lane
  float lt = st.l;
  {
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lt), __float_as_uint(lt),
                                                      false, false);
    lt = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt),
                                                      false, false);
    lt = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  }
  const int h = lane >> 4;
  float* part = a.ws + (((int64_t)seq * a.h_q + head) * a.n_split + split) * (D + 2);
#pragma unroll
  for (int dt = 0; dt < Row16<D>::NDT; ++dt)
    *reinterpret_cast<f32x4*>(part + 16 * dt + 4 * h) = st.o[dt];
  if (h == 0) {
    part[D] = st.m;
    part[D + 1] = lt;
  }
}

// ---------------------------------------------------------------------------
// Tree planner: union of the drafts' kept blocks per KV head (sorted, with the
// bitmask of drafts that kept each block).  One workgroup per KV head.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 512;
__global__ __launch_bounds__(kPlanThreads) void tree_union_kernel(
    const int32_t* block_idx, int n_draft, int h_kv, int topk, int64_t n_b, int32_t* ublk,
    uint64_t* umask, int32_t* ulen, int union_cap) {
  __shared__ uint32_t buf[64 * kSortCap];
  __shared__ int scan_lds[kPlanThreads / 64];
  const int g = blockIdx.x;
  int N = 1;
  while (N < n_draft * topk) N <<= 1;
  if (N < kPlanThreads) N = kPlanThreads;
  for (int i = threadIdx.x; i < N; i += kPlanThreads) {
    uint32_t key = 0xffffffffu;
    if (i < n_draft * topk) {
      const int t = i / topk, j = i % topk;
      const int32_t b = block_idx[((int64_t)t * h_kv + g) * topk + j];
      if (b >= 0 && b < n_b) key = ((uint32_t)b << 6) | (uint32_t)t;
    }
    buf[i] = key;
  }
  __syncthreads();
  bitonic_sort<kPlanThreads>(buf, N);
  const int C = N / kPlanThreads;
  const int c0 = threadIdx.x * C;
  int heads = 0;
  for (int i = c0; i < c0 + C; ++i) {
    const uint32_t key = buf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (buf[i - 1] >> 6) != (key >> 6)) ++heads;
  }
  int total;
  int slot = block_excl_scan<kPlanThreads>(heads, &total, scan_lds);
  for (int i = c0; i < c0 + C; ++i) {
    const uint32_t key = buf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (buf[i - 1] >> 6) != (key >> 6)) {
      uint64_t msk = 0;
      for (int i2 = i; i2 < N && buf[i2] != 0xffffffffu && (buf[i2] >> 6) == (key >> 6); ++i2)
        msk |= 1ull << (buf[i2] & 63u);
      if (slot < union_cap) {
        ublk[(int64_t)g * union_cap + slot] = (int32_t)(key >> 6);
        umask[(int64_t)g * union_cap + slot] = msk;
      }
      ++slot;
    }
  }
  if (threadIdx.x == 0) ulen[g] = total < union_cap ? total : union_cap;
}

// Same result for contexts of at most kUnionBitmapBlocks blocks, without a
// sort: every draft ORs its bit into a per-block 64-bit mask in LDS, then one
// scan over the blocks compacts the non-zero ones in ascending order.
constexpr int kUnionBitmapBlocks = 8192;      // 64 KB of masks
__global__ __launch_bounds__(kPlanThreads) void tree_union_bitmap_kernel(
    const int32_t* block_idx, int n_draft, int h_kv, int topk, int n_b, int32_t* ublk,
    uint64_t* umask, int32_t* ulen, int union_cap) {
  __shared__ uint64_t mask[kUnionBitmapBlocks];
  __shared__ int scan_lds[kPlanThreads / 64];
  const int g = blockIdx.x;
  for (int b = threadIdx.x; b < n_b; b += kPlanThreads) mask[b] = 0ull;
  __syncthreads();
  for (int i = threadIdx.x; i < n_draft * topk; i += kPlanThreads) {
    const int t = i / topk, j = i % topk;
    const int32_t b = block_idx[((int64_t)t * h_kv + g) * topk + j];
    if (b >= 0 && b < n_b) atomicOr((unsigned long long*)&mask[b], 1ull << t);
  }
  __syncthreads();
  // thread k owns blocks [k*C, (k+1)*C): count, scan, write in order
  const int C = (n_b + kPlanThreads - 1) / kPlanThreads;
  const int b0 = threadIdx.x * C, b1 = min(n_b, b0 + C);
  int cnt = 0;
  for (int b = b0; b < b1; ++b) cnt += mask[b] != 0ull;
  int total;
  int slot = block_excl_scan<kPlanThreads>(cnt, &total, scan_lds);
  for (int b = b0; b < b1; ++b) {
    const uint64_t m = mask[b];
    if (m != 0ull) {
      if (slot < union_cap) {
        ublk[(int64_t)g * union_cap + slot] = b;
        umask[(int64_t)g * union_cap + slot] = m;
      }
      ++slot;
    }
  }
  if (threadIdx.x == 0) ulen[g] = total < union_cap ? total : union_cap;
}

// ---------------------------------------------------------------------------
// Merge of split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// ---------------------------------------------------------------------------
template <int D, typename TOut>
__global__ __launch_bounds__(64) void combine_kernel(const float* ws, int n_split, TOut* out,
                                                     float* lse) {
  constexpr int kMaxSplit = 64;
  constexpr int kBatch = 32;                 // splits whose o values are loaded together
  const int rh = blockIdx.x;   // row * h_q + head
  const int lane = threadIdx.x;
  const float* base = ws + (int64_t)rh * n_split * (D + 2);
  // lane s holds split s (n_split <= 64) for the weights; every lane holds
  // d = lane + 64 i of each split for the sums.  The o loads of a batch of
  // splits are issued together with the (m, l) loads, so the merge waits for
  // memory about once per kBatch splits instead of once per split.
  float m = kNoMax, l = 0.0f;
  if (lane < n_split) {
    l = base[lane * (D + 2) + D + 1];
    m = base[lane * (D + 2) + D];
  }
  float acc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.0f;
  float ov[kBatch][D / 64];
  const int nb0 = n_split < kBatch ? n_split : kBatch;
#pragma unroll
  for (int s2 = 0; s2 < kBatch; ++s2)
#pragma unroll
    for (int i = 0; i < D / 64; ++i)
      ov[s2][i] = s2 < nb0 ? base[s2 * (D + 2) + lane + 64 * i] : 0.0f;
  m = l > 0.0f ? m : kNoMax;
  const float M = wave_max(m);
  const float w = l > 0.0f ? fast_exp2(m - M) : 0.0f;
  const float L = wave_sum(w * l);
  for (int sb = 0; sb < n_split; sb += kBatch) {
    if (sb > 0) {
#pragma unroll
      for (int s2 = 0; s2 < kBatch; ++s2)
#pragma unroll
        for (int i = 0; i < D / 64; ++i)
          ov[s2][i] = sb + s2 < n_split ? base[(sb + s2) * (D + 2) + lane + 64 * i] : 0.0f;
    }
#pragma unroll
    for (int s2 = 0; s2 < kBatch; ++s2) {
      const int sp = sb + s2 < kMaxSplit ? sb + s2 : kMaxSplit - 1;
      // weight of split sp (0 for splits past n_split: lanes >= n_split hold w = 0)
      const float ww = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sp));
#pragma unroll
      for (int i = 0; i < D / 64; ++i) acc[i] = __builtin_fmaf(ww, ov[s2][i], acc[i]);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
    Elem<TOut>::store(out + (int64_t)rh * D + lane + 64 * i, acc[i] * inv);
  if (lse && lane == 0) lse[rh] = (M + __log2f(L)) * kLn2;
}

}  // namespace infllmv2

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
using namespace infllmv2;

namespace {

// Splits per (row, KV head): enough workgroups to cover the GPU for batched
// decode and tree verification while keeping the float32 partials small.
// Decode aims at kDecodeWaves single-wave workgroups in all (at most two per
// CU, as the 64 KB staging ring allows): a larger batch gets fewer splits, so
// each wave streams more chunks through its ring and the combine merges fewer
// partials.  With the selection inside each wave, 256 beat 512 on a ragged
// batch of 8 up to 128K (44.6 -> 42.4 us per step) and tied at batch 1 and
// batch 32.  Tree verification keeps one round of kTreeWaves (16 drafts at
// 128K: 51.2 us against 55.4 us at 256).
constexpr int kMaxDecodeSplits = 32;
constexpr int kDecodeWaves = 256;
constexpr int kTreeWaves = 512;
constexpr int kMaxTreeSplits = 32;
constexpr int kMaxCombineSplits = 64;      // lanes of the combine kernel

template <int D, int G, int W, int MODE, int PF = 1>
int launch_attn(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, G, W, MODE, PF>), grid, dim3(W * 64), 0, st, a);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

// 16-head groups: kRows16Tpw tokens per wave, INFLLMV2_ROWS16_WAVES tokens
// per workgroup.
#ifndef INFLLMV2_ROWS16_WAVES
#define INFLLMV2_ROWS16_WAVES 8
#endif
#ifndef INFLLMV2_ROWS16_STAGES
#define INFLLMV2_ROWS16_STAGES 2
#endif
#ifndef INFLLMV2_ROWS16_TPW
#define INFLLMV2_ROWS16_TPW 1
#endif
constexpr int kRows16Tpw = INFLLMV2_ROWS16_TPW;      // tokens per wave
constexpr int kRows16Waves = INFLLMV2_ROWS16_WAVES / kRows16Tpw;
constexpr int kRows16Stages = INFLLMV2_ROWS16_STAGES;

// Prefill uses W = min(4, G) waves (TT = 32/G * W <= 32 tokens per tile).
template <int D>
int dispatch_prefill(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
#ifndef INFLLMV2_PREFILL_PF
#define INFLLMV2_PREFILL_PF 4
#endif
  constexpr int PF = INFLLMV2_PREFILL_PF;
  if (G == 16) {
    if (kRows16Tpw == 1 && a.ring_min > 1)
      hipLaunchKernelGGL((attn16_prefill_kernel<D, kRows16Waves, kRows16Stages, 1, true>),
                         grid, dim3(kRows16Waves * 64), 0, st, a);
    else
      hipLaunchKernelGGL((attn16_prefill_kernel<D, kRows16Waves, kRows16Stages, kRows16Tpw>),
                         grid, dim3(kRows16Waves * 64), 0, st, a);
    return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
  }
  switch (G) {
    case 1:  return launch_attn<D, 1, 1, kPrefill, PF>(a, grid, st);
    case 2:  return launch_attn<D, 2, 2, kPrefill, PF>(a, grid, st);
    case 4:  return launch_attn<D, 4, 4, kPrefill, PF>(a, grid, st);
    case 8:  return launch_attn<D, 8, 4, kPrefill, PF>(a, grid, st);
    case 16: return launch_attn<D, 16, 4, kPrefill, PF>(a, grid, st);
    case 32: return launch_attn<D, 32, 4, kPrefill, PF>(a, grid, st);
  }
  return INFLLMV2_ERR_UNSUPPORTED;
}

// tokens per prefill tile for a group size (must match dispatch_group)
int prefill_tile_tokens(int G) {
  switch (G) {
    case 1: return 32;
    case 2: return 32;
    case 4: return 32;
    case 8: return 16;
    case 16: return kRows16Waves * kRows16Tpw;
    case 32: return 4;
  }
  return 0;
}

// Tree verification uses all drafts in one tile when they fit: W = 8 waves.
template <int D>
int dispatch_tree(int G, const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1:  return launch_attn<D, 1, 1, kTree>(a, grid, st);
    case 2:  return launch_attn<D, 2, 2, kTree>(a, grid, st);
    case 4:  return launch_attn<D, 4, 4, kTree>(a, grid, st);
    case 8:  return launch_attn<D, 8, 8, kTree>(a, grid, st);
    case 16: return launch_attn<D, 16, 8, kTree>(a, grid, st);
    case 32: return launch_attn<D, 32, 8, kTree>(a, grid, st);
  }
  return INFLLMV2_ERR_UNSUPPORTED;
}
int tree_tile_tokens(int G) {
  switch (G) {
    case 1: return 32;
    case 2: return 32;
    case 4: return 32;
    case 8: return 32;
    case 16: return 16;
    case 32: return 8;
  }
  return 0;
}

// 16-head groups: kpl 0 takes the kept-block lists, 16 / 32 / 64 selects in
// the kernel from the block scores
template <int D, bool TREE>
int launch_decode16(int kpl, const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (kpl) {
    case 0: hipLaunchKernelGGL((attn16_decode_kernel<D, TREE, 0>), grid, dim3(64), 0, st, a);
      break;
    case 16: hipLaunchKernelGGL((attn16_decode_kernel<D, TREE, 16>), grid, dim3(64), 0, st, a);
      break;
    case 32: hipLaunchKernelGGL((attn16_decode_kernel<D, TREE, 32>), grid, dim3(64), 0, st, a);
      break;
    case 64: hipLaunchKernelGGL((attn16_decode_kernel<D, TREE, 64>), grid, dim3(64), 0, st, a);
      break;
    default: return INFLLMV2_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

template <int D>
int dispatch_decode(int G, const AttnArgs& a, dim3 grid, hipStream_t st, int kpl) {
  if (G == 16) return launch_decode16<D, false>(kpl, a, grid, st);
  if (kpl != 0) return INFLLMV2_ERR_UNSUPPORTED;
  switch (G) {
    case 1:  return launch_attn<D, 1, 4, kDecode>(a, grid, st);
    case 2:  return launch_attn<D, 2, 4, kDecode>(a, grid, st);
    case 4:  return launch_attn<D, 4, 4, kDecode>(a, grid, st);
    case 8:  return launch_attn<D, 8, 4, kDecode>(a, grid, st);
    case 16: return launch_attn<D, 16, 4, kDecode>(a, grid, st);
    case 32: return launch_attn<D, 32, 4, kDecode>(a, grid, st);
  }
  return INFLLMV2_ERR_UNSUPPORTED;
}

}  // namespace

namespace infllmv2 {

// Largest number of entries (kept blocks or all blocks) one decode row walks.
int64_t decode_max_entries(int64_t max_seqlen, const Resolved& r) {
  if (max_seqlen < r.dense_len) return ceil_div(max_seqlen, r.B);
  const int64_t dense_max = ceil_div(r.dense_len > 1 ? r.dense_len - 1 : 1, r.B);
  return r.topk > dense_max ? r.topk : dense_max;
}

// Split count for `units` 64-key units: at most `max_default` splits, but
// enough that one split's entries fit the kernel's LDS list.  Callers reject
// counts above kMaxCombineSplits.
int64_t split_count(int64_t units, int64_t cpb, int64_t max_default) {
  int64_t n = units < max_default ? units : max_default;
  const int64_t need = ceil_div(units, (int64_t)(kSplitEntryCap - 1) * cpb);
  return n < need ? need : (n < 1 ? 1 : n);
}

int64_t decode_splits(int batch, int h_kv, int64_t max_seqlen, const Resolved& r) {
  const int64_t cpb = ceil_div(r.B, kChunk);
  const int64_t units = (int64_t)(batch > 0 ? batch : 1) * (h_kv > 0 ? h_kv : 1);
  int64_t cap = ceil_div((int64_t)kDecodeWaves, units);
  if (cap > kMaxDecodeSplits) cap = kMaxDecodeSplits;
  return split_count(decode_max_entries(max_seqlen, r) * cpb, cpb, cap);
}

int64_t tree_union_cap(int n_draft, int64_t n_ctx, const Resolved& r) {
  const int64_t n_b = ceil_div(n_ctx, r.B);
  const int64_t u = (int64_t)n_draft * r.topk;
  return u < n_b ? u : n_b;
}

int64_t tree_splits(int n_draft, int64_t n_ctx, const Resolved& r) {
  const int64_t n_b = ceil_div(n_ctx, r.B);
  const int64_t entries = n_ctx < r.dense_len ? n_b : tree_union_cap(n_draft, n_ctx, r);
  // + 1 entry's worth for the chunk of draft tokens
  const int64_t cpb = ceil_div(r.B, kChunk);
  const int64_t units = entries * cpb + 1;
  return split_count(units, cpb, kMaxTreeSplits);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t partial_bytes(int rows, int h_q, int d, int64_t n_split) {
  return align256((size_t)rows * h_q * n_split * (d + 2) * sizeof(float));
}

size_t decode_workspace_bytes(int batch, int h_q, int h_kv, int d, int64_t max_seqlen,
                              const Resolved& r);

}  // namespace infllmv2

static int common_attn_checks(int dtype, int h_q, int h_kv, int d) {
  if (!dtype_ok(dtype)) return INFLLMV2_ERR_INVALID_ARG;
  INFLLMV2_TRY(check_heads(h_q, h_kv));
  if (!head_dim_ok(d)) return INFLLMV2_ERR_UNSUPPORTED;
  return INFLLMV2_OK;
}


extern "C" int infllmv2_sparse_attn_prefill(int dtype, const void* q, int32_t n_q,
                                            const void* k, const void* v, int64_t cap,
                                            int64_t n_k, int32_t h_q, int32_t h_kv, int32_t d,
                                            const int32_t* block_idx, void* out, float* lse,
                                            const infllmv2_params* p, void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if (!q || !k || !v || !out) return INFLLMV2_ERR_INVALID_ARG;
  if (n_q < 0 || n_k <= 0 || cap < n_k || n_q > n_k) return INFLLMV2_ERR_INVALID_ARG;
  if (cap > INT32_MAX) return INFLLMV2_ERR_UNSUPPORTED;
  const bool dense = n_k < r.dense_len;
  if (!dense && !block_idx) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_q == 0) return INFLLMV2_OK;
  AttnArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.block_idx = dense ? nullptr : block_idx;
  a.out = (uint16_t*)out; a.lse = lse;
  a.cap = cap; a.n_k = n_k; a.n_rows = n_q; a.h_q = h_q; a.h_kv = h_kv; a.topk = r.topk;
  a.B = r.B; a.dense_len = r.dense_len; a.scale_log2 = r.scale * kLog2e;
  // Small top-k (the 128-token-block top-6 variant): most of a tile's union
  // is kept by one or two of its tokens, and those blocks go through each
  // token's own pass (attention 0.310 -> 0.273 ms on the 128K chunk, 8-token
  // tiles).  At top-64 the union is 1.6x a token's own list but the own
  // pass, whose loads are not prefetched, costs ~3x the shared ring per
  // block, so every block stays on the ring.
  a.ring_min = r.topk <= 16 ? 3 : 0;
  hipStream_t st = (hipStream_t)stream;
#ifdef INFLLMV2_DEBUG
  if (!dense) INFLLMV2_TRY(debug_check_rows(block_idx, n_q, h_kv, r, n_k, n_q, nullptr, 0, st));
#endif
  if (dtype == INFLLMV2_F32) return prefill_f32(a, d, st);
  const int G = h_q / h_kv;
  if (!group_ok_for_mfma(G)) return INFLLMV2_ERR_UNSUPPORTED;
  const int TT = prefill_tile_tokens(G);
  a.n_tiles = (int)ceil_div(n_q, TT);
  const int64_t nblocks = (int64_t)a.n_tiles * h_kv;
  if (nblocks >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
  dim3 grid((unsigned)nblocks);
  return d == 128 ? dispatch_prefill<128>(G, a, grid, st) : dispatch_prefill<64>(G, a, grid, st);
}

namespace {

// The selection a decode or tree call makes itself from block scores.
struct SelectIn {
  const float* scores;        // [rows][h_kv][nb_cap]
  int64_t nb_cap;
  int32_t* out;               // [rows][h_kv][topk]
};

// Rows of up to 64 * KPL blocks select inside the 16-head kernels; 0: longer.
int select_kpl(int64_t n_blocks) {
  return n_blocks <= 64 * 16 ? 16 : n_blocks <= 64 * 32 ? 32 : n_blocks <= 64 * 64 ? 64 : 0;
}

// Decode with kept-block lists (sel NULL) or with its own selection from
// block scores (sel set): inside the 16-head kernel when the rows fit it,
// else by the top-k kernel into sel->out first.
int decode_call(int dtype, const void* q, int32_t batch, const void* k, const void* v,
                int64_t cap, const int32_t* seqlens, int32_t max_seqlen, int32_t h_q,
                int32_t h_kv, int32_t d, const int32_t* block_idx, const SelectIn* sel,
                void* out, float* lse, void* ws, size_t ws_bytes, const Resolved& r,
                hipStream_t st) {
  if (!q || !k || !v || !out || !seqlens) return INFLLMV2_ERR_INVALID_ARG;
  if (batch < 0 || max_seqlen <= 0 || cap < max_seqlen) return INFLLMV2_ERR_INVALID_ARG;
  if (cap > INT32_MAX) return INFLLMV2_ERR_UNSUPPORTED;
  const bool sparse = max_seqlen >= r.dense_len;
  const int64_t n_blocks = ceil_div((int64_t)max_seqlen, (int64_t)r.B);
  const bool lists_ok =
      sel ? sel->scores && sel->out && sel->nb_cap >= n_blocks : block_idx != nullptr;
  if (sparse && !lists_ok) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return INFLLMV2_ERR_INVALID_ARG;
  if (batch == 0) return INFLLMV2_OK;
  if (sel && (int64_t)batch * h_kv >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
  const int64_t n_split = decode_splits(batch, h_kv, max_seqlen, r);
  if (n_split > kMaxCombineSplits) return INFLLMV2_ERR_UNSUPPORTED;
  const size_t need = decode_workspace_bytes(batch, h_q, h_kv, d, max_seqlen, r);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return INFLLMV2_ERR_WORKSPACE;
  const int G = h_q / h_kv;
  if (dtype != INFLLMV2_F32 && !group_ok_for_mfma(G)) return INFLLMV2_ERR_UNSUPPORTED;
  const int kpl = sel && sparse && dtype != INFLLMV2_F32 && G == 16 ? select_kpl(n_blocks) : 0;
  if (sel && sparse && kpl == 0) {
    // the top-k kernel writes the lists the attention then reads
    TopkArgs t = {};
    t.scores = sel->scores; t.row_is_seq = 1; t.seqlens = seqlens; t.block_idx = sel->out;
    t.nb_cap = sel->nb_cap; t.h_kv = h_kv; t.B = r.B; t.topk = r.topk; t.init = r.init;
    t.local = r.local; t.dense_len = r.dense_len; t.batch = batch;
    INFLLMV2_TRY(launch_select_topk(t, batch, st));
    block_idx = sel->out;
  }
  AttnArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.block_idx = kpl ? nullptr : (sparse ? block_idx : nullptr); a.seqlens = seqlens;
  a.out = (uint16_t*)out; a.lse = lse; a.ws = (float*)ws;
  a.cap = cap; a.n_k = max_seqlen; a.n_rows = batch; a.h_q = h_q; a.h_kv = h_kv;
  a.topk = r.topk; a.B = r.B; a.dense_len = r.dense_len; a.scale_log2 = r.scale * kLog2e;
  a.n_split = (int)n_split;
  if (kpl) {
    a.scores = sel->scores; a.nb_cap = sel->nb_cap; a.sel_out = sel->out;
    a.init = r.init; a.local = r.local;
  }
#ifdef INFLLMV2_DEBUG
  if (sparse && !kpl)
    INFLLMV2_TRY(debug_check_rows(block_idx, batch, h_kv, r, max_seqlen, 0, seqlens, 1, st));
#endif
  if (dtype == INFLLMV2_F32) return decode_f32(a, d, st);
  dim3 grid((unsigned)n_split, h_kv, batch);
  INFLLMV2_TRY(d == 128 ? dispatch_decode<128>(G, a, grid, st, kpl)
                        : dispatch_decode<64>(G, a, grid, st, kpl));
  if (d == 128)
    hipLaunchKernelGGL((combine_kernel<128, uint16_t>), dim3(batch * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL((combine_kernel<64, uint16_t>), dim3(batch * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

}  // namespace

extern "C" int infllmv2_sparse_attn_decode(int dtype, const void* q, int32_t batch,
                                           const void* k, const void* v, int64_t cap,
                                           const int32_t* seqlens, int32_t max_seqlen,
                                           int32_t h_q, int32_t h_kv, int32_t d,
                                           const int32_t* block_idx, void* out, float* lse,
                                           void* ws, size_t ws_bytes,
                                           const infllmv2_params* p, void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  return decode_call(dtype, q, batch, k, v, cap, seqlens, max_seqlen, h_q, h_kv, d, block_idx,
                     nullptr, out, lse, ws, ws_bytes, r, (hipStream_t)stream);
}

extern "C" int infllmv2_sparse_attn_decode_topk(int dtype, const void* q, int32_t batch,
                                                const void* k, const void* v, int64_t cap,
                                                const int32_t* seqlens, int32_t max_seqlen,
                                                int32_t h_q, int32_t h_kv, int32_t d,
                                                const float* scores, int64_t nb_cap,
                                                int32_t* block_idx, void* out, float* lse,
                                                void* ws, size_t ws_bytes,
                                                const infllmv2_params* p, void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  const SelectIn sel = {scores, nb_cap, block_idx};
  return decode_call(dtype, q, batch, k, v, cap, seqlens, max_seqlen, h_q, h_kv, d, nullptr,
                     &sel, out, lse, ws, ws_bytes, r, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate: the
// split partials live in a fixed device array of this library, one copy per
// GPU, held until the process ends.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[INFLLMV2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];       // device address of `scratch`, per device

// The array's device address on the current device, looked up once per
// device.  In host code `scratch` names a host-side stand-in, so only this
// address may be handed to kernels.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return INFLLMV2_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return INFLLMV2_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return INFLLMV2_OK;
}
}  // namespace

extern "C" int infllmv2_sparse_attn_decode_noalloc(int dtype, const void* q, int32_t batch,
                                                   const void* k, const void* v, int64_t cap,
                                                   const int32_t* seqlens, int32_t max_seqlen,
                                                   int32_t h_q, int32_t h_kv, int32_t d,
                                                   const int32_t* block_idx, void* out,
                                                   float* lse, const infllmv2_params* p,
                                                   void* stream) {
  // the size check needs valid sizes: the decode call's own checks run first
  // on everything but the workspace
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if (batch < 0 || max_seqlen <= 0) return INFLLMV2_ERR_INVALID_ARG;
  const size_t need = decode_workspace_bytes(batch, h_q, h_kv, d, max_seqlen, r);
  if (need > (size_t)INFLLMV2_NOALLOC_SCRATCH_BYTES) return INFLLMV2_ERR_WORKSPACE;
  void* ws = nullptr;
  INFLLMV2_TRY(scratch_address(&ws));
  return infllmv2_sparse_attn_decode(dtype, q, batch, k, v, cap, seqlens, max_seqlen, h_q,
                                     h_kv, d, block_idx, out, lse, ws,
                                     (size_t)INFLLMV2_NOALLOC_SCRATCH_BYTES, p, stream);
}

namespace infllmv2 {
size_t tree_workspace_bytes(int n_draft, int h_q, int h_kv, int d, int64_t n_ctx,
                            const Resolved& r) {
  const int64_t ucap = tree_union_cap(n_draft, n_ctx, r);
  return partial_bytes(n_draft, h_q, d, tree_splits(n_draft, n_ctx, r)) +
         align256((size_t)h_kv * ucap * 4) + align256((size_t)h_kv * ucap * 8) +
         align256((size_t)h_kv * 4);
}
size_t decode_workspace_bytes(int batch, int h_q, int h_kv, int d, int64_t max_seqlen,
                              const Resolved& r) {
  return partial_bytes(batch, h_q, d, decode_splits(batch, h_kv, max_seqlen, r));
}
}  // namespace infllmv2

namespace {

// Tree verification with kept-block lists (sel NULL) or with its own
// selection from block scores (as decode_call).
int tree_call(int dtype, const void* q, int32_t n_draft, const void* k, const void* v,
              int64_t cap, int64_t n_ctx, const void* k_draft, const void* v_draft,
              const uint64_t* tree_mask, int32_t h_q, int32_t h_kv, int32_t d,
              const int32_t* block_idx, const SelectIn* sel, void* out, float* lse, void* ws,
              size_t ws_bytes, const Resolved& r, hipStream_t st) {
  if (!q || !k || !v || !k_draft || !v_draft || !tree_mask || !out)
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_draft < 0 || n_draft > 64 || n_ctx <= 0 || cap < n_ctx) return INFLLMV2_ERR_INVALID_ARG;
  if (cap > INT32_MAX) return INFLLMV2_ERR_UNSUPPORTED;
  const bool dense = n_ctx < r.dense_len;
  const int64_t n_b = ceil_div(n_ctx, r.B);
  const bool lists_ok = sel ? sel->scores && sel->out && sel->nb_cap >= n_b : block_idx != nullptr;
  if (!dense && !lists_ok) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(k_draft) || !aligned16(v_draft))
    return INFLLMV2_ERR_INVALID_ARG;
  if (n_draft == 0) return INFLLMV2_OK;
  const int64_t n_split = tree_splits(n_draft, n_ctx, r);
  if (n_split > kMaxCombineSplits) return INFLLMV2_ERR_UNSUPPORTED;
  const size_t need = tree_workspace_bytes(n_draft, h_q, h_kv, d, n_ctx, r);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return INFLLMV2_ERR_WORKSPACE;
  const int G = h_q / h_kv;
  if (dtype != INFLLMV2_F32 && !group_ok_for_mfma(G)) return INFLLMV2_ERR_UNSUPPORTED;
  const int kpl = sel && !dense && dtype != INFLLMV2_F32 && G == 16 ? select_kpl(n_b) : 0;
  if (sel && !dense && kpl == 0) {
    // the top-k kernel writes the lists the attention then reads: every
    // draft is a row at the context's last position
    TopkArgs t = {};
    t.scores = sel->scores; t.fixed_len = n_ctx; t.block_idx = sel->out;
    t.nb_cap = sel->nb_cap; t.h_kv = h_kv; t.B = r.B; t.topk = r.topk; t.init = r.init;
    t.local = r.local; t.dense_len = r.dense_len; t.batch = 1;
    INFLLMV2_TRY(launch_select_topk(t, n_draft, st));
    block_idx = sel->out;
  }
  const int64_t ucap = tree_union_cap(n_draft, n_ctx, r);
  AttnArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.block_idx = dense || kpl ? nullptr : block_idx;
  a.k_draft = (const uint16_t*)k_draft; a.v_draft = (const uint16_t*)v_draft;
  a.tree_mask = tree_mask;
  a.out = (uint16_t*)out; a.lse = lse; a.ws = (float*)ws;
  char* tail = (char*)ws + partial_bytes(n_draft, h_q, d, n_split);
  a.union_blk = (const int32_t*)tail;
  a.union_mask = (const uint64_t*)(tail + align256((size_t)h_kv * ucap * 4));
  a.union_len = (const int32_t*)(tail + align256((size_t)h_kv * ucap * 4) +
                                 align256((size_t)h_kv * ucap * 8));
  a.union_cap = (int)ucap;
  a.cap = cap; a.n_k = n_ctx; a.n_rows = n_draft; a.h_q = h_q; a.h_kv = h_kv;
  a.topk = r.topk; a.B = r.B; a.dense_len = r.dense_len; a.scale_log2 = r.scale * kLog2e;
  a.n_split = (int)n_split;
  if (kpl) {
    a.scores = sel->scores; a.nb_cap = sel->nb_cap; a.sel_out = sel->out;
    a.init = r.init; a.local = r.local;
  }
#ifdef INFLLMV2_DEBUG
  INFLLMV2_TRY(debug_check_masks(tree_mask, n_draft, st));
  if (!dense && !kpl)
    INFLLMV2_TRY(debug_check_rows(block_idx, n_draft, h_kv, r, n_ctx, 0, nullptr, 2, st));
#endif
  if (dtype == INFLLMV2_F32) return tree_f32(a, d, st);
  if (G == 16) {
    // 16-head groups: each draft is a row of the decode kernel over the
    // shared context (its own kept blocks, then the draft chunk); splits as
    // for decode (one resident round of waves), within the workspace's count
    const int64_t cpb = ceil_div(r.B, kChunk);
    const int64_t row_units = (dense ? n_b : r.topk) * cpb + 1;
    int64_t ns = ceil_div((int64_t)kTreeWaves, (int64_t)n_draft * h_kv);
    ns = std::min<int64_t>(ns, n_split);
    ns = std::max<int64_t>(ns, ceil_div(row_units, (int64_t)(kSplitEntryCap - 1) * cpb));
    if (ns > n_split) return INFLLMV2_ERR_UNSUPPORTED;     // cannot happen: see tree_splits
    a.n_split = (int)ns;
    dim3 grid16((unsigned)ns, h_kv, (unsigned)n_draft);
    INFLLMV2_TRY((d == 128 ? launch_decode16<128, true>(kpl, a, grid16, st)
                           : launch_decode16<64, true>(kpl, a, grid16, st)));
    if (d == 128)
      hipLaunchKernelGGL((combine_kernel<128, uint16_t>), dim3(n_draft * h_q), dim3(64), 0, st,
                         a.ws, a.n_split, (uint16_t*)out, lse);
    else
      hipLaunchKernelGGL((combine_kernel<64, uint16_t>), dim3(n_draft * h_q), dim3(64), 0, st,
                         a.ws, a.n_split, (uint16_t*)out, lse);
    return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
  }
  const int TT = tree_tile_tokens(G);
  if (!dense) {
    if (n_b <= kUnionBitmapBlocks)
      hipLaunchKernelGGL(tree_union_bitmap_kernel, dim3(h_kv), dim3(kPlanThreads), 0, st,
                         block_idx, n_draft, h_kv, r.topk, (int)n_b, (int32_t*)a.union_blk,
                         (uint64_t*)a.union_mask, (int32_t*)a.union_len, a.union_cap);
    else
      hipLaunchKernelGGL(tree_union_kernel, dim3(h_kv), dim3(kPlanThreads), 0, st, block_idx,
                         n_draft, h_kv, r.topk, n_b, (int32_t*)a.union_blk,
                         (uint64_t*)a.union_mask, (int32_t*)a.union_len, a.union_cap);
    if (hipGetLastError() != hipSuccess) return INFLLMV2_ERR_HIP;
  }
  dim3 grid((unsigned)n_split, h_kv, (unsigned)ceil_div(n_draft, TT));
  INFLLMV2_TRY(d == 128 ? dispatch_tree<128>(G, a, grid, st) : dispatch_tree<64>(G, a, grid, st));
  if (d == 128)
    hipLaunchKernelGGL((combine_kernel<128, uint16_t>), dim3(n_draft * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL((combine_kernel<64, uint16_t>), dim3(n_draft * h_q), dim3(64), 0, st,
                       a.ws, a.n_split, (uint16_t*)out, lse);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

}  // namespace

extern "C" int infllmv2_tree_verify(int dtype, const void* q, int32_t n_draft, const void* k,
                                    const void* v, int64_t cap, int64_t n_ctx,
                                    const void* k_draft, const void* v_draft,
                                    const uint64_t* tree_mask, int32_t h_q, int32_t h_kv,
                                    int32_t d, const int32_t* block_idx, void* out, float* lse,
                                    void* ws, size_t ws_bytes, const infllmv2_params* p,
                                    void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  return tree_call(dtype, q, n_draft, k, v, cap, n_ctx, k_draft, v_draft, tree_mask, h_q, h_kv,
                   d, block_idx, nullptr, out, lse, ws, ws_bytes, r, (hipStream_t)stream);
}

extern "C" int infllmv2_tree_verify_topk(int dtype, const void* q, int32_t n_draft,
                                         const void* k, const void* v, int64_t cap,
                                         int64_t n_ctx, const void* k_draft,
                                         const void* v_draft, const uint64_t* tree_mask,
                                         int32_t h_q, int32_t h_kv, int32_t d,
                                         const float* scores, int64_t nb_cap,
                                         int32_t* block_idx, void* out, float* lse, void* ws,
                                         size_t ws_bytes, const infllmv2_params* p,
                                         void* stream) {
  INFLLMV2_TRY(common_attn_checks(dtype, h_q, h_kv, d));
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  const SelectIn sel = {scores, nb_cap, block_idx};
  return tree_call(dtype, q, n_draft, k, v, cap, n_ctx, k_draft, v_draft, tree_mask, h_q, h_kv,
                   d, nullptr, &sel, out, lse, ws, ws_bytes, r, (hipStream_t)stream);
}
