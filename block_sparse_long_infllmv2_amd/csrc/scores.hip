// Block relevance scores: each query row's GQA group scores the semantic
// kernels it can see, and the kernel scores are max-pooled onto the blocks
// they overlap.
// Source: "MiniCPM4: running LLMs on phones and PCs" (xugj520.cn), section 1.1
// InfLLM v2 (queries are scored against semantic kernels and blocks are chosen
// from those scores, avoiding token-level work).
//
//   sigma[m] = scale * (sum_{h in g} q_h) . ck[g][m],  window m visible iff
//              m*s + ks - 1 <= pos
//   S[b]     = max over visible windows m overlapping block b (-inf if none)
//
// Streaming kernel (one workgroup per (row, KV head, chunk of blocks)): the
// group-summed query sits in LDS, d/E threads dot one compressed-key row,
// the window scores of the chunk go to LDS and one thread per block pools
// them.  It is HBM-bound for decode-sized row counts.
#include "host_common.h"
#include "score_common.h"

namespace infllmv2 {

template <typename T, int D>
__global__ __launch_bounds__(kScoreThreads) void block_scores_stream_kernel(ScoreArgs a) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int TPW = D / E;                       // threads per window row
  constexpr int WPP = kScoreThreads / TPW;         // windows per pass
  __shared__ float qs[D];
  __shared__ float sig[kScoreMaxWindows];

  const int r = blockIdx.x / a.chunks_per_row, g = blockIdx.y;
  const int chunk = blockIdx.x % a.chunks_per_row;
  const int seq = a.row_seq ? a.row_seq[r] : 0;
  if (seq < 0 || seq >= a.batch) return;           // malformed row: skipped
  const int64_t L = a.seqlens[seq];
  if (L < a.dense_len) return;                     // dense sequence: no scores
  const int64_t pos = a.row_pos ? a.row_pos[r] : L - 1;
  if (pos < 0 || pos >= L || pos > a.max_pos) return;  // outside the launch bounds
  const int64_t b_own = pos / a.B;
  const int64_t b0 = (int64_t)chunk * a.blocks_per_wg;
  if (b0 > b_own) return;
  const int64_t b1 = min(b0 + a.blocks_per_wg - 1, b_own);
  const int64_t n_vis = pos >= a.ks - 1 ? (pos - a.ks + 1) / a.s + 1 : 0;
  const int64_t m_lo = first_window_of_block(b0, a.B, a.ks, a.s);
  const int64_t m_hi = min(last_window_of_block(b1, a.B, a.s), n_vis - 1);

  // group-summed query, pre-multiplied by the softmax scale
  const int G = a.h_q / a.h_kv;
  const T* qrow = (const T*)a.q + ((int64_t)r * a.h_q + (int64_t)g * G) * D;
  for (int d = threadIdx.x; d < D; d += kScoreThreads) {
    float acc = 0.0f;
    // heads in batches of 8 loads in flight together
    for (int h0 = 0; h0 < G; h0 += 8) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = h0 + j < G ? Elem<T>::load(qrow + (h0 + j) * D + d) : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += x[j];
    }
    qs[d] = acc * a.scale;
  }
  __syncthreads();

  const int sub = threadIdx.x / TPW, lane = threadIdx.x % TPW;
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = qs[lane * E + e];
  const T* ckb = (const T*)a.ck + ((int64_t)seq * a.h_kv + g) * a.nc_cap * D + lane * E;
  // kPasses passes of WPP windows each: all their loads go out before any is
  // used, so a workgroup waits for memory once per kPasses * WPP windows.
  // Two passes, with chunks of up to 64 blocks (flushed steps against eight
  // passes and 32 blocks): 128K batch 1 37.4 -> 36.5 us, 16-draft tree 51.6 ->
  // 48.1 us, batch 32 83.5 -> 80.0 us; ragged batch of 8 within 1 %.
  constexpr int kPasses = 2;
  for (int64_t mb = m_lo; mb <= m_hi; mb += (int64_t)WPP * kPasses) {
    u32x4 w[kPasses];
#pragma unroll
    for (int pp = 0; pp < kPasses; ++pp) {
      const int64_t m = mb + (int64_t)pp * WPP + sub;
      const u32x4 z = {0u, 0u, 0u, 0u};
      w[pp] = m <= m_hi ? ldg16(ckb + m * D) : z;
    }
#pragma unroll
    for (int pp = 0; pp < kPasses; ++pp) {
      const int64_t m = mb + (int64_t)pp * WPP + sub;
      float x[E];
      Elem<T>::unpack(w[pp], x);
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) part += qv[e] * x[e];
#pragma unroll
      for (int o = TPW / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
      if (lane == 0 && m <= m_hi) sig[m - m_lo] = part;
    }
  }
  __syncthreads();

  float* out = a.scores + ((int64_t)r * a.h_kv + g) * a.nb_cap;
  for (int64_t b = b0 + threadIdx.x; b <= b1; b += kScoreThreads) {
    const int64_t lo = first_window_of_block(b, a.B, a.ks, a.s);
    const int64_t hi = min(last_window_of_block(b, a.B, a.s), m_hi);
    float v = -INFINITY;
    for (int64_t m = lo; m <= hi; ++m) v = fmaxf(v, sig[m - m_lo]);
    out[b] = v;
  }
}


// ---------------------------------------------------------------------------
// Matrix-core variant for many rows of one sequence (prefill chunks, draft
// batches) with windows of two strides (ks = 2*s) and blocks of 4 or 8
// strides: with B = 4*s block b overlaps windows 4b-1 .. 4b+3 (its four "own"
// windows and the last own window of block b-1), with B = 8*s windows
// 8b-1 .. 8b+7 (the default 64/32/16 and the 128-token-block variant).
//
// sigma^T = CK . qsum^T on v_mfma_f32_32x32x16_bf16: the A operand is 32
// windows x 16 dims of compressed keys, the B operand 16 dims x 32 rows of
// the group-summed query times the softmax scale.  That float32 sum is split
// into hi + lo bfloat16 parts and both are multiplied, which keeps ~16
// significant bits so the scores match a float32 dot product to ~1e-5
// relative.
// In the 32x32 accumulator a lane (row j, half h) holds windows 8q + 4h + e
// (e = 0..3): with B = 4*s exactly the four own windows of block 2q + h of
// the tile, the fifth (halo) window from the other half-wave or the previous
// tile; with B = 8*s half of block q's own windows, the other half and the
// halo from the other half-wave or the previous tile.
//
// Workgroup = 64 rows x one KV head; its 8 waves take contiguous ranges of
// 32-window tiles, so qsum is built once (in LDS) per workgroup, and each
// wave multiplies every compressed-key fragment it loads by two 32-row
// groups.
// ---------------------------------------------------------------------------
constexpr int kMfmaRG = 2;               // 32-row groups per wave (share A fragments)
constexpr int kMfmaRows = 32 * kMfmaRG;  // rows per workgroup
constexpr int kMfmaWaves = 8;            // waves per workgroup, splitting the windows
// Pooled block scores of consecutive tiles (32 windows each: 8 blocks of 4
// windows or 4 blocks of 8) are gathered per wave in LDS and written out as
// whole 32-block (128-byte) row pieces.
constexpr int kStageBlocks = 32;
constexpr int kStageStride = kStageBlocks + 4;   // floats per staged row (16-byte pad)

// Maximum of two window scores for the pooling.  Scores are finite or -inf
// (windows past a row), so the NaN-propagating maximum gives what fmaxf
// gives; it is issued as v_maximum3_f32 with no canonicalising v_max of each
// operand, which fmaxf's NaN-ignoring semantics need on matrix-core results.
__device__ __forceinline__ float pool_max(float x, float y) {
  return __builtin_elementwise_maximum(x, y);
}

// WPB = windows per block (B / s): 4 or 8.
template <int D, int WPB>
__global__ __launch_bounds__(kMfmaWaves * 64) void block_scores_mfma_kernel(ScoreArgs a, int n_row_tiles) {
  static_assert(WPB == 4 || WPB == 8, "block = 4 or 8 window strides");
  constexpr int KS = D / 16;
  constexpr int RG = kMfmaRG;
  constexpr int BPT = 32 / WPB;                    // blocks per 32-window tile
  constexpr int kStageTiles = kStageBlocks / BPT;  // tiles per staged group
  __shared__ __attribute__((aligned(16))) uint16_t qlds[2][kMfmaRows][D + 8];
  __shared__ int pos_lds[kMfmaRows];
  __shared__ int own_lds[kMfmaRows];               // the row's own block, -1: no row
  __shared__ __attribute__((aligned(16))) float stage[kMfmaWaves][kMfmaRows * kStageStride];

  const int w = xcd_contiguous_index(blockIdx.x, gridDim.x);
  const int g = w / n_row_tiles, tile = w % n_row_tiles;
  const int r0 = tile * kMfmaRows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.h_q / a.h_kv;
  const int64_t L = a.seqlens[0];
  if (L < a.dense_len) return;

  // group-summed query rows -> hi/lo bf16 in LDS; positions
  for (int it = tid; it < kMfmaRows * (D / 8); it += kMfmaWaves * 64) {
    const int rr = it / (D / 8), c = it % (D / 8);
    const int row = r0 + rr;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    if (row < a.rows) {
      const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)row * a.h_q + (int64_t)g * G) * D + c * 8;
      // heads in batches of 16 loads issued together (the head count is a
      // run-time value; a plain loop would wait for each load in turn)
      for (int h0 = 0; h0 < G; h0 += 16) {
        u32x4 w[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (h0 + j < G) w[j] = ldg16(qp + (int64_t)(h0 + j) * D);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (h0 + j < G) {
            float x[8];
            Elem<uint16_t>::unpack(w[j], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += x[e];
          }
      }
    }
    // the softmax scale goes into the query sum, so accumulators hold sigma
    u32x4 hi, lo;
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = acc[e] * a.scale;
      hb[e] = float_to_bf16_bits(v);
      lb[e] = float_to_bf16_bits(v - bf16_bits_to_float(hb[e]));
    }
    hi.x = hb[0] | (hb[1] << 16); hi.y = hb[2] | (hb[3] << 16);
    hi.z = hb[4] | (hb[5] << 16); hi.w = hb[6] | (hb[7] << 16);
    lo.x = lb[0] | (lb[1] << 16); lo.y = lb[2] | (lb[3] << 16);
    lo.z = lb[4] | (lb[5] << 16); lo.w = lb[6] | (lb[7] << 16);
    *reinterpret_cast<u32x4*>(&qlds[0][rr][c * 8]) = hi;
    *reinterpret_cast<u32x4*>(&qlds[1][rr][c * 8]) = lo;
  }
  if (tid < kMfmaRows) {
    const int row = r0 + tid;
    int pos = -1;
    if (row < a.rows) {
      const int64_t p = a.row_pos ? a.row_pos[row] : L - 1;
      pos = (p >= L || p > a.max_pos || p < 0) ? -1 : (int)p;
    }
    pos_lds[tid] = pos;
    own_lds[tid] = pos < 0 ? -1 : pos / a.B;
  }
  __syncthreads();

  // this lane: column `col` of row groups rg = 0..RG-1 (row r0 + 32 rg + col)
  bf16x8 qh[RG][KS], ql[RG][KS];
  int pos[RG], n_vis[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int rr = 32 * rg + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qh[rg][ks] = *reinterpret_cast<const bf16x8*>(&qlds[0][rr][16 * ks + 8 * half]);
      ql[rg][ks] = *reinterpret_cast<const bf16x8*>(&qlds[1][rr][16 * ks + 8 * half]);
    }
    pos[rg] = pos_lds[rr];
    // visible windows: m*s + ks - 1 <= pos (32-bit: the host bounds max_pos)
    n_vis[rg] = pos[rg] >= a.ks - 1 ? (pos[rg] - a.ks + 1) / a.s + 1 : 0;
  }
  int tile_max_pos = -1, tile_min_vis = 0x7fffffff;
  for (int j = 0; j < kMfmaRows; ++j) {
    const int pj = pos_lds[j];
    tile_max_pos = max(tile_max_pos, pj);
    if (pj >= 0) tile_min_vis = min(tile_min_vis, pj >= a.ks - 1 ? (pj - a.ks + 1) / a.s + 1 : 0);
  }
  tile_max_pos = __builtin_amdgcn_readfirstlane(tile_max_pos);   // same in every lane
  tile_min_vis = __builtin_amdgcn_readfirstlane(tile_min_vis);
  const int nb_tile = tile_max_pos < 0 ? 0 : tile_max_pos / a.B + 1;   // blocks to score
  const int n_tiles = (nb_tile + BPT - 1) / BPT;
  const uint16_t* ckb = (const uint16_t*)a.ck + (int64_t)g * a.nc_cap * D;
  const int nc_cap = (int)min(a.nc_cap, (int64_t)0x7fffffff);

  // dot of this lane's query half with one compressed key (VALU), combined
  // over the two half-waves: the halo window before a wave's first tile
  auto single_window = [&](int m, int rg) -> float {
    float part = 0.0f;
    if (m >= 0 && m < nc_cap) {
      const uint16_t* c = ckb + (int64_t)m * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
        Elem<uint16_t>::unpack(ldg16(c + 16 * ks + 8 * half), x);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          part += ((float)qh[rg][ks][e] + (float)ql[rg][ks][e]) * x[e];
      }
    }
    const float full = part + swap_halves(part);
    return (m >= 0 && m < n_vis[rg]) ? full : -INFINITY;
  };

  // each wave takes a contiguous range of tiles (8 blocks = 32 windows each);
  // the halo of a tile's first block is the previous tile's last window,
  // carried in registers (computed directly only for the range's first tile)
  const int per_wave = (n_tiles + kMfmaWaves - 1) / kMfmaWaves;
  const int t_begin = __builtin_amdgcn_readfirstlane(wave) * per_wave;   // a scalar tile loop
  const int t_end = min(n_tiles, t_begin + per_wave);
  float carry[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
    carry[rg] = t_begin < t_end ? single_window(t_begin * 32 - 1, rg) : -INFINITY;
  // A-operand fragments of a tile: window 32 tt + col, dims 16ks + 8half
  auto load_tile = [&](int tt, u32x4* fr) {
    const int mrow = tt * 32 + col;
    if (tt * 32 + 31 < nc_cap) {               // whole tile inside the buffer (uniform)
      const uint16_t* crow = ckb + (int64_t)mrow * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) fr[ks] = ldg16(crow + 16 * ks);
      return;
    }
    const bool in = mrow < nc_cap;
    const uint16_t* crow = ckb + (int64_t)(in ? mrow : 0) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 wv = ldg16(crow + 16 * ks);
      const u32x4 z = {0u, 0u, 0u, 0u};
      fr[ks] = in ? wv : z;
    }
  };
  // Write the staged group that tile t closes: lane l takes row 8 i + l / 8
  // and blocks 4 (l % 8) .. + 3 of the group, so each store instruction
  // covers 8 rows x 128 contiguous bytes.  Only this wave's tiles of the
  // group are written, and only blocks up to the row's own block.
  float* sw = stage[wave];
  auto flush = [&](int t) {
    const int g0 = (t / kStageTiles) * kStageTiles;          // first tile of the group
    const int tb = max(g0, t_begin), te = t;                 // staged tiles tb .. te
    const int piece = lane & 7, sub = lane >> 3;
    const int blk = BPT * g0 + 4 * piece;                    // first block of the piece
    const bool in = blk >= BPT * tb && blk < BPT * (te + 1);
#pragma unroll 1
    for (int i = 0; i < kMfmaRows / 8; ++i) {
      const int rr = 8 * i + sub;
      const int bo = own_lds[rr];
      if (!in || bo < 0) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(&sw[rr * kStageStride + 4 * piece]);
      float* o = a.scores + ((int64_t)(r0 + rr) * a.h_kv + g) * a.nb_cap + blk;
      if (blk + 3 <= bo && a.vec_store) {
        *reinterpret_cast<f32x4*>(o) = v;
      } else {
        if (blk + 0 <= bo) o[0] = v.x;
        if (blk + 1 <= bo) o[1] = v.y;
        if (blk + 2 <= bo) o[2] = v.z;
        if (blk + 3 <= bo) o[3] = v.w;
      }
    }
  };
  u32x4 frag[KS];
  if (t_begin < t_end) load_tile(t_begin, frag);
  for (int t = t_begin; t < t_end; ++t) {
    const int mt = t * 32;                     // first own window of the tile
    u32x4 cur[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cur[ks] = frag[ks];
    if (t + 1 < t_end) load_tile(t + 1, frag);  // next tile's loads in flight
    f32x16 acc[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rg][v] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(&cur[ks]);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        acc[rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qh[rg][ks], acc[rg], 0, 0, 0);
        acc[rg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ql[rg][ks], acc[rg], 0, 0, 0);
      }
    }
    const bool full_vis = mt + 32 <= tile_min_vis;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      // per 4-window group q of the lane's half: its maximum and last window
      // (windows 8q + 4 half .. + 3 of the tile); tiles wholly visible to
      // every row of the workgroup skip the masking
      float own[4], last[4];
      if (full_vis) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          own[q] = pool_max(pool_max(acc[rg][4 * q], acc[rg][4 * q + 1]),
                         pool_max(acc[rg][4 * q + 2], acc[rg][4 * q + 3]));
          last[q] = acc[rg][4 * q + 3];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = mt + 8 * q + 4 * half + e;
            const float x = m < n_vis[rg] ? acc[rg][4 * q + e] : -INFINITY;
            mx = pool_max(mx, x);
            if (e == 3) last[q] = x;
          }
          own[q] = mx;
        }
      }
      float other[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) other[q] = swap_halves(last[q]);
      if constexpr (WPB == 4) {
        // block 2q + half of the tile: the lane's four windows; its halo
        // window is the last own window of the block before it:
        // half 1 <- (q, half 0); half 0 <- (q-1, half 1)
        float bs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float halo = half ? other[q] : (q > 0 ? other[q - 1] : carry[rg]);
          bs[q] = pool_max(own[q], halo);
        }
        carry[rg] = other[3];     // for half-0 lanes: last window of block 7
        // regroup: half 0 -> blocks 0..3 of the tile, half 1 -> 4..7
        const float x0 = swap_halves(half ? bs[0] : bs[2]);
        const float x1 = swap_halves(half ? bs[1] : bs[3]);
        f32x4 w4;
        if (half == 0) { w4.x = bs[0]; w4.y = x0; w4.z = bs[1]; w4.w = x1; }
        else           { w4.x = x0; w4.y = bs[2]; w4.z = x1; w4.w = bs[3]; }
        // staged: row 32 rg + col, blocks 8 (t % kStageTiles) + 4 half .. + 3
        *reinterpret_cast<f32x4*>(&sw[(32 * rg + col) * kStageStride +
                                     8 * (t % kStageTiles) + 4 * half]) = w4;
      } else {
        // block q of the tile: windows 8q .. 8q+7, four in each half; its
        // halo window 8q - 1 is the last window of block q - 1 (half 1), or
        // of the previous tile for q = 0
        float bs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float both = pool_max(own[q], swap_halves(own[q]));
          const float halo = q > 0 ? (half ? last[q - 1] : other[q - 1]) : carry[rg];
          bs[q] = pool_max(both, halo);
        }
        carry[rg] = half ? last[3] : other[3];     // window 31 of the tile
        if (half == 0) {
          const f32x4 w4 = {bs[0], bs[1], bs[2], bs[3]};
          *reinterpret_cast<f32x4*>(&sw[(32 * rg + col) * kStageStride +
                                       4 * (t % kStageTiles)]) = w4;
        }
      }
    }
    if ((t + 1) % kStageTiles == 0 || t + 1 == t_end) flush(t);
  }
}

// ---------------------------------------------------------------------------
// score_mode 1: sigma[m] = sum over the group's heads of each head's softmax
// over the windows visible to the row (the other plain reading of the group
// score).  One workgroup (4 waves) per (row, KV head): a wave takes tiles of
// 16 windows; on v_mfma_f32_16x16x32_bf16 the tile's logits for the group's
// (up to 16) heads land as D[window][head] (lane (head j, group q) holds
// windows 4q .. 4q+3 of the tile); float32 inputs compute the same logits
// on the VALU in the same lane layout.
//   pass 1: per head, the online max and sum of exp over the visible windows
//           (log2 domain), merged over lanes and waves;
//   pass 2: the logits again, each head's normalised share, summed over the
//           16 head lanes into sig[m] (LDS, one float per visible window);
// then every block takes the max of sig over its visible windows.
// ---------------------------------------------------------------------------
constexpr int kSoftmaxWaves = 4;
constexpr int kSoftmaxMaxWindows = 16384;    // LDS: one float per visible window

template <typename T, int D>
__global__ __launch_bounds__(kSoftmaxWaves * 64) void block_scores_softmax_kernel(ScoreArgs a) {
  __shared__ float sig[kSoftmaxMaxWindows];
  __shared__ float st_m[kSoftmaxWaves][16], st_s[kSoftmaxWaves][16];
  const int r = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 15, qg = lane >> 4;               // head, 4-window group
  const int seq = a.row_seq ? a.row_seq[r] : 0;
  if (seq < 0 || seq >= a.batch) return;
  const int64_t L = a.seqlens[seq];
  if (L < a.dense_len) return;
  const int64_t pos = a.row_pos ? a.row_pos[r] : L - 1;
  if (pos < 0 || pos >= L || pos > a.max_pos) return;
  const int b_own = (int)(pos / a.B);
  const int n_vis = pos >= a.ks - 1 ? (int)((pos - a.ks + 1) / a.s) + 1 : 0;
  const int G = a.h_q / a.h_kv;
  const bool head_ok = j < G;
  const float c = a.scale * kLog2e;                      // logits in log2 units
  const T* qrow = (const T*)a.q + ((int64_t)r * a.h_q + (int64_t)g * G + (head_ok ? j : 0)) * D;
  const T* ckb = (const T*)a.ck + ((int64_t)seq * a.h_kv + g) * a.nc_cap * D;
  const int n_tiles = (n_vis + 15) / 16;

  // bf16: this lane's query slices (B operand: head j, dims 32 ks + 8 qg ..
  // + 8); float32: the group's queries in LDS (each lane computes full dots)
  constexpr int KS = D / 32;
  bf16x8 qb[KS];
  __shared__ __attribute__((aligned(16))) float qs[sizeof(T) == 2 ? 1 : 16][D];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (head_ok) w = ldg16(qrow + 32 * ks + 8 * qg);
      qb[ks] = *reinterpret_cast<const bf16x8*>(&w);
    }
  } else {
    const T* qg0 = (const T*)a.q + ((int64_t)r * a.h_q + (int64_t)g * G) * D;
    for (int i = tid; i < 16 * D; i += kSoftmaxWaves * 64)
      qs[i / D][i % D] = i / D < G ? Elem<T>::load(qg0 + i) : 0.0f;
    __syncthreads();
  }

  // logits (log2 units) of tile t for head j at windows 16 t + 4 qg + e
  auto tile_logits = [&](int t, float (&lg)[4]) {
    const int w0 = 16 * t;
    if constexpr (sizeof(T) == 2) {
      const int wi = w0 + j;                             // A row of this lane: window w0 + j
      const bool in = wi < n_vis;
      const T* crow = ckb + (int64_t)(in ? wi : 0) * D + 8 * qg;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 w = ldg16(crow + 32 * ks);
        if (!in) w = u32x4{0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(&w),
                                                      qb[ks], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) lg[e] = acc[e] * c;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = w0 + 4 * qg + e;
        const T* crow = ckb + (int64_t)(m < n_vis ? m : 0) * D;
        float dot = 0.0f;
#pragma unroll 4
        for (int d = 0; d < D; d += 4) {
          float x[4];
          Elem<T>::unpack(ldg16(crow + d), x);
          const f32x4 qv = *reinterpret_cast<const f32x4*>(&qs[j][d]);
#pragma unroll
          for (int u = 0; u < 4; ++u) dot = __builtin_fmaf(qv[u], x[u], dot);
        }
        lg[e] = dot * c;
      }
    }
  };

  // pass 1: per head, running max and sum of 2^(logit - max)
  float hm = -INFINITY, hs = 0.0f;
  for (int t = wave; t < n_tiles; t += kSoftmaxWaves) {
    float lg[4];
    tile_logits(t, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * t + 4 * qg + e;
      if (m < n_vis) {
        const float nm = fmaxf(hm, lg[e]);
        hs = hs * fast_exp2(hm - nm) + fast_exp2(lg[e] - nm);
        hm = nm;
      }
    }
  }
  // merge the four lanes of head j (lanes j + 16 q), then the waves
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float om = __shfl_xor(hm, o, 64), os = __shfl_xor(hs, o, 64);
    const float nm = fmaxf(hm, om);
    hs = (hm == -INFINITY ? 0.0f : hs * fast_exp2(hm - nm)) +
         (om == -INFINITY ? 0.0f : os * fast_exp2(om - nm));
    hm = nm;
  }
  if (lane < 16) { st_m[wave][lane] = hm; st_s[wave][lane] = hs; }
  __syncthreads();
  float M = -INFINITY, S = 0.0f;
#pragma unroll
  for (int w = 0; w < kSoftmaxWaves; ++w) {
    const float om = st_m[w][j], os = st_s[w][j];
    const float nm = fmaxf(M, om);
    S = (M == -INFINITY ? 0.0f : S * fast_exp2(M - nm)) +
        (om == -INFINITY ? 0.0f : os * fast_exp2(om - nm));
    M = nm;
  }
  const float inv = S > 0.0f ? 1.0f / S : 0.0f;

  // pass 2: each head's share, summed over the 16 head lanes
  for (int t = wave; t < n_tiles; t += kSoftmaxWaves) {
    float lg[4];
    tile_logits(t, lg);
    float sh[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * t + 4 * qg + e;
      float v = (head_ok && m < n_vis) ? fast_exp2(lg[e] - M) * inv : 0.0f;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
      sh[e] = v;
    }
    if (j == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * t + 4 * qg + e;
        if (m < n_vis) sig[m] = sh[e];
      }
    }
  }
  __syncthreads();

  // block b: max of sig over its visible windows (-inf if none)
  float* out = a.scores + ((int64_t)r * a.h_kv + g) * a.nb_cap;
  for (int b = tid; b <= b_own; b += kSoftmaxWaves * 64) {
    const int64_t lo = first_window_of_block(b, a.B, a.ks, a.s);
    const int64_t hi = min(last_window_of_block(b, a.B, a.s), (int64_t)n_vis - 1);
    float v = -INFINITY;
    for (int64_t m = lo; m <= hi; ++m) v = fmaxf(v, sig[m]);
    out[b] = v;
  }
}

template <typename T, int D>
static int launch_scores(const ScoreArgs& a, int rows, hipStream_t st) {
  dim3 grid((unsigned)((int64_t)a.chunks_per_row * rows), a.h_kv, 1);
  hipLaunchKernelGGL((block_scores_stream_kernel<T, D>), grid, dim3(kScoreThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
}

}  // namespace infllmv2

using namespace infllmv2;

extern "C" int infllmv2_block_scores(int dtype, const void* q, int32_t rows,
                                     const int32_t* row_seq, const int32_t* row_pos,
                                     int32_t h_q, int32_t h_kv, int32_t d, const void* ck,
                                     int32_t batch, int64_t nc_cap, const int32_t* seqlens,
                                     float* scores, int64_t nb_cap, int32_t max_pos,
                                     const infllmv2_params* p, void* stream) {
  if (!dtype_ok(dtype)) return INFLLMV2_ERR_INVALID_ARG;
  if (!q || !ck || !seqlens || !scores) return INFLLMV2_ERR_INVALID_ARG;
  if (rows < 0 || batch <= 0 || nc_cap <= 0 || nb_cap <= 0 || max_pos < 0)
    return INFLLMV2_ERR_INVALID_ARG;
  INFLLMV2_TRY(check_heads(h_q, h_kv));
  if (!head_dim_ok(d)) return INFLLMV2_ERR_UNSUPPORTED;
  Resolved r;
  INFLLMV2_TRY(check_params(p, d, &r));
  if ((int64_t)max_pos / r.B + 1 > nb_cap) return INFLLMV2_ERR_INVALID_ARG;
  if (num_windows((int64_t)max_pos + 1, r.ks, r.s) > nc_cap) return INFLLMV2_ERR_INVALID_ARG;
  if (!aligned16(ck) || !aligned16(q)) return INFLLMV2_ERR_INVALID_ARG;
  if (r.score_mode == 1) {
    if (h_q / h_kv > 16) return INFLLMV2_ERR_UNSUPPORTED;
    if (num_windows((int64_t)max_pos + 1, r.ks, r.s) > kSoftmaxMaxWindows)
      return INFLLMV2_ERR_UNSUPPORTED;
  }
  if (rows == 0) return INFLLMV2_OK;
  ScoreArgs a;
  a.q = q; a.row_seq = row_seq; a.row_pos = row_pos; a.ck = ck; a.seqlens = seqlens;
  a.scores = scores; a.nc_cap = nc_cap; a.nb_cap = nb_cap; a.h_q = h_q; a.h_kv = h_kv;
  a.B = r.B; a.ks = r.ks; a.s = r.s; a.dense_len = r.dense_len; a.scale = r.scale;
  a.batch = batch; a.max_pos = max_pos; a.rows = rows;
  a.vec_store = (nb_cap % 4 == 0) && aligned16(scores);
  const int64_t nb_launch = (int64_t)max_pos / r.B + 1;
  const int bpw = stream_blocks_per_wg(r.B, r.ks, r.s, nb_launch, rows, h_kv);
  if (bpw < 1) return INFLLMV2_ERR_UNSUPPORTED;
  a.blocks_per_wg = bpw;
  a.chunks_per_row = (int)ceil_div(nb_launch, bpw);
  if ((int64_t)a.chunks_per_row * rows >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (r.score_mode == 1) {
    dim3 grid((unsigned)rows, (unsigned)h_kv);
    if (dtype == INFLLMV2_BF16) {
      if (d == 128)
        hipLaunchKernelGGL((block_scores_softmax_kernel<uint16_t, 128>), grid,
                           dim3(kSoftmaxWaves * 64), 0, st, a);
      else
        hipLaunchKernelGGL((block_scores_softmax_kernel<uint16_t, 64>), grid,
                           dim3(kSoftmaxWaves * 64), 0, st, a);
    } else {
      if (d == 128)
        hipLaunchKernelGGL((block_scores_softmax_kernel<float, 128>), grid,
                           dim3(kSoftmaxWaves * 64), 0, st, a);
      else
        hipLaunchKernelGGL((block_scores_softmax_kernel<float, 64>), grid,
                           dim3(kSoftmaxWaves * 64), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
  }
  const bool mfma_geometry = r.ks == 2 * r.s && (r.B == 4 * r.s || r.B == 8 * r.s);
  if (dtype == INFLLMV2_BF16 && batch == 1 && row_seq == nullptr && mfma_geometry &&
      rows >= kMfmaMinRows) {
    const int n_row_tiles = (int)ceil_div(rows, kMfmaRows);
    if ((int64_t)n_row_tiles * h_kv >= (1ll << 31)) return INFLLMV2_ERR_UNSUPPORTED;
    dim3 grid((unsigned)(n_row_tiles * h_kv));
    const bool wide = r.B == 8 * r.s;
    if (d == 128 && !wide)
      hipLaunchKernelGGL((block_scores_mfma_kernel<128, 4>), grid, dim3(kMfmaWaves * 64), 0, st, a,
                         n_row_tiles);
    else if (d == 128)
      hipLaunchKernelGGL((block_scores_mfma_kernel<128, 8>), grid, dim3(kMfmaWaves * 64), 0, st, a,
                         n_row_tiles);
    else if (!wide)
      hipLaunchKernelGGL((block_scores_mfma_kernel<64, 4>), grid, dim3(kMfmaWaves * 64), 0, st, a,
                         n_row_tiles);
    else
      hipLaunchKernelGGL((block_scores_mfma_kernel<64, 8>), grid, dim3(kMfmaWaves * 64), 0, st, a,
                         n_row_tiles);
    return hipGetLastError() == hipSuccess ? INFLLMV2_OK : INFLLMV2_ERR_HIP;
  }
  if (dtype == INFLLMV2_BF16)
    return d == 128 ? launch_scores<uint16_t, 128>(a, rows, st)
                    : launch_scores<uint16_t, 64>(a, rows, st);
  return d == 128 ? launch_scores<float, 128>(a, rows, st)
                  : launch_scores<float, 64>(a, rows, st);
}
