// LDS staging helpers shared by the bf16 attention kernels (forward and
// backward): swizzled 64-key K/V tiles copied with direct global->LDS loads,
// 16-byte and transposing fragment reads, and the sorted union of the kept
// blocks of a tile of query tokens.
#pragma once

#include "attn_common.h"

namespace infllmv2 {

// ---------------------------------------------------------------------------
// Direct staging: global_load_lds_dwordx4 moves 16 bytes per lane from HBM
// straight into LDS (lane l of one instruction lands at M0 + 16 l), so a
// chunk in flight holds no registers and costs no LDS write instructions.
// K and V tiles keep the natural [key][d] layout; the 16-byte column chunk c
// of row r is stored at chunk position c ^ f(r), which keeps both fragment
// reads free of bank conflicts on the 64-bank LDS:
//   K (16-byte reads, 16 lanes per pass): 16 consecutive rows reading one
//     logical chunk hit 16 distinct 16-byte bank groups;
//   V (8-byte transposing reads, 32 lanes per pass): 4 consecutive rows x 4
//     consecutive chunks hit 16 distinct groups.
// f depends on r mod 16 only, so tiles of 16 rows repeat the same pattern.
// ---------------------------------------------------------------------------
template <int D>
struct Swz {
  static constexpr int RB = 2 * D;              // bytes per row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int TILE = kChunk * RB;      // bytes per K or V tile
  __device__ static __forceinline__ int f(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

// One 16-byte-per-lane copy global -> LDS.  `lds_addr` (wave-uniform) is the
// byte address of lane 0's destination; `gbase` (wave-uniform) plus the
// lane's byte offset `voff` is its source.  M0 must be written one wait state
// before the load that reads it.
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are still in
// flight (they complete in issue order) and its LDS reads are done, then
// meet the other waves.  The compiler does not see the direct loads, so this
// is the only wait that orders them before the LDS reads of their tile.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

template <int D, int NT, class SW = Swz<D>>
struct DmaTile {
  static constexpr int CPR = SW::CPR;
  static constexpr int RB = SW::RB;
  // 16-byte slots per tile; with more threads than slots, the first
  // kActive threads (whole waves) copy and the others issue nothing
  static constexpr int kSlots = SW::TILE / 16;
  static constexpr int kActive = kSlots >= NT ? NT : kSlots;
  static constexpr int kLoads = kSlots / kActive;          // per copying thread and tile
  static_assert(kActive % 64 == 0 && kSlots % kActive == 0, "tile copy shape");
  static_assert(2 * kLoads <= 63, "vmcnt range");
  // Instruction i, thread t -> LDS slot s = i*kActive + t: row s / CPR,
  // position s % CPR.  When one instruction spans a multiple of 16 rows, the
  // swizzle phase f(r) is the same for every i and the source offsets differ
  // by a whole number of rows: one base offset, the row step goes to the pointer.
  static constexpr int kRowsPerInst = kActive / CPR;
  static constexpr bool kUniform = kRowsPerInst % 16 == 0;
  // source byte offsets in a full tile; the uniform case recomputes its single
  // offset at each issue (a few VALU) instead of holding a register
  uint32_t voff[kUniform ? 1 : kLoads];

  __device__ static __forceinline__ uint32_t offset(int i, int tid) {
    const int s = i * kActive + (tid % kActive), r = s / CPR;
    return (uint32_t)(r * RB + (((s % CPR) ^ SW::f(r)) * 16));
  }
  __device__ __forceinline__ void init(int tid) {
    if constexpr (!kUniform) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) voff[i] = offset(i, tid);
    }
  }
  // rows >= nv are copies of row nv - 1 (finite data; the softmax masks them)
  __device__ __forceinline__ void issue(uint32_t lds_tile, const uint16_t* g, int nv, int tid,
                                        int wave) const {
    if (kActive < NT && wave * 64 >= kActive) return;
    if (nv == kChunk) {
      const uint32_t off0 = kUniform ? offset(0, tid) : 0u;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        if constexpr (kUniform)
          lds_dma16(lds_tile + (uint32_t)(i * kActive + wave * 64) * 16u,
                    g + i * kRowsPerInst * D, off0);
        else
          lds_dma16(lds_tile + (uint32_t)(i * kActive + wave * 64) * 16u, g, voff[i]);
      }
    } else {
      const int last = nv > 0 ? nv - 1 : 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int s = i * kActive + tid, r = s / CPR;
        const int rr = r < last ? r : last;
        lds_dma16(lds_tile + (uint32_t)(i * kActive + wave * 64) * 16u, g,
                  (uint32_t)(rr * RB + (((s % CPR) ^ SW::f(r)) * 16)));
      }
    }
  }
};

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
  return *reinterpret_cast<const lds_bf16x8*>((uintptr_t)addr);
}
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte pieces addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr8(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)addr);
}

// ---------------------------------------------------------------------------
// Bitonic sort (ascending) of N uint32 keys in LDS by NT threads.
// ---------------------------------------------------------------------------
template <int NT>
__device__ void bitonic_sort(uint32_t* buf, int N) {
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < N; i += NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint32_t a = buf[i], b = buf[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) { buf[i] = b; buf[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
}

template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < NT / 64; ++w) {
    const int t = lds[w];
    if (w < wid) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Union of the kept-block lists of TT tokens: sorted unique block ids with a
// bitmask of the tokens (bit t) that kept each, written to ents[] as
// (block, mask).  `sortbuf` holds N >= TT*topk (power of two) words; returns
// the union length.
template <int NT, int TT>
__device__ int build_union(const int32_t* block_idx, int tok0, int h_kv, int g, int n_tok,
                           int topk, int n_b, uint32_t* sortbuf, int N, int2* ents,
                           int* scan_lds) {
  for (int i = threadIdx.x; i < N; i += NT) {
    uint32_t key = 0xffffffffu;
    const int t = i / topk, j = i % topk;
    if (t < n_tok && i < TT * topk) {
      const int32_t b = block_idx[((int64_t)(tok0 + t) * h_kv + g) * topk + j];
      if (b >= 0 && b < n_b) key = ((uint32_t)b << 5) | (uint32_t)t;
    }
    sortbuf[i] = key;
  }
  __syncthreads();
  bitonic_sort<NT>(sortbuf, N);
  // thread t scans C consecutive sorted keys (N: a power of two, so either a
  // multiple of NT or below it, one key per thread then)
  const int C = N >= NT ? N / NT : 1;
  const int c0 = threadIdx.x * C;
  const int c1 = min(c0 + C, N);
  int heads = 0;
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = sortbuf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (sortbuf[i - 1] >> 5) != (key >> 5)) ++heads;
  }
  int total;
  int slot = block_excl_scan<NT>(heads, &total, scan_lds);
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = sortbuf[i];
    if (key == 0xffffffffu) break;
    if (i == 0 || (sortbuf[i - 1] >> 5) != (key >> 5)) {
      uint32_t msk = 0;
      for (int i2 = i; i2 < N && sortbuf[i2] != 0xffffffffu && (sortbuf[i2] >> 5) == (key >> 5);
           ++i2)
        msk |= 1u << (sortbuf[i2] & 31u);
      ents[slot] = make_int2((int)(key >> 5), (int)msk);
      ++slot;
    }
  }
  __syncthreads();
  return total;
}

template <int S> struct StageTag { static constexpr int value = S; };

// K and V tiles use different chunk swizzles, each free of LDS bank
// conflicts for its own read pattern (checked with the bank-conflict counter
// on gfx950; both depend on r mod 16 only):
//   K, 16-byte reads: 16 consecutive rows read one logical chunk;
//   V, transposing 8-byte reads: 8 consecutive rows x chunk pair {2m, 2m+1}.
template <int D>
struct Swz16K {
  static constexpr int RB = 2 * D;
  static constexpr int CPR = D / 8;
  static constexpr int TILE = kChunk * RB;
  __device__ static __forceinline__ int f(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
};
template <int D>
struct Swz16V {
  static constexpr int RB = 2 * D;
  static constexpr int CPR = D / 8;
  static constexpr int TILE = kChunk * RB;
  __device__ static __forceinline__ int f(int r) {
    return D == 128 ? 2 * (r & 7) + ((r >> 3) & 1) : 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
  }
};
template <int D> using Swz16 = Swz16V<D>;   // tile geometry (same for K and V)

// A tile read both ways: as rows (lane (jj, hh) reads row jj, logical chunk
// 4 ks + hh, with 16-byte reads) and transposed (row 4 hh + jj / 4, chunk
// 2 dt + (jj % 4) / 2, half jj % 2, with 8-byte transposing reads), as the
// backward kernels read theirs.  For D = 128, f is the XOR-linear map of the
// row's low four bits with f(1) = 12, f(2) = 15, f(4) = 4, f(8) = 5: of all
// 20160 such maps, timed on gfx950 for exactly these two patterns
// (probes/lds_swizzle_search.hip), one within 5 % of the fastest for both.
// Swz16V runs the row reads 1.7x slower (bank conflicts), Swz16K the
// transposed reads 1.8x.  Other D keep Base's map.
template <int D, class Base>
struct Swz16RT : Base {
  __device__ static __forceinline__ int f(int r) {
    if constexpr (D == 128)
      return (-(r & 1) & 12) ^ (-((r >> 1) & 1) & 15) ^ (-((r >> 2) & 1) & 4) ^
             (-((r >> 3) & 1) & 5);
    else
      return Base::f(r);
  }
};

}  // namespace infllmv2
