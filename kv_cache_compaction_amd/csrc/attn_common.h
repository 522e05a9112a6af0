// Shared pieces of the eviction-masked attention kernels (forward and
// backward): the per-key-tile e summary and the live-tile iterator.
//
// The mask M_ij = [j <= i] and [i < e_j] replays compaction: e_j is the trace
// index of the event that evicted key j (KV-streams explainer, trainer paragraph; paper
// page Fig. 2A).  For a key tile T and a query range [i0, i1):
//   skip    if min(T) > i1 - 1 or max_{j in T} e_j <= i0
//   full    if max(T) <= i0 and min_{j in T} e_j >= i1 (and T lies inside N)
//   partial otherwise (the mask is applied element by element).
#pragma once

#include "ks_common.h"

namespace ksattn {

constexpr int kKeyTile = 64;  // keys per summary tile

// emin/emax over key tiles of kKeyTile keys: ws layout [B][ntiles] each.
__global__ void tile_summary_kernel(const int32_t* __restrict__ e, int32_t* __restrict__ emin,
                                    int32_t* __restrict__ emax, int N, int ntiles);

size_t summary_bytes(int B, int N);
ks_status launch_summary(const int32_t* e, void* ws, int B, int N, hipStream_t s,
                         int32_t** emin, int32_t** emax);

// Iterates, in increasing order, the key tiles t <= tmax with emax[t] > i0.
// Every lane of the wave computes the same sequence (ballot over 64 tiles).
struct LiveTiles {
  const int32_t* emax;
  int tmax, i0, base;
  uint64_t mask;
  __device__ __forceinline__ void init(const int32_t* em, int tmax_, int i0_) {
    emax = em;
    tmax = tmax_;
    i0 = i0_;
    base = -64;
    mask = 0;
  }
  __device__ __forceinline__ int next() {
    while (mask == 0) {
      base += 64;
      if (base > tmax) return -1;
      const int t = base + lane_id();
      const bool live = t <= tmax && emax[t] > i0;
      mask = __ballot(live);
    }
    const int t = base + __builtin_ctzll(mask);
    mask &= mask - 1;
    return t;
  }
};

// ---------------------------------------------------------------------------
// LDS tiles of 128-element bf16 rows (D = 128).  A staged row occupies 272
// bytes (256 of data + 16 of padding), and within every block of 16 rows,
// row 4a + b is stored at position 4b + a.  Both access patterns of the MFMA
// loops are then free of bank conflicts:
//   * 16-byte reads of one chunk from 16 consecutive rows (the rows land on
//     16 distinct 16-byte bank groups because of the 16-byte padding), and
//   * ds_read_b64_tr_b16 transpose reads, where 32 lanes read 4 consecutive
//     rows x 32 consecutive columns (the permutation spreads the 4 rows 4
//     positions apart, so row + chunk covers all 16 bank groups once),
// and every operand address is a per-lane base plus a compile-time offset.
// ---------------------------------------------------------------------------
constexpr int kTileRow = 136;  // bf16 elements per staged row

__device__ __forceinline__ int tile_prow(int r) {
  return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ void tile_store_chunk(bf16_t* t, int row, int chunk, u32x4 v) {
  *reinterpret_cast<u32x4*>(t + tile_prow(row) * kTileRow + chunk * 8) = v;
}

// per-lane base of operand reads that give lane l row (rbase + l % 32)
__device__ __forceinline__ int tile_lane_a(int lane) { return tile_prow(lane & 31) * kTileRow; }

// 16-byte chunk `chunk` of row rbase + lane % 32 (rbase a multiple of 16)
__device__ __forceinline__ bf16x8 tile_chunk(const bf16_t* t, int lane_a, int rbase, int chunk) {
  return *reinterpret_cast<const bf16x8*>(t + lane_a + rbase * kTileRow + chunk * 8);
}

__device__ __forceinline__ bf16x4 lds_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

// per-lane base of the transpose reads below
__device__ __forceinline__ int tile_lane_t(int lane) {
  const int j = lane & 15, g = lane >> 4, h = lane >> 5;
  return (4 * (j >> 2) + h) * kTileRow + 16 * (g & 1) + 4 * (j & 3);
}

// A operand of a 32x32x16 MFMA that contracts over tile ROWS: lane l gets
// X[k(v)][dbase + l % 32] for v = 0..7 with
//   k(v) = r0 + 8 * (v / 4) + 4 * (l / 32) + v % 4    (r0 a multiple of 16),
// the k order in which a 32x32 accumulator holds its rows, so P^T or dS^T
// taken straight from an S accumulator is the matching B operand.
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte reads of lanes 4r + i / 4 (r = 0..3); lane 4r + q
// reads row k(r) (stored at position 4 q' ... see tile_prow) and columns
// dbase + 16 (group % 2) + 4 q .. +3.
__device__ __forceinline__ bf16x8 tile_frag_t(const bf16_t* t, int lane_t, int r0, int dbase) {
  const bf16_t* p = t + lane_t + r0 * kTileRow + dbase;
  const bf16x4 lo = lds_tr16(p);                 // v = 0..3: rows r0 + 4h + r
  const bf16x4 hi = lds_tr16(p + 2 * kTileRow);  // v = 4..7: rows r0 + 8 + 4h + r
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc + sum of the 8 bf16 values (packed dot products with (1, 1))
__device__ __forceinline__ float sum_bf16x8(bf16x8 x, float acc) {
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
  return acc;
}

}  // namespace ksattn
