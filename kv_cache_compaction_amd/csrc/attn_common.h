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

// Per-key-tile summary of e (tiles of kKeyTile keys), kept in the workspace:
//   erec [B][ntiles][kErec]  per tile: e of its 64 keys (0 past N), then
//                            {min e, max e, 0, 0}; 272 bytes, one DMA unit
//   emin, emax [B][ntiles]   the same minima and maxima as plain arrays
constexpr int kErec = kKeyTile + 4;
struct TileSummary {
  int32_t* erec;
  int32_t* emin;
  int32_t* emax;
};

__global__ void tile_summary_kernel(const int32_t* __restrict__ e, TileSummary ts, int N,
                                    int ntiles);

size_t summary_bytes(int B, int N);
ks_status launch_summary(const int32_t* e, void* ws, int B, int N, hipStream_t s,
                         TileSummary* ts);

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

// max and sum of x over the lane pair (l, l ^ 32): v_permlane32_swap
// exchanges the two halves of the wave in registers (a VALU op; a shuffle
// would go through LDS)
__device__ __forceinline__ float max_lane_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_lane_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// ---------------------------------------------------------------------------
// LDS-DMA staging.  global_load_lds_dwordx4 copies 16 bytes per lane from
// global memory into LDS at (wave-uniform base + 16 * lane) without passing
// through registers.  Waits are explicit: a wave waits for its own DMA loads
// with wait_vm, then a fence-free barrier makes every wave's loads visible.
// Every wave issues the same number of DMA loads per staged unit, so the
// count a wave may leave in flight is a compile-time constant.  Pipelined
// loops run a whole number of unrolled steps (no early exit from inside
// the unrolled body) and land the prologue's loads before the loop: with
// those two shapes the compiler's own wait analysis adds no further waits.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;

// an LDS-typed view of a __shared__ array: DMA targets stay in the LDS
// address space (no generic-pointer round trip and its null check)
__device__ __forceinline__ lds_bf16_t* lds_ptr(bf16_t* shared_array) {
  return (lds_bf16_t*)(shared_array);
}

__device__ __forceinline__ void lds_dma16(const void* src, lds_bf16_t* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_dst), 16,
                                   0, 0);
}

// wait until at most N vector-memory operations of this wave are pending
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // s_waitcnt fields: vmcnt[3:0], expcnt[6:4] (7 = no wait), lgkmcnt[11:8]
  // (15 = no wait), vmcnt[5:4] in bits 15:14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// workgroup barrier without a memory fence; the empty asm statements keep
// the compiler from moving memory accesses across it
__device__ __forceinline__ void bar_nofence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Live key tiles of a workgroup: the tiles t in [t0, t1] with emax[t] > i0,
// in increasing order, written to an LDS list by all 512 threads (each wave
// scans 256 consecutive tiles, 4 per lane).  Entries are t - t0.  Returns
// the count; the list is valid after the internal barrier.  Covers at most
// kLiveWindow tiles per call (t1 - t0 < kLiveWindow).
// ---------------------------------------------------------------------------
constexpr int kLiveWindow = 2048;

__device__ __forceinline__ int build_live_list(const int32_t* __restrict__ emax_b, int t0,
                                               int t1, int i0, uint16_t* list, int* wsum) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  uint64_t m[4];
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = t0 + 256 * w + 64 * u + lane;
    const int em = emax_b[min(t, t1)];  // unconditional load: no branch around it
    const bool live = t <= t1 && em > i0;
    m[u] = __ballot(live);
    cnt += __popcll(m[u]);
  }
  if (lane == 0) wsum[w] = cnt;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int c = wsum[v];
    base += v < w ? c : 0;
    total += c;
  }
  const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if ((m[u] >> lane) & 1)
      list[base + __popcll(m[u] & below)] = static_cast<uint16_t>(256 * w + 64 * u + lane);
    base += __popcll(m[u]);
  }
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// One staged key tile: the K tile (64 rows in the padded layout above, 1088
// 16-byte slots), the V tile (1088 slots) and the tile's e record (17 slots
// used of 64).  Each DMA instruction reads from one tensor, so its address
// is a wave-uniform base plus a 32-bit lane offset.  The 34 K/V instructions
// are K_j, V_j, j = 0..16, covering slots [64 j, 64 j + 64) of their tile;
// pad slots receive a copy of a data chunk.  Wave w issues K_w, K_(w+8),
// V_w, V_(w+8), and, by w % 3, one of K_16, V_16 and the e record, which two
// or three waves then write with the same bytes: every wave issues exactly 5
// DMA loads per tile.
// ---------------------------------------------------------------------------
constexpr int kKvTileSlots = kKeyTile * 17;                 // slots per K or V tile
constexpr int kKvElems = 2 * kKeyTile * kTileRow + 512;     // bf16 elements per staged tile
constexpr int kKvDma = 5;                                   // DMA loads per wave per tile

struct KvStager {
  uint32_t rc;     // (row, chunk) of this lane's slot in K_w, K_(w+8), K_16 (10 bits each)
  int w, sel;      // sel = w % 3: 0 K_16, 1 V_16, 2 e record

  __device__ static int slot_rc(int s) {  // s: slot within a tile
    const int p = s / 17, c = s - 17 * p;
    return tile_prow(p) | (min(c, 15) << 6);
  }
  __device__ void init(int wave, int lane) {
    w = wave;
    sel = w % 3;
    rc = static_cast<uint32_t>(slot_rc(64 * w + lane)) |
            (static_cast<uint32_t>(slot_rc(64 * (w + 8) + lane)) << 10) |
            (static_cast<uint32_t>(slot_rc(1024 + lane)) << 20);
  }
  // byte offset of a slot's source row chunk (rows past N - 1 clamp to it)
  __device__ __forceinline__ static uint32_t off(uint32_t d, int lim, int tokb) {
    const int r = static_cast<int>(d & 63), c = static_cast<int>((d >> 6) & 15);
    return static_cast<uint32_t>(min(r, lim) * tokb + c * 16);
  }
  // kb, vb: token 0 of this (batch, kv head); tok: elements between tokens;
  // erb: e records of this batch
  __device__ __forceinline__ void issue(lds_bf16_t* dst, int t, const bf16_t* kb, const bf16_t* vb,
                                        int tok, const int32_t* erb, int N) const {
    const int j0 = t * kKeyTile;
    const int lim = N - 1 - j0;
    const int tokb = tok * 2;
    const char* kt = reinterpret_cast<const char*>(kb + static_cast<size_t>(j0) * tok);
    const char* vt = reinterpret_cast<const char*>(vb + static_cast<size_t>(j0) * tok);
    const uint32_t o0 = off(rc, lim, tokb), o1 = off(rc >> 10, lim, tokb);
    lds_bf16_t* const vdst = dst + kKeyTile * kTileRow;
    lds_dma16(kt + o0, dst + 64 * w * 8);
    lds_dma16(kt + o1, dst + 64 * (w + 8) * 8);
    lds_dma16(vt + o0, vdst + 64 * w * 8);
    lds_dma16(vt + o1, vdst + 64 * (w + 8) * 8);
    const uint32_t o2 = off(rc >> 20, lim, tokb);
    const uint32_t oe = static_cast<uint32_t>((lane_id() % 17) * 16);
    const char* base5 = sel == 0   ? kt
                        : sel == 1 ? vt
                                   : reinterpret_cast<const char*>(
                                         erb + static_cast<size_t>(t) * kErec);
    // one LDS base plus a selected offset keeps the target buffer visible to
    // the compiler's wait analysis
    const int d5 = sel == 0   ? 1024 * 8
                   : sel == 1 ? kKeyTile * kTileRow + 1024 * 8
                              : 2 * kKeyTile * kTileRow;
    lds_dma16(base5 + (sel == 2 ? oe : o2), dst + d5);
  }
};

// e of keys 4p .. 4p + 3 of a staged tile, and the tile's minimum e
__device__ __forceinline__ int4 staged_e4(const bf16_t* kv, int p) {
  return reinterpret_cast<const int4*>(kv + 2 * kKeyTile * kTileRow)[p];
}
__device__ __forceinline__ int staged_emin(const bf16_t* kv) {
  return reinterpret_cast<const int*>(kv + 2 * kKeyTile * kTileRow)[kKeyTile];
}

}  // namespace ksattn
