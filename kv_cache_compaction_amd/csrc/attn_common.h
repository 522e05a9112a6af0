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

}  // namespace ksattn
