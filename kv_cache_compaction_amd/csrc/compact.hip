// Block-table compaction: splice evicted 16-token blocks out of each
// sequence's block table and join the surviving block references in order
// (KV-streams explainer, paragraph on vLLM's 16-token blocks and the block
// table: no empty slots may remain, so whole blocks are removed and the rest
// concatenated).
//
// One workgroup per sequence.  Each pass covers 4 entries per thread
// (1024 threads -> 4096 entries, one pass for every table up to 4096
// blocks).  Within a pass: a wave-wide ballot + mbcnt gives each thread its
// rank among the kept entries of its wave, wave totals are scanned in LDS,
// and kept entries are scattered to base + rank.  Tables are int32 and the
// whole row is touched once, so the kernel is bandwidth/latency bound.
#include "ks_common.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kPer = 4;  // entries per thread per pass
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int lane_rank(uint64_t mask) {
  // number of set bits of `mask` below this lane
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__global__ __launch_bounds__(kThreads) void compact_kernel(
    const int32_t* __restrict__ tin, const int32_t* __restrict__ nin,
    const uint8_t* __restrict__ keep, int32_t* __restrict__ tout,
    int32_t* __restrict__ nout, const int32_t* __restrict__ pin,
    int32_t* __restrict__ pout, int MB) {
  __shared__ int wsum[kWaves];
  const int b = blockIdx.x;
  const size_t row = static_cast<size_t>(b) * MB;
  int n = nin[b];
  n = n < 0 ? 0 : (n > MB ? MB : n);
  const int tid = threadIdx.x, w = tid >> 6;
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += kThreads * kPer) {
    // this thread's kPer consecutive entries
    const int k0 = c0 + tid * kPer;
    int flags[kPer];
    int vals[kPer];
    int poss[kPer];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int k = k0 + u;
      const bool ok = k < n && keep[row + k] != 0;
      flags[u] = ok;
      vals[u] = ok ? tin[row + k] : 0;
      poss[u] = (ok && pin) ? pin[row + k] : 0;
      cnt += ok;
    }
    // exclusive prefix of `cnt` over the workgroup: within-wave via ballots of
    // each bit of cnt (cnt <= 4 needs 3 bits), then across waves through LDS
    int pre = 0;
    int tot_w = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
      const uint64_t m = __ballot((cnt >> bit) & 1);
      pre += lane_rank(m) << bit;
      tot_w += __popcll(m) << bit;
    }
    if ((tid & 63) == 0) wsum[w] = tot_w;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int s = wsum[i];
      off += (i < w) ? s : 0;
      tot += s;
    }
    int dst = base + off + pre;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (flags[u]) {
        tout[row + dst] = vals[u];
        if (pout) pout[row + dst] = poss[u];
        ++dst;
      }
    }
    base += tot;
    __syncthreads();  // wsum reuse
  }
  for (int k = base + tid; k < MB; k += kThreads) {
    tout[row + k] = -1;
    if (pout) pout[row + k] = -1;
  }
  if (tid == 0) nout[b] = base;
}

}  // namespace

extern "C" ks_status ks_compact_block_table(const int32_t* table_in, const int32_t* nblk_in,
                                            const uint8_t* keep, int32_t* table_out,
                                            int32_t* nblk_out, const int32_t* pos_in,
                                            int32_t* pos_out, int B, int max_blocks,
                                            void* stream) {
  KS_REQUIRE(B >= 0 && max_blocks >= 0, "ks_compact_block_table: B=%d max_blocks=%d", B,
             max_blocks);
  if (B == 0) return KS_OK;
  KS_REQUIRE(table_in && nblk_in && keep && table_out && nblk_out,
             "ks_compact_block_table: null pointer argument");
  KS_REQUIRE((pos_in == nullptr) == (pos_out == nullptr),
             "ks_compact_block_table: pos_in and pos_out must both be set or both NULL");
  const size_t bytes = static_cast<size_t>(B) * max_blocks * sizeof(int32_t);
  auto overlap = [&](const void* a, const void* c) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(c);
    return bytes && x < y + bytes && y < x + bytes;
  };
  KS_REQUIRE(!overlap(table_in, table_out),
             "ks_compact_block_table: table_out must not alias table_in");
  if (pos_in) {
    KS_REQUIRE(!overlap(pos_in, pos_out) && !overlap(pos_out, table_out) &&
                   !overlap(pos_out, table_in),
               "ks_compact_block_table: pos_out must not alias the other tables");
  }
  hipLaunchKernelGGL(compact_kernel, dim3(B), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), table_in, nblk_in, keep, table_out,
                     nblk_out, pos_in, pos_out, max_blocks);
  return ks_check_launch("ks_compact_block_table");
}
