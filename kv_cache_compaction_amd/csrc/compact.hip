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
  if (MB == 0) {
    if (tid == 0) nout[b] = 0;
    return;
  }
  int base = 0;
  // the first pass runs before the length is known (its loads do not depend
  // on it); later passes only while entries remain
  int c0 = 0;
  do {
    // this thread's kPer consecutive entries
    const int k0 = c0 + tid * kPer;
    int flags[kPer];
    int vals[kPer];
    int poss[kPer];
    int cnt = 0;
    // every load address is known up front: issue them all (inside the row)
    // before any of them is needed, so the pass costs one memory round trip
    int kp[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int k = min(k0 + u, MB - 1);
      kp[u] = keep[row + k];
      vals[u] = tin[row + k];
      poss[u] = pin ? pin[row + k] : 0;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const bool ok = k0 + u < n && kp[u] != 0;
      flags[u] = ok;
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
    c0 += kThreads * kPer;
  } while (c0 < n);
  for (int k = base + tid; k < MB; k += kThreads) {
    tout[row + k] = -1;
    if (pout) pout[row + k] = -1;
  }
  if (tid == 0) nout[b] = base;
}

// ---------------------------------------------------------------------------
// Several events in one launch.  Thread t owns positions 4t .. 4t + 3 of the
// current table of its sequence, so the keep flags of every event sit at
// fixed addresses: the flags of the first kPreRounds events are loaded with
// the table row, before any pass runs.  The row lives in LDS (two copies,
// written alternately) until the last event.
// ---------------------------------------------------------------------------
constexpr int kRoundBlocks = kThreads * kPer;  // 4096 entries
constexpr int kPreRounds = 8;

__device__ __forceinline__ uint32_t keep_word(const uint8_t* kr, int k0, int MB) {
  uint32_t wv = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = min(k0 + u, MB - 1);
    wv |= static_cast<uint32_t>(kr[k] != 0) << (8 * u);
  }
  return wv;
}

__global__ __launch_bounds__(kThreads) void compact_rounds_kernel(
    const int32_t* __restrict__ tin, const int32_t* __restrict__ nin,
    const uint8_t* __restrict__ keep, int rounds, int32_t* __restrict__ tout,
    int32_t* __restrict__ nout, const int32_t* __restrict__ pin,
    int32_t* __restrict__ pout, int B, int MB) {
  __shared__ int rowt[2][kRoundBlocks];
  __shared__ int rowp[2][kRoundBlocks];
  __shared__ int wsum[kWaves];
  const int b = blockIdx.x;
  const size_t row = static_cast<size_t>(b) * MB;
  const size_t rstride = static_cast<size_t>(B) * MB;  // between events' keep masks
  const int tid = threadIdx.x, w = tid >> 6;
  const int k0 = tid * kPer;
  int vals[kPer], poss[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = min(k0 + u, MB - 1);
    vals[u] = tin[row + k];
    poss[u] = pin ? pin[row + k] : 0;
  }
  uint32_t kw[kPreRounds];
#pragma unroll
  for (int r = 0; r < kPreRounds; ++r)
    kw[r] = r < rounds ? keep_word(keep + r * rstride + row, k0, MB) : 0u;
  int n = nin[b];
  n = n < 0 ? 0 : (n > MB ? MB : n);

  int cur = 0;
  for (int r = 0; r < rounds; ++r) {
    uint32_t kwr = 0;
#pragma unroll
    for (int i = 0; i < kPreRounds; ++i) kwr = i == r ? kw[i] : kwr;
    if (r >= kPreRounds) kwr = keep_word(keep + r * rstride + row, k0, MB);
    int flags[kPer];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      flags[u] = (k0 + u < n) && ((kwr >> (8 * u)) & 1u);
      cnt += flags[u];
    }
    int pre = 0, tot_w = 0;
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
      const int sw = wsum[i];
      off += (i < w) ? sw : 0;
      tot += sw;
    }
    int dst = off + pre;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (flags[u]) {
        rowt[cur][dst] = vals[u];
        rowp[cur][dst] = poss[u];
        ++dst;
      }
    }
    __syncthreads();  // the new row is complete; wsum may be rewritten
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int k = min(k0 + u, kRoundBlocks - 1);
      vals[u] = rowt[cur][k];
      poss[u] = rowp[cur][k];
    }
    n = tot;
    cur ^= 1;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = k0 + u;
    if (k < MB) {
      tout[row + k] = k < n ? vals[u] : -1;
      if (pout) pout[row + k] = k < n ? poss[u] : -1;
    }
  }
  if (tid == 0) nout[b] = n;
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

extern "C" ks_status ks_compact_block_table_rounds(const int32_t* table_in,
                                                   const int32_t* nblk_in,
                                                   const uint8_t* keep, int rounds,
                                                   int32_t* table_out, int32_t* nblk_out,
                                                   const int32_t* pos_in, int32_t* pos_out,
                                                   int B, int max_blocks, void* stream) {
  KS_REQUIRE(B >= 0 && max_blocks >= 0, "ks_compact_block_table_rounds: B=%d max_blocks=%d", B,
             max_blocks);
  KS_REQUIRE(rounds >= 0 && rounds <= KS_MAX_ROUNDS,
             "ks_compact_block_table_rounds: rounds=%d outside [0, %d]", rounds, KS_MAX_ROUNDS);
  KS_REQUIRE(max_blocks <= KS_MAX_ROUND_BLOCKS,
             "ks_compact_block_table_rounds: max_blocks=%d above %d", max_blocks,
             KS_MAX_ROUND_BLOCKS);
  if (B == 0) return KS_OK;
  KS_REQUIRE(table_in && nblk_in && table_out && nblk_out && (keep || rounds == 0),
             "ks_compact_block_table_rounds: null pointer argument");
  KS_REQUIRE((pos_in == nullptr) == (pos_out == nullptr),
             "ks_compact_block_table_rounds: pos_in and pos_out must both be set or both NULL");
  const size_t bytes = static_cast<size_t>(B) * max_blocks * sizeof(int32_t);
  auto overlap = [&](const void* a, const void* c) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(c);
    return bytes && x < y + bytes && y < x + bytes;
  };
  KS_REQUIRE(!overlap(table_in, table_out),
             "ks_compact_block_table_rounds: table_out must not alias table_in");
  if (pos_in) {
    KS_REQUIRE(!overlap(pos_in, pos_out) && !overlap(pos_out, table_out) &&
                   !overlap(pos_out, table_in),
               "ks_compact_block_table_rounds: pos_out must not alias the other tables");
  }
  if (max_blocks == 0) {  // nothing to move; lengths clamp to 0
    hipLaunchKernelGGL(compact_kernel, dim3(B), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), table_in, nblk_in, keep, table_out,
                       nblk_out, pos_in, pos_out, max_blocks);
    return ks_check_launch("ks_compact_block_table_rounds");
  }
  hipLaunchKernelGGL(compact_rounds_kernel, dim3(B), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), table_in, nblk_in, keep, rounds,
                     table_out, nblk_out, pos_in, pos_out, B, max_blocks);
  return ks_check_launch("ks_compact_block_table_rounds");
}
