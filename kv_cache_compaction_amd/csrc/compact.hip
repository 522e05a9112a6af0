// Block-table compaction: splice evicted 16-token blocks out of each
// sequence's block table and join the surviving block references in order
// (KV-streams explainer, paragraph on vLLM's 16-token blocks and the block
// table: no empty slots may remain, so whole blocks are removed and the rest
// concatenated).
//
// One workgroup per sequence for rows of up to 4096 entries (4 entries per
// thread, 1024 threads: one pass); longer rows get one workgroup per
// 4096-entry chunk (below).  Within a pass: a wave-wide ballot + mbcnt gives each thread its
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

// Rows whose length is a multiple of 16 entries, on 16-byte aligned tables:
// one workgroup per row of up to 4096 entries, one pass, 256 threads x 16
// consecutive entries read with four 16-byte loads (and the keep flags with
// one).  Kept entries are placed at their ranks in LDS and the row (kept
// entries, then -1) is written out with 16-byte stores, each store
// instruction covering 1 KB of the row.  Other rows take compact_kernel.
constexpr int kCThreads = 256;
constexpr int kCPer = 16;
constexpr int kCWaves = kCThreads / 64;
constexpr int kCRow = kCThreads * kCPer;   // 4096 entries

__global__ __launch_bounds__(kCThreads) void compact_vec_kernel(
    const int32_t* __restrict__ tin, const int32_t* __restrict__ nin,
    const uint8_t* __restrict__ keep, int32_t* __restrict__ tout,
    int32_t* __restrict__ nout, const int32_t* __restrict__ pin,
    int32_t* __restrict__ pout, int MB) {
  __shared__ int wsum[kCWaves];
  __shared__ __attribute__((aligned(16))) int stage[kCRow];
  const int b = blockIdx.x;
  const size_t row = static_cast<size_t>(b) * MB;
  const int tid = threadIdx.x, w = tid >> 6;
  if (MB == 0) {
    if (tid == 0) nout[b] = 0;
    return;
  }
  // the loads do not depend on the length: they go out with its load
  const int k0 = tid * kCPer;
  int vals[kCPer];
  uint32_t kw[kCPer / 4];  // keep flags, one byte each, four per word
  const bool vec = k0 + kCPer <= MB;  // threads past the row end read nothing
  if (vec) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(keep + row + k0);
    kw[0] = kv[0];
    kw[1] = kv[1];
    kw[2] = kv[2];
    kw[3] = kv[3];
#pragma unroll
    for (int qd = 0; qd < kCPer / 4; ++qd) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(tin + row + k0 + 4 * qd);
#pragma unroll
      for (int c = 0; c < 4; ++c) vals[4 * qd + c] = static_cast<int>(t[c]);
    }
  } else {
#pragma unroll
    for (int qd = 0; qd < kCPer / 4; ++qd) kw[qd] = 0u;
#pragma unroll
    for (int u = 0; u < kCPer; ++u) vals[u] = 0;
  }
  int n = nin[b];
  n = n < 0 ? 0 : (n > MB ? MB : n);
  uint32_t fl = 0;
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kCPer; ++u) {
    const bool ok = k0 + u < n && ((kw[u >> 2] >> (8 * (u & 3))) & 0xffu) != 0;
    fl |= static_cast<uint32_t>(ok) << u;
    cnt += ok;
  }
  // exclusive prefix of `cnt` over the workgroup: within-wave via ballots of
  // each bit of cnt (cnt <= 16 needs 5 bits), then across waves through LDS
  int pre = 0;
  int tot_w = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t m = __ballot((cnt >> bit) & 1);
    pre += lane_rank(m) << bit;
    tot_w += __popcll(m) << bit;
  }
  if ((tid & 63) == 0) wsum[w] = tot_w;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kCWaves; ++i) {
    const int s = wsum[i];
    off += (i < w) ? s : 0;
    tot += s;
  }
  // the kept entries at their ranks, then the whole row written out in order
  auto place_and_write = [&](const int* v, int32_t* dst_row) {
    int d = off + pre;
#pragma unroll
    for (int u = 0; u < kCPer; ++u)
      if ((fl >> u) & 1u) stage[d++] = v[u];
    __syncthreads();
    // thread t writes entries 4 t + 1024 q .. + 3
#pragma unroll
    for (int qd = 0; qd < kCPer / 4; ++qd) {
      const int x = 4 * tid + kCThreads * 4 * qd;
      if (x < MB) {
        u32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          o[c] = static_cast<uint32_t>(x + c < tot ? stage[x + c] : -1);
        *reinterpret_cast<u32x4*>(dst_row + x) = o;
      }
    }
  };
  place_and_write(vals, tout + row);
  if (pout) {
    // positions follow the same selection, through the same staging buffer
    __syncthreads();
    int pv[kCPer];
    if (vec) {
#pragma unroll
      for (int qd = 0; qd < kCPer / 4; ++qd) {
        const u32x4 p = *reinterpret_cast<const u32x4*>(pin + row + k0 + 4 * qd);
#pragma unroll
        for (int c = 0; c < 4; ++c) pv[4 * qd + c] = static_cast<int>(p[c]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kCPer; ++u) pv[u] = 0;
    }
    place_and_write(pv, pout + row);
  }
  if (tid == 0) nout[b] = tot;
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

// ---------------------------------------------------------------------------
// Rows longer than one pass (token tables of single-token blocks reach tens
// of thousands of entries): one workgroup per 4096-entry chunk, so a long
// row is spread over the chip instead of looping in one workgroup.  Each
// workgroup counts the kept entries before its chunk and in the whole row
// from the keep flags (one byte per entry, read by every chunk of the row
// and so served from L2), then compacts its own chunk at that offset and
// fills the part of [kept, MB) that falls in its chunk with -1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// kept entries among [0, n) of a keep row: all of them, and those before c0
// (both summed over the workgroup; every thread gets the sums)
__device__ __forceinline__ void count_kept(const uint8_t* __restrict__ kr, int n, int c0,
                                           int* red, int& before, int& all) {
  const int tid = threadIdx.x, w = tid >> 6;
  int cb = 0, ca = 0;
  for (int k = tid * kPer; k < n; k += kThreads * kPer) {
    int f[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) f[u] = kr[min(k + u, n - 1)] != 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int ok = (k + u < n) & f[u];
      ca += ok;
      cb += (k + u < c0) ? ok : 0;
    }
  }
  cb = wave_sum(cb);
  ca = wave_sum(ca);
  if ((tid & 63) == 0) {
    red[w] = cb;
    red[kWaves + w] = ca;
  }
  __syncthreads();
  before = 0;
  all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    before += red[i];
    all += red[kWaves + i];
  }
}

__global__ __launch_bounds__(kThreads) void compact_chunk_kernel(
    const int32_t* __restrict__ tin, const int32_t* __restrict__ nin,
    const uint8_t* __restrict__ keep, int32_t* __restrict__ tout,
    int32_t* __restrict__ nout, const int32_t* __restrict__ pin,
    int32_t* __restrict__ pout, int MB, int write_n) {
  __shared__ int wsum[kWaves];
  __shared__ int red[2 * kWaves];
  const int c = blockIdx.x, b = blockIdx.y;
  const size_t row = static_cast<size_t>(b) * MB;
  int n = nin[b];
  n = n < 0 ? 0 : (n > MB ? MB : n);
  const int tid = threadIdx.x, w = tid >> 6;
  const int c0 = c * kRoundBlocks;
  const int k0 = c0 + tid * kPer;
  // this chunk's entries: the addresses do not depend on the counts
  int kp[kPer], vals[kPer], poss[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = min(k0 + u, MB - 1);
    kp[u] = keep[row + k];
    vals[u] = tin[row + k];
    poss[u] = pin ? pin[row + k] : 0;
  }
  int before, all;
  count_kept(keep + row, n, c0, red, before, all);
  int flags[kPer];
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    flags[u] = k0 + u < n && kp[u] != 0;
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
  int off = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) off += (i < w) ? wsum[i] : 0;
  int dst = before + off + pre;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (flags[u]) {
      tout[row + dst] = vals[u];
      if (pout) pout[row + dst] = poss[u];
      ++dst;
    }
  }
  const int c1 = min(c0 + kRoundBlocks, MB);
  for (int k = max(c0, all) + tid; k < c1; k += kThreads) {
    tout[row + k] = -1;
    if (pout) pout[row + k] = -1;
  }
  if (write_n && c == 0 && tid == 0) nout[b] = all;
}

// lengths after compaction, for the case nblk_out aliases nblk_in (the chunk
// kernel's workgroups all read nblk_in, so none of them may overwrite it)
__global__ __launch_bounds__(kThreads) void count_kept_kernel(
    const int32_t* __restrict__ nin, const uint8_t* __restrict__ keep,
    int32_t* __restrict__ nout, int MB) {
  __shared__ int red[2 * kWaves];
  const int b = blockIdx.x;
  int n = nin[b];
  n = n < 0 ? 0 : (n > MB ? MB : n);
  int before, all;
  count_kept(keep + static_cast<size_t>(b) * MB, n, 0, red, before, all);
  if (threadIdx.x == 0) nout[b] = all;
}

// ---------------------------------------------------------------------------
// Several events on rows longer than 4096 entries (token tables): the row
// does not fit on chip, but which of its entries survive does.  Thread t
// owns entries [64 t, 64 t + 64) of the original row as one 64-bit word of
// survival bits.  The alive entries of a word sit at consecutive positions
// [base, base + cnt) of the table an event applies to (base: a workgroup
// scan of the per-word counts), so their keep flags are one 64-bit window
// of the event's flags packed into bits in LDS; the window is deposited onto
// the word's set bits (directly when it keeps or drops all of them, which
// is every word away from an evicted run's ends).  kRowSplit workgroups per
// row replay the events (one bit per entry: cheap) and each writes a
// quarter of the compacted row, so the row's reads and writes spread over
// four times as many compute units.
// ---------------------------------------------------------------------------
constexpr int kLongBits = 64;                        // entries per thread
constexpr int kLongMax = kThreads * kLongBits;       // 65536 entries
constexpr int kRowSplit = 4;                         // workgroups per row

// exclusive prefix of v over the workgroup's threads (in thread order); the
// total goes to `total`.  Contains one barrier.
__device__ __forceinline__ int block_scan(int v, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    x += lane >= o ? y : 0;
  }
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int sw = wtot[i];
    off += i < w ? sw : 0;
    tot += sw;
  }
  total = tot;
  return off + x - v;
}

// The 16-byte chunks that hold flags [64 t, 64 t + 64) of one keep row, read
// at aligned addresses clamped to the chunks that hold bytes of the row (so
// no load leaves the pages the row lives on).  Issued one event ahead.
struct KeepChunks {
  u32x4 c[5];
  int shift;  // bytes from the first chunk to flag 64 t
};

__device__ __forceinline__ void keep_issue(const uint8_t* krow, int MB, int t, KeepChunks& k) {
  const uintptr_t row = reinterpret_cast<uintptr_t>(krow);
  const uintptr_t last = (row + static_cast<uintptr_t>(MB) - 1) & ~static_cast<uintptr_t>(15);
  const uintptr_t a0 = (row + static_cast<uintptr_t>(64) * t) & ~static_cast<uintptr_t>(15);
  k.shift = static_cast<int>(row + static_cast<uintptr_t>(64) * t - a0);
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const uintptr_t a = a0 + 16 * u < last ? a0 + 16 * u : last;
    k.c[u] = *reinterpret_cast<const u32x4*>(a);
  }
}

// four flag bytes -> four bits (bit i set iff byte i is nonzero)
__device__ __forceinline__ uint32_t nz_nibble(uint32_t x) {
  const uint32_t nz = (((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;
  return ((nz >> 7) | (nz >> 14) | (nz >> 21) | (nz >> 28)) & 0xfu;
}

// flags [64 t, 64 t + 64) as bits; flags at or past `len` read as 0
__device__ __forceinline__ uint64_t keep_bits(const KeepChunks& k, int t, int len) {
  uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 20; ++i) w[i / 8] |= nz_nibble(k.c[i / 4][i % 4]) << (4 * (i % 8));
  // bit offset = byte offset (one bit per flag byte)
  const uint32_t lo = __builtin_amdgcn_alignbit(w[1], w[0], k.shift);
  const uint32_t hi = __builtin_amdgcn_alignbit(w[2], w[1], k.shift);
  uint64_t bits = (static_cast<uint64_t>(hi) << 32) | lo;
  const int valid = len - 64 * t;
  if (valid < 64) bits = valid <= 0 ? 0 : bits & ((uint64_t(1) << valid) - 1);
  return bits;
}

__device__ __forceinline__ uint64_t low_bits(int n) {
  return n >= 64 ? ~uint64_t(0) : (uint64_t(1) << n) - 1;
}

// bit i of `src` placed on the i-th set bit of `mask`
__device__ __forceinline__ uint64_t deposit(uint64_t src, uint64_t mask) {
  uint64_t out = 0;
  while (mask) {
    const uint64_t low = mask & (~mask + 1);
    if (src & 1) out |= low;
    src >>= 1;
    mask &= mask - 1;
  }
  return out;
}

__global__ __launch_bounds__(kThreads) void compact_rounds_long_kernel(
    const int32_t* __restrict__ tin, const int32_t* __restrict__ nin,
    const uint8_t* __restrict__ keep, int rounds, int32_t* __restrict__ tout,
    int32_t* __restrict__ nout, const int32_t* __restrict__ pin,
    int32_t* __restrict__ pout, int B, int MB, int split) {
  __shared__ uint64_t kbits[kThreads + 1];   // one event's flags, by table position
  __shared__ uint64_t fword[kThreads];       // survival words after the last event
  __shared__ int fbase[kThreads];            // output position of each word's first entry
  __shared__ int wtot[kWaves];
  // the row's workgroups are B apart in the grid, so with B a multiple of 8
  // they run on one XCD and its L2 serves the keep rows they all read
  const int b = blockIdx.x % B, part = blockIdx.x / B;
  const int tid = threadIdx.x;
  const size_t row = static_cast<size_t>(b) * MB;
  const size_t rstride = static_cast<size_t>(B) * MB;
  int n = nin[b];
  n = n < 0 ? 0 : (n > MB ? MB : n);
  const int e0 = 64 * tid;
  uint64_t word = e0 >= n ? 0 : low_bits(n - e0);
  if (tid == 0) kbits[kThreads] = 0;

  KeepChunks kc;
  if (rounds > 0) keep_issue(keep + row, MB, tid, kc);
  for (int r = 0; r < rounds; ++r) {
    const int cnt = __popcll(word);
    int len;  // entries of the table this event applies to
    const int base = block_scan(cnt, wtot, len);
    // the event's flags as bits (only positions inside that table are ever
    // consulted: every window below lies in [0, len))
    if (64 * tid < len) kbits[tid] = keep_bits(kc, tid, MB);
    // the next event's flags: in flight while this one is applied
    if (r + 1 < rounds) keep_issue(keep + (r + 1) * rstride + row, MB, tid, kc);
    __syncthreads();
    if (cnt) {
      const int q = base >> 6, sh = base & 63;
      uint64_t km = kbits[q] >> sh;
      if (sh) km |= kbits[q + 1] << (64 - sh);
      km &= low_bits(cnt);
      if (km == 0)
        word = 0;
      else if (km != low_bits(cnt))
        word = deposit(km, word);
    }
    __syncthreads();  // kbits is rewritten by the next event
  }

  int total;
  const int base = block_scan(__popcll(word), wtot, total);
  fword[tid] = word;
  fbase[tid] = base;
  __syncthreads();
  // this workgroup's share of the row: entries [e_lo, e_hi), 16 per thread
  // per pass, loads (clamped into the row) all in flight before the stores
  const int words = (MB + kLongBits - 1) / kLongBits;
  const int sw = (words + split - 1) / split;
  const int e_lo = part * sw * kLongBits, e_hi = min(MB, e_lo + sw * kLongBits);
#pragma unroll 1
  for (int c0 = e_lo; c0 < e_hi; c0 += 16 * kThreads) {
    int dst[16], v[16], pv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = c0 + tid + kThreads * j;
      const int ec = min(e, MB - 1);
      const uint64_t fw = e < e_hi ? fword[ec >> 6] : 0;
      const int bit = ec & 63;
      dst[j] = (fw >> bit) & 1 ? fbase[ec >> 6] + __popcll(fw & ((uint64_t(1) << bit) - 1)) : -1;
      v[j] = tin[row + ec];
      pv[j] = pin ? pin[row + ec] : 0;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (dst[j] >= 0) {
        tout[row + dst[j]] = v[j];
        if (pout) pout[row + dst[j]] = pv[j];
      }
    }
  }
  // the tail [total, MB) is -1, split between the row's workgroups
  const int tail = MB - total;
  const int per = (tail + split - 1) / split;
  const int t0 = total + part * per, t1 = min(MB, t0 + per);
  for (int k = t0 + tid; k < t1; k += kThreads) {
    tout[row + k] = -1;
    if (pout) pout[row + k] = -1;
  }
  if (part == 0 && tid == 0) nout[b] = total;
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
  // rows of zero entries: only the lengths are read and written
  KS_REQUIRE(nblk_in && nblk_out && (max_blocks == 0 || (table_in && keep && table_out)),
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_blocks <= kRoundBlocks) {
    // whole rows by 16-byte loads and stores when every row starts aligned
    const bool vec = max_blocks % kCPer == 0 && ks_aligned16(table_in) && ks_aligned16(keep) &&
                     ks_aligned16(table_out) && (!pos_in || ks_aligned16(pos_in)) &&
                     (!pos_out || ks_aligned16(pos_out));
    if (vec)
      hipLaunchKernelGGL(compact_vec_kernel, dim3(B), dim3(kCThreads), 0, s, table_in, nblk_in,
                         keep, table_out, nblk_out, pos_in, pos_out, max_blocks);
    else
      hipLaunchKernelGGL(compact_kernel, dim3(B), dim3(kThreads), 0, s, table_in, nblk_in, keep,
                         table_out, nblk_out, pos_in, pos_out, max_blocks);
    return ks_check_launch("ks_compact_block_table");
  }
  KS_REQUIRE(B < 65536, "ks_compact_block_table: B=%d too large for rows above %d entries", B,
             kRoundBlocks);
  const int nchunks = (max_blocks + kRoundBlocks - 1) / kRoundBlocks;
  const bool n_alias = nblk_in == nblk_out;
  hipLaunchKernelGGL(compact_chunk_kernel, dim3(nchunks, B), dim3(kThreads), 0, s, table_in,
                     nblk_in, keep, table_out, nblk_out, pos_in, pos_out, max_blocks,
                     n_alias ? 0 : 1);
  ks_status st = ks_check_launch("ks_compact_block_table");
  if (st != KS_OK || !n_alias) return st;
  hipLaunchKernelGGL(count_kept_kernel, dim3(B), dim3(kThreads), 0, s, nblk_in, keep, nblk_out,
                     max_blocks);
  return ks_check_launch("ks_compact_block_table(count)");
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
  KS_REQUIRE(nblk_in && nblk_out &&
                 (max_blocks == 0 || (table_in && table_out && (keep || rounds == 0))),
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
  static_assert(kLongMax == KS_MAX_ROUND_BLOCKS, "round limit");
  if (max_blocks <= kRoundBlocks)
    hipLaunchKernelGGL(compact_rounds_kernel, dim3(B), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), table_in, nblk_in, keep, rounds,
                       table_out, nblk_out, pos_in, pos_out, B, max_blocks);
  else {
    // several workgroups per row, unless the lengths are updated in place
    // (every workgroup reads nblk_in; only one may then exist per row)
    const int split = nblk_in == nblk_out ? 1 : kRowSplit;
    KS_REQUIRE(static_cast<int64_t>(B) * split < (int64_t{1} << 31),
               "ks_compact_block_table_rounds: grid too large");
    hipLaunchKernelGGL(compact_rounds_long_kernel, dim3(B * split), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), table_in, nblk_in, keep, rounds,
                       table_out, nblk_out, pos_in, pos_out, B, max_blocks, split);
  }
  return ks_check_launch("ks_compact_block_table_rounds");
}
