// Input checks for callers that want to verify what they hand the other
// entry points.  The kernels never read outside their buffers on inputs that
// break the stated preconditions (an eviction record with e_j <= j makes the
// token invisible to every query; an invalid table entry turns that
// sequence's decode output into NaN), so these checks are a debugging aid,
// not a guard the hot path depends on.  Each writes one count per sequence
// and nothing else; one workgroup per sequence, no atomics.
#include "ks_common.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int block_sum(int x) {
  __shared__ int part[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) t += part[i];
  return t;
}

__global__ __launch_bounds__(kThreads) void check_e_kernel(const int32_t* __restrict__ e,
                                                           int N, int32_t* __restrict__ bad) {
  const int b = blockIdx.x;
  const int32_t* row = e + static_cast<size_t>(b) * N;
  int c = 0;
  for (int j = threadIdx.x; j < N; j += kThreads) c += row[j] <= j;
  c = block_sum(c);
  if (threadIdx.x == 0) bad[b] = c;
}

__global__ __launch_bounds__(kThreads) void check_table_kernel(
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens, int MB, int NB,
    int BS, int32_t* __restrict__ bad) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  const long long cap = static_cast<long long>(BS) * MB;
  const int n = L <= 0 ? 0 : static_cast<int>((min(static_cast<long long>(L), cap) + BS - 1) / BS);
  const int32_t* row = table + static_cast<size_t>(b) * MB;
  int c = 0;
  for (int x = threadIdx.x; x < n; x += kThreads)
    c += static_cast<unsigned>(row[x]) >= static_cast<unsigned>(NB);
  c = block_sum(c);
  if (threadIdx.x == 0) bad[b] = c + ((L < 0 || L > cap) ? 1 : 0);
}

}  // namespace

extern "C" ks_status ks_check_eviction_record(const int32_t* e, int B, int N, int32_t* bad,
                                              void* stream) {
  KS_REQUIRE(B >= 0 && N >= 0, "ks_check_eviction_record: B=%d N=%d", B, N);
  KS_REQUIRE(B < (1 << 30), "ks_check_eviction_record: B too large");
  if (B == 0) return KS_OK;
  KS_REQUIRE(bad && (e || N == 0), "ks_check_eviction_record: null pointer");
  hipLaunchKernelGGL(check_e_kernel, dim3(B), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), e, N, bad);
  return ks_check_launch("ks_check_eviction_record");
}

extern "C" ks_status ks_check_block_table(const int32_t* table, const int32_t* seq_lens, int B,
                                          int max_blocks, int num_pool_blocks, int block_size,
                                          int32_t* bad, void* stream) {
  KS_REQUIRE(B >= 0 && max_blocks >= 0 && num_pool_blocks >= 0,
             "ks_check_block_table: bad sizes");
  KS_REQUIRE(block_size == 1 || block_size == KS_BLOCK,
             "ks_check_block_table: block_size %d (1 or 16)", block_size);
  KS_REQUIRE(B < (1 << 30), "ks_check_block_table: B too large");
  if (B == 0) return KS_OK;
  KS_REQUIRE(bad && seq_lens && (table || max_blocks == 0), "ks_check_block_table: null pointer");
  hipLaunchKernelGGL(check_table_kernel, dim3(B), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), table, seq_lens, max_blocks,
                     num_pool_blocks, block_size, bad);
  return ks_check_launch("ks_check_block_table");
}
