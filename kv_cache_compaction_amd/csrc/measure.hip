// Measurement aids (not part of the method).
//
// mfma_rate_kernel: the bf16 MFMA rate this GPU sustains at the attention
// kernels' occupancy, as the reference beside the published dense peak.
// Each workgroup is 8 waves (2 per SIMD, the occupancy the attention kernels
// run at); every wave issues v_mfma_f32_32x32x16_bf16 back to back on four
// independent accumulators, so no MFMA waits on the one before it.  Nothing
// but MFMAs runs in the loop.
//
// dq_atomics_kernel: the dQ traffic of a single-pass backward that would
// add dQ from the dK/dV walk.  Same grid and walk as that kernel (a
// workgroup per 256 keys of one (trace, kv head), query chunks of 32 rows
// from the end of its range down, the group's query heads innermost); each
// (chunk, head) adds its 32 x 128 fp32 dQ partial with global fp32 atomic
// adds into a [B, N, Hq, 128] accumulator.  No arithmetic besides the adds,
// so its time is a lower bound on what those adds cost.
#include "ks_common.h"
#include "../../include/ks_measure.h"

namespace {

constexpr int kChains = 4;

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_rate_kernel(
    const bf16_t* __restrict__ seed, float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(seed + 8 * lane);
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(seed + 512 + 8 * lane);
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the loop alive
}

constexpr int kDqKeys = 256;  // keys per workgroup of the dK/dV walk
constexpr int kDqRows = 32;   // query rows per chunk

__global__ __launch_bounds__(512) void dq_atomics_kernel(float* __restrict__ acc,
                                                         const int32_t* __restrict__ cend,
                                                         int B, int N, int Hq, int Hkv,
                                                         int nkt) {
  const int nbh = B * Hkv;
  const int kt = blockIdx.x / nbh, bh = blockIdx.x % nbh;
  const int b = bh / Hkv, hkv = bh % Hkv, G = Hq / Hkv;
  const int c_begin = kt * kDqKeys / kDqRows;
  const int c_end = cend[static_cast<size_t>(b) * nkt + kt];
  const int nc = c_end > c_begin ? c_end - c_begin : 0;
  const int t = threadIdx.x;
  const float one = 1.0f;
  for (int idx = 0; idx < nc * G; ++idx) {
    const int c = c_end - 1 - idx / G;
    const int h = hkv * G + idx % G;
    float* base = acc + (static_cast<size_t>(b) * N + static_cast<size_t>(c) * kDqRows) * Hq * 128 +
                  static_cast<size_t>(h) * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int x = i * 512 + t;
      const int row = x >> 7, d = x & 127;
      if (c * kDqRows + row < N)
        __hip_atomic_fetch_add(base + static_cast<size_t>(row) * Hq * 128 + d, one,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

extern "C" ks_status ks_measure_dq_atomics(float* acc, const int32_t* cend, int B, int N, int Hq,
                                           int Hkv, void* stream) {
  KS_REQUIRE(B > 0 && N > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0,
             "ks_measure_dq_atomics: bad sizes");
  KS_REQUIRE(acc && cend, "ks_measure_dq_atomics: null pointer");
  const int nkt = (N + kDqKeys - 1) / kDqKeys;
  const long long grid = static_cast<long long>(B) * Hkv * nkt;
  KS_REQUIRE(grid < (1LL << 31), "ks_measure_dq_atomics: grid too large");
  hipLaunchKernelGGL(dq_atomics_kernel, dim3(static_cast<unsigned>(grid)), dim3(512), 0,
                     static_cast<hipStream_t>(stream), acc, cend, B, N, Hq, Hkv, nkt);
  return ks_check_launch("ks_measure_dq_atomics");
}

extern "C" double ks_measure_mfma_flops(int workgroups, int iters) {
  return 2.0 * 32 * 32 * 16 * 8 * kChains * static_cast<double>(iters) * 8 * workgroups;
}

extern "C" ks_status ks_measure_mfma_bf16(const void* seed, float* sink, int workgroups,
                                          int iters, void* stream) {
  KS_REQUIRE(workgroups > 0 && iters > 0, "ks_measure_mfma_bf16: bad sizes");
  KS_REQUIRE(seed && sink, "ks_measure_mfma_bf16: null pointer");
  KS_REQUIRE(ks_aligned16(seed), "ks_measure_mfma_bf16: seed must be 16-byte aligned");
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(512), 0,
                     static_cast<hipStream_t>(stream), static_cast<const bf16_t*>(seed), sink,
                     iters);
  return ks_check_launch("ks_measure_mfma_bf16");
}
