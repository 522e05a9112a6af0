// Measurement aid (not part of the method): the bf16 MFMA rate this GPU
// sustains at the attention kernels' occupancy, as the reference beside the
// published dense peak.  Each workgroup is 8 waves (2 per SIMD, the
// occupancy the attention kernels run at); every wave issues
// v_mfma_f32_32x32x16_bf16 back to back on four independent accumulators,
// so no MFMA waits on the one before it.  Nothing but MFMAs runs in the loop.
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

}  // namespace

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
