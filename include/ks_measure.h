/*
 * ks_measure.h -- measurement aid of libks.so (not part of the hot path).
 *
 * ks_measure_mfma_bf16 runs a loop of nothing but v_mfma_f32_32x32x16_bf16
 * instructions (four independent accumulators per wave) in `workgroups`
 * workgroups of 8 waves, 2 waves per SIMD -- the occupancy of the attention
 * kernels -- so that its rate, timed by the caller, is the bf16 MFMA rate
 * this GPU sustains at that occupancy and at the clock it holds under such
 * a load, next to the published dense peak.
 *
 * seed  device memory, >= 1024 bf16 values (16-byte aligned); the MFMA
 *       operands
 * sink  device memory, >= workgroups * 512 floats; receives one sum per
 *       thread so the loop is not removed
 * iters loop trips; every trip issues 32 MFMAs per wave
 * ks_measure_mfma_flops(workgroups, iters) is the flop count of one call.
 *
 * ks_measure_dq_atomics issues the dQ traffic a single-pass backward would
 * add from the dK/dV walk (every dK/dV workgroup of 256 keys adding a
 * 32 x 128 fp32 partial per 32-row query chunk and query head, with global
 * fp32 atomic adds) and nothing else, so its time, taken by the caller, is
 * a lower bound on the cost of those adds.
 * acc   device fp32 [B, N, Hq, 128] (contents are added to)
 * cend  device int32 [B, ceil(N / 256)]: one past the last 32-row chunk
 *       the keys of each 256-key tile are live for, ceil(min(N, max e) / 32)
 * Errors as for the entry points of ks.h.
 */
#ifndef KS_MEASURE_H
#define KS_MEASURE_H

#include "ks.h"

#ifdef __cplusplus
extern "C" {
#endif

double ks_measure_mfma_flops(int workgroups, int iters);
ks_status ks_measure_mfma_bf16(const void* seed, float* sink, int workgroups, int iters,
                               void* stream);
ks_status ks_measure_dq_atomics(float* acc, const int32_t* cend, int B, int N, int Hq, int Hkv,
                                void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KS_MEASURE_H */
