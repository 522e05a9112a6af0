// Internal helpers shared by the libks kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ks.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;  // storage type of one bf16 value

// ---------------------------------------------------------------------------
// host-side error plumbing (defined in ks_api.cpp)
// ---------------------------------------------------------------------------
ks_status ks_fail(ks_status st, const char* fmt, ...);
ks_status ks_check_launch(const char* what);

// RoPE preparation of the fused attention entry points (rope.hip): the
// (cos, sin) table of every token's logical position ([B*N][D/2] float2)
// and, when k_raw is non-null, the keys rotated out of place into k_rot
size_t rope_table_bytes(int B, int N, int D);
ks_status launch_rope_prep(const uint16_t* k_raw, uint16_t* k_rot, const int32_t* pos,
                           float2* table, long long ntok, int Hkv, int D, float base,
                           hipStream_t s);

#define KS_REQUIRE(cond, ...)                                  \
  do {                                                         \
    if (!(cond)) return ks_fail(KS_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

static inline bool ks_aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Query heads per wave in the GQA kernels: the largest of 4, 2, 1 that
// divides the group size G = Hq / Hkv, so the heads of one wave always share
// one kv head (the kernels are instantiated for these three values only).
static inline int ks_heads_per_wave(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fp32 -> bf16, round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

// two fp32 -> packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// RoPE at logical position (rotate-half pairing of k and k + D/2): the angle
// theta = pos * base^(-2k/D) is formed and reduced in fp64 (positions reach
// the tens of thousands, where an fp32 angle is off by ~1e-3 rad), then the
// pair rotates in fp32.  Every kernel that rotates uses these two helpers,
// so a key or query rotated by any of them is bit-identical.
__device__ __forceinline__ float2 rope_cos_sin(double pos, int k, int D, double log2_base,
                                               bool inverse = false) {
  const double inv_freq = exp2(-2.0 * k / D * log2_base);
  double theta = pos * inv_freq;
  if (inverse) theta = -theta;
  double s, c;
  sincos(theta, &s, &c);
  return make_float2(static_cast<float>(c), static_cast<float>(s));
}
// (x, y) = (x[k], x[k + D/2]) -> (x cos - y sin, y cos + x sin)
__device__ __forceinline__ void rope_rotate(float& x, float& y, float2 cs) {
  const float xr = __builtin_fmaf(x, cs.x, -(y * cs.y));
  const float yr = __builtin_fmaf(y, cs.x, x * cs.y);
  x = xr;
  y = yr;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// lane index within the 64-wide wavefront
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

static constexpr float KS_LOG2E = 1.4426950408889634f;
static constexpr float KS_LN2 = 0.6931471805599453f;
