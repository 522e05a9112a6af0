// RoPE at logical position, in place on Q and K.
//
// KV-streams keeps physical storage and logical position apart: a retained
// key keeps the rotation of its original position wherever it is stored, and
// new queries and keys continue the original count (KV-streams explainer on
// wqu.guru, paragraph on RoPE after compaction).  The caller passes the
// logical position of every token; this kernel only rotates.
//
// A workgroup handles kTok tokens.  The angles theta_k = pos * base^(-2k/D)
// are formed in fp64 (positions reach 65,792, where an fp32 angle would be off
// by ~4e-3 rad), reduced by the device library's fp64 sincos (rope_cos_sin)
// and kept in LDS as fp32 pairs, shared by every head of the token.  Each thread then rotates
// vector chunks of (x[k], x[k + D/2]): 8 bf16 or 4 fp32 per half.  The pass
// streams Q and K once (read + write), so it is HBM bound.
#include "ks_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 4;
constexpr int kMaxHalf = 128;

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int n = 4;
  typedef f32x4 type;
};
template <>
struct Vec<bf16_t> {
  static constexpr int n = 8;
  typedef u32x4 type;
};

__device__ __forceinline__ void rot_chunk(f32x4& a, f32x4& b, const float2* cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = a[i], y = b[i];
    rope_rotate(x, y, cs[i]);
    a[i] = x;
    b[i] = y;
  }
}

__device__ __forceinline__ void rot_chunk(u32x4& a, u32x4& b, const float2* cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x0 = lo_bf16(a[i]), x1 = hi_bf16(a[i]);
    float y0 = lo_bf16(b[i]), y1 = hi_bf16(b[i]);
    rope_rotate(x0, y0, cs[2 * i]);
    rope_rotate(x1, y1, cs[2 * i + 1]);
    a[i] = pack_bf16x2(x0, x1);
    b[i] = pack_bf16x2(y0, y1);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(T* __restrict__ q, T* __restrict__ k,
                                                         const int32_t* __restrict__ pos,
                                                         long long ntok, int Hq, int Hkv,
                                                         int D, double log2_base, int inverse) {
  constexpr int V = Vec<T>::n;
  typedef typename Vec<T>::type VT;
  __shared__ float2 cs[kTok][kMaxHalf];
  const int half = D >> 1;
  const long long t0 = static_cast<long long>(blockIdx.x) * kTok;
  for (int idx = threadIdx.x; idx < kTok * half; idx += kThreads) {
    const int tt = idx / half, kk = idx - tt * half;
    const long long t = t0 + tt;
    if (t < ntok)
      cs[tt][kk] = rope_cos_sin(static_cast<double>(pos[t]), kk, D, log2_base, inverse != 0);
  }
  __syncthreads();
  const int cpr = half / V;  // chunks per head
  const int nq = q ? Hq : 0, nk = k ? Hkv : 0;
  const int per_tok = (nq + nk) * cpr;
  for (int idx = threadIdx.x; idx < kTok * per_tok; idx += kThreads) {
    const int tt = idx / per_tok;
    const int r = idx - tt * per_tok;
    const long long t = t0 + tt;
    if (t >= ntok) continue;
    const int hh = r / cpr, ch = r - hh * cpr;
    T* base = (hh < nq) ? q + (t * Hq + hh) * static_cast<long long>(D)
                        : k + (t * Hkv + (hh - nq)) * static_cast<long long>(D);
    VT* pa = reinterpret_cast<VT*>(base + ch * V);
    VT* pb = reinterpret_cast<VT*>(base + half + ch * V);
    VT a = *pa, b = *pb;
    rot_chunk(a, b, &cs[tt][ch * V]);
    *pa = a;
    *pb = b;
  }
}

// Preparation of the RoPE-fused attention (bf16): per token, the (cos, sin)
// pairs of its logical position go to `table` ([ntok][D/2] float2) and, when
// k_raw is given, every kv head of its key is rotated out of place into k_rot.
// The pairs are rope_cos_sin's, so a row rotated with them is bit-identical
// to ks_rope_logical's.
__global__ __launch_bounds__(kThreads) void rope_prep_kernel(
    const bf16_t* __restrict__ k_raw, bf16_t* __restrict__ k_rot, const int32_t* __restrict__ pos,
    float2* __restrict__ table, long long ntok, int Hkv, int D, double log2_base) {
  typedef u32x4 VT;
  constexpr int V = 8;
  __shared__ float2 cs[kTok][kMaxHalf];
  const int half = D >> 1;
  const long long t0 = static_cast<long long>(blockIdx.x) * kTok;
  for (int idx = threadIdx.x; idx < kTok * half; idx += kThreads) {
    const int tt = idx / half, kk = idx - tt * half;
    const long long t = t0 + tt;
    if (t < ntok) {
      const float2 c = rope_cos_sin(static_cast<double>(pos[t]), kk, D, log2_base);
      cs[tt][kk] = c;
      table[t * half + kk] = c;
    }
  }
  if (!k_raw) return;
  __syncthreads();
  const int cpr = half / V;  // chunks per head
  const int per_tok = Hkv * cpr;
  for (int idx = threadIdx.x; idx < kTok * per_tok; idx += kThreads) {
    const int tt = idx / per_tok;
    const int r = idx - tt * per_tok;
    const long long t = t0 + tt;
    if (t >= ntok) continue;
    const int hh = r / cpr, ch = r - hh * cpr;
    const long long off = (t * Hkv + hh) * static_cast<long long>(D) + ch * V;
    VT a = *reinterpret_cast<const VT*>(k_raw + off);
    VT b = *reinterpret_cast<const VT*>(k_raw + off + half);
    rot_chunk(a, b, &cs[tt][ch * V]);
    *reinterpret_cast<VT*>(k_rot + off) = a;
    *reinterpret_cast<VT*>(k_rot + off + half) = b;
  }
}

}  // namespace

size_t rope_table_bytes(int B, int N, int D) {
  return (static_cast<size_t>(B) * N * (D / 2) * sizeof(float2) + 255) &
         ~static_cast<size_t>(255);
}

ks_status launch_rope_prep(const bf16_t* k_raw, bf16_t* k_rot, const int32_t* pos,
                           float2* table, long long ntok, int Hkv, int D, float base,
                           hipStream_t s) {
  const long long nblocks = (ntok + kTok - 1) / kTok;
  if (nblocks >= (1LL << 31)) return ks_fail(KS_ERR_INVALID_ARG, "RoPE preparation: too many tokens");
  hipLaunchKernelGGL(rope_prep_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s,
                     k_raw, k_rot, pos, table, ntok, Hkv, D, log2(static_cast<double>(base)));
  return ks_check_launch("RoPE preparation");
}

extern "C" ks_status ks_rope_logical(void* q, void* k, const int32_t* pos, int B, int N, int Hq,
                                     int Hkv, int D, int dtype, float base, int inverse,
                                     void* stream) {
  KS_REQUIRE(B >= 0 && N >= 0 && Hq >= 0 && Hkv >= 0, "ks_rope_logical: negative size");
  KS_REQUIRE(dtype == KS_F32 || dtype == KS_BF16, "ks_rope_logical: dtype %d", dtype);
  KS_REQUIRE(D >= 16 && D <= 2 * kMaxHalf && D % 16 == 0, "ks_rope_logical: D=%d unsupported",
             D);
  KS_REQUIRE(base > 1.0f, "ks_rope_logical: base must be > 1");
  const long long ntok = static_cast<long long>(B) * N;
  if (ntok == 0 || (Hq == 0 && Hkv == 0) || (!q && !k)) return KS_OK;
  KS_REQUIRE(pos, "ks_rope_logical: pos is NULL");
  KS_REQUIRE((!q || ks_aligned16(q)) && (!k || ks_aligned16(k)),
             "ks_rope_logical: q/k must be 16-byte aligned");
  const long long nblocks = (ntok + kTok - 1) / kTok;
  KS_REQUIRE(nblocks < (1LL << 31), "ks_rope_logical: too many tokens");
  const double log2_base = log2(static_cast<double>(base));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == KS_F32)
    hipLaunchKernelGGL(rope_kernel<float>, dim3(nblocks), dim3(kThreads), 0, s,
                       static_cast<float*>(q), static_cast<float*>(k), pos, ntok,
                       Hq, Hkv, D, log2_base, inverse);
  else
    hipLaunchKernelGGL(rope_kernel<bf16_t>, dim3(nblocks), dim3(kThreads), 0, s,
                       static_cast<bf16_t*>(q), static_cast<bf16_t*>(k), pos, ntok, Hq, Hkv, D,
                       log2_base, inverse);
  return ks_check_launch("ks_rope_logical");
}
