// Eviction-masked attention forward over a continuous rollout trace.
//
// The trainer replays compaction as a mask: query i attends key j iff
// j <= i < e_j, e_j being the trace index of the event that evicted j
// (KV-streams explainer, trainer paragraph; paper page, Fig. 2A).  Surviving
// keys are the ones computed during generation simply because K and V are
// those of the continuous trace.
//
// Two kernels:
//   fwd_bf16_kernel  bf16 inputs, fp32 accumulation, 32x32x16 bf16 MFMA.
//   fwd_f32_kernel   fp32 inputs and arithmetic on the VALU (small traces).
//
// bf16 kernel layout (gfx950, wave64):
//   * a workgroup = 4 waves = 64*RS query rows x HPW query heads of one kv
//     head (HPW * RS = 4); each wave owns 64 rows of one head (two 32-row
//     MFMA blocks), so every K/V fragment read from LDS feeds two MFMAs;
//   * key tiles of 64 keys are staged in LDS, double buffered, K as [key][d]
//     and V transposed to [d][key], both XOR-swizzled for conflict-free
//     16-byte fragment reads;
//   * S^T = K Q^T puts one query per lane column, so the softmax statistics
//     of a query live in one lane pair (l, l ^ 32) and P^T feeds
//     O^T += V^T P^T straight from registers;
//   * the running maximum is updated lazily (only when a tile's maximum
//     exceeds it by 2^kTau), which removes almost every O rescale;
//   * key tiles no row of the workgroup can see are skipped with the per-tile
//     max of e (a wave ballot over 64 tiles at a time); tiles every row sees
//     in full skip the element-wise mask;
//   * the 1-D grid is remapped so that consecutive query tiles of one head
//     run on the same XCD and share its L2.
#include "attn_common.h"

namespace ksattn {

// ---------------------------------------------------------------------------
// per-key-tile summary of e
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void tile_summary_kernel(const int32_t* __restrict__ e,
                                                          TileSummary ts, int N, int ntiles) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int j = t * kKeyTile + threadIdx.x;
  const bool ok = j < N;
  const int x = ok ? e[static_cast<size_t>(b) * N + j] : 0;
  int32_t* rec = ts.erec + (static_cast<size_t>(b) * ntiles + t) * kErec;
  rec[threadIdx.x] = x;
  int mn = ok ? x : 0x7fffffff;
  int mx = ok ? x : static_cast<int>(0x80000000);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, __shfl_xor(mn, off));
    mx = max(mx, __shfl_xor(mx, off));
  }
  if (threadIdx.x < 4) rec[kKeyTile + threadIdx.x] = threadIdx.x == 0 ? mn : threadIdx.x == 1 ? mx : 0;
  if (threadIdx.x == 0) {
    const size_t i = static_cast<size_t>(b) * ntiles + t;
    ts.emin[i] = mn;
    ts.emax[i] = mx;
  }
}

size_t summary_bytes(int B, int N) {
  const size_t nt = (static_cast<size_t>(N) + kKeyTile - 1) / kKeyTile;
  const size_t bt = static_cast<size_t>(B) * nt;
  return (bt * (kErec + 2) * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}

ks_status launch_summary(const int32_t* e, void* ws, int B, int N, hipStream_t s,
                         TileSummary* ts) {
  const int nt = (N + kKeyTile - 1) / kKeyTile;
  const size_t bt = static_cast<size_t>(B) * nt;
  // 16-byte aligned records first, then the plain minima and maxima
  ts->erec = static_cast<int32_t*>(ws);
  ts->emin = ts->erec + bt * kErec;
  ts->emax = ts->emin + bt;
  hipLaunchKernelGGL(tile_summary_kernel, dim3(nt, B), dim3(64), 0, s, e, *ts, N, nt);
  return ks_check_launch("eviction-mask tile summary");
}

namespace {

constexpr float kTau = 8.0f;  // lazy-rescale slack (log2 units)

// ---------------------------------------------------------------------------
// fp32 forward (VALU): one wave per 64 query rows of one head
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(64) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ e, const int32_t* __restrict__ emin,
    const int32_t* __restrict__ emax, float* __restrict__ o, float* __restrict__ lse, int N,
    int Hq, int Hkv, int ntiles, float sl2) {
  constexpr int T = kKeyTile;
  constexpr int C = 16;  // keys per softmax chunk
  __shared__ float Ks[T][DH];
  __shared__ float Vs[T][DH];
  __shared__ int Es[T];
  const int qt = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int hkv = hq / (Hq / Hkv);
  const int lane = threadIdx.x;
  const int i0 = qt * T, i = i0 + lane;
  const int i1 = min(N, i0 + T);
  const bool rv = i < N;
  float qr[DH], acc[DH];
  {
    const float* qp = q + ((static_cast<size_t>(b) * N + (rv ? i : 0)) * Hq + hq) * DH;
#pragma unroll
    for (int d = 0; d < DH; ++d) {
      qr[d] = rv ? qp[d] * sl2 : 0.f;
      acc[d] = 0.f;
    }
  }
  float m = -1e30f, l = 0.f;
  const size_t tok = static_cast<size_t>(Hkv) * DH;
  const float* kb = k + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * DH;
  const float* vb = v + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * DH;
  LiveTiles it;
  it.init(emax + static_cast<size_t>(b) * ntiles, (i1 - 1) / T, i0);
  for (int t = it.next(); t >= 0; t = it.next()) {
    const int j0 = t * T;
    for (int idx = lane; idx < T * DH / 4; idx += 64) {
      const int r = idx / (DH / 4), c = idx % (DH / 4);
      const int j = j0 + r;
      f32x4 kv4 = {0.f, 0.f, 0.f, 0.f}, vv4 = {0.f, 0.f, 0.f, 0.f};
      if (j < N) {
        kv4 = *reinterpret_cast<const f32x4*>(kb + j * tok + c * 4);
        vv4 = *reinterpret_cast<const f32x4*>(vb + j * tok + c * 4);
      }
      *reinterpret_cast<f32x4*>(&Ks[r][c * 4]) = kv4;
      *reinterpret_cast<f32x4*>(&Vs[r][c * 4]) = vv4;
    }
    Es[lane] = (j0 + lane < N) ? e[static_cast<size_t>(b) * N + j0 + lane] : 0;
    __syncthreads();
    for (int c0 = 0; c0 < T; c0 += C) {
      float s[C];
      float mx = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < C; ++jj) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < DH; ++d) dot = fmaf(qr[d], Ks[c0 + jj][d], dot);
        const int j = j0 + c0 + jj;
        const bool live = j <= i && i < Es[c0 + jj] && j < N;
        s[jj] = live ? dot : -INFINITY;
        mx = fmaxf(mx, s[jj]);
      }
      const float mn = fmaxf(m, mx);
      const float f = exp2f(m - mn);
      m = mn;
      l *= f;
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] *= f;
#pragma unroll
      for (int jj = 0; jj < C; ++jj) {
        const float p = exp2f(s[jj] - m);
        l += p;
#pragma unroll
        for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, Vs[c0 + jj][d], acc[d]);
      }
    }
    __syncthreads();
  }
  if (rv) {
    float* op = o + ((static_cast<size_t>(b) * N + i) * Hq + hq) * DH;
    const float inv = l > 0.f ? 1.f / l : 0.f;  // a row that sees no key: O = 0
#pragma unroll
    for (int d = 0; d < DH; ++d) op[d] = acc[d] * inv;
    if (lse) lse[(static_cast<size_t>(b) * Hq + hq) * N + i] = (m + log2f(l)) * KS_LN2;
  }
}

// ---------------------------------------------------------------------------
// bf16 forward (MFMA)
// ---------------------------------------------------------------------------
template <int DH, int HPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ e, const int32_t* __restrict__ emin,
    const int32_t* __restrict__ emax, bf16_t* __restrict__ o, float* __restrict__ lse, int B,
    int N, int Hq, int Hkv, int ntiles, int nqt, int total_wg, float sl2) {
  constexpr int RS = 4 / HPW;     // 64-row subtiles per workgroup
  constexpr int BM = 64 * RS;     // query rows per workgroup
  constexpr int KT = kKeyTile;    // keys per tile
  constexpr int NSTEP = DH / 16;  // k-steps of Q K^T
  constexpr int NDB = DH / 32;    // 32-row d blocks of O^T
  constexpr int CH = DH / 8;      // 16-byte chunks per key row
  constexpr int KCH = KT * CH / 256;  // K chunks loaded per thread
  constexpr int VPAIRS = (KT / 4) * CH;  // (4-key group, d chunk) pairs

  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KT * DH];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][DH * KT];
  __shared__ __attribute__((aligned(16))) int Es[2][KT];

  // XCD-aware remap: workgroup lin runs on XCD lin % 8; give each XCD a
  // contiguous range of logical tiles.
  int lin = blockIdx.x;
  lin = (lin & 7) * (total_wg >> 3) + (lin >> 3);
  const int ngrp = Hq / HPW;
  if (lin >= B * ngrp * nqt) return;
  // query tiles in descending order: the first tiles of a trace see only a
  // short causal prefix, so they are the short workgroups left for the end
  const int qt = nqt - 1 - lin % nqt;
  const int grp = (lin / nqt) % ngrp;
  const int b = lin / (nqt * ngrp);

  const int G = Hq / Hkv;
  const int hq0 = grp * HPW;
  const int hkv = hq0 / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hq = hq0 + (w % HPW);
  const int i0 = qt * BM;
  const int wi0 = i0 + (w / HPW) * 64;
  const int i1 = min(N, i0 + BM);
  const int lq = lane & 31, lh = lane >> 5;

  const size_t tok = static_cast<size_t>(Hkv) * DH;  // elements between tokens of K/V
  const bf16_t* kb = k + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * DH;
  const bf16_t* vb = v + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * DH;
  const int32_t* eb = e + static_cast<size_t>(b) * N;
  const int32_t* eminb = emin + static_cast<size_t>(b) * ntiles;

  // Q as the B operand of S^T = K Q^T: lane (lq, lh) holds row lq of each
  // 32-row block, d = 16*step + 8*lh .. +8.
  bf16x8 qf[2][NSTEP];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wi0 + qb * 32 + lq;
    const bf16_t* qp = q + (static_cast<size_t>(b) * N + (row < N ? row : 0)) * Hq * DH +
                       static_cast<size_t>(hq) * DH + lh * 8;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qp + s * 16);
      if (row >= N) x = u32x4{0u, 0u, 0u, 0u};
      qf[qb][s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  float mrow[2] = {-1e30f, -1e30f}, lrow[2] = {0.f, 0.f};

  // ---- tile staging ------------------------------------------------------
  u32x4 kr[KCH];
  u32x4 vr[4];
  int er = 0;
  auto load_tile = [&](int t) {
    const int j0 = t * KT;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int idx = tid + 256 * u;
      const int row = idx / CH, c = idx % CH;
      const int j = j0 + row;
      kr[u] = j < N ? *reinterpret_cast<const u32x4*>(kb + j * tok + c * 8)
                    : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < VPAIRS) {
      const int kg = tid % (KT / 4), dc = tid / (KT / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * kg + i;
        vr[i] = j < N ? *reinterpret_cast<const u32x4*>(vb + j * tok + dc * 8)
                      : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < KT) er = (j0 + tid < N) ? eb[j0 + tid] : 0;
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int idx = tid + 256 * u;
      const int row = idx / CH, c = idx % CH;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * DH + ((c ^ (row & (CH - 1))) * 8)]) = kr[u];
    }
    if (tid < VPAIRS) {
      const int kg = tid % (KT / 4), dc = tid / (KT / 4);
      // slot of key 4*kg: bits 2 and 3 of the key swapped within its 16-group
      const int slot = 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int d = dc * 8 + dd;
        const int wsel = dd >> 1;
        uint32_t lo, hi;
        if (dd & 1) {
          lo = (vr[0][wsel] >> 16) | (vr[1][wsel] & 0xffff0000u);
          hi = (vr[2][wsel] >> 16) | (vr[3][wsel] & 0xffff0000u);
        } else {
          lo = (vr[0][wsel] & 0xffffu) | (vr[1][wsel] << 16);
          hi = (vr[2][wsel] & 0xffffu) | (vr[3][wsel] << 16);
        }
        const int chunk = (slot >> 3) ^ ((d >> 1) & 7);
        *reinterpret_cast<u32x2*>(&Vt[buf][d * KT + chunk * 8 + (slot & 7)]) = u32x2{lo, hi};
      }
    }
    if (tid < KT) Es[buf][tid] = er;
  };

  // ---- one key tile ------------------------------------------------------
  auto compute = [&](int buf, int j0, bool partial) {
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      f32x16 sacc[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[0][r] = sacc[1][r] = 0.f;
      const int krow = kbk * 32 + lq;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const int c = 2 * s + lh;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &Ks[buf][krow * DH + ((c ^ (krow & (CH - 1))) * 8)]);
        sacc[0] = mfma32x32x16(kf, qf[0][s], sacc[0]);
        sacc[1] = mfma32x32x16(kf, qf[1][s], sacc[1]);
      }
      bf16x8 pf[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = sacc[qb][r] * sl2;
        if (partial) {
          const int i = wi0 + qb * 32 + lq;
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int kl = kbk * 32 + rg * 8 + lh * 4;
            const int4 ev = *reinterpret_cast<const int4*>(&Es[buf][kl]);
            const int ee[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int j = j0 + kl + c;
              const bool live = j <= i && i < ee[c] && j < N;
              sv[rg * 4 + c] = live ? sv[rg * 4 + c] : -INFINITY;
            }
          }
        }
        float mx = sv[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
        mx = max_lane_pair32(mx);
        const bool need = mx > mrow[qb] + kTau;
        if (__ballot(need)) {
          const float f = need ? fast_exp2(mrow[qb] - mx) : 1.f;
          mrow[qb] = need ? mx : mrow[qb];
          lrow[qb] *= f;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= f;
        }
        float ps = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 pk;
#pragma unroll
          for (int vv = 0; vv < 8; ++vv) {
            const float p = fast_exp2(sv[ks * 8 + vv] - mrow[qb]);
            ps += p;
            pk[vv] = (__bf16)p;
          }
          pf[qb][ks] = pk;
        }
        lrow[qb] += ps;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 32 + lq;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int chunk = (4 * kbk + 2 * ks + lh) ^ ((d >> 1) & 7);
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&Vt[buf][d * KT + chunk * 8]);
          oacc[0][db] = mfma32x32x16(vf, pf[0][ks], oacc[0][db]);
          oacc[1][db] = mfma32x32x16(vf, pf[1][ks], oacc[1][db]);
        }
      }
    }
  };

  // ---- main loop over live key tiles -------------------------------------
  LiveTiles it;
  it.init(emax + static_cast<size_t>(b) * ntiles, (i1 - 1) / KT, i0);
  int t = it.next();
  if (t >= 0) {
    load_tile(t);
    store_tile(0);
  }
  __syncthreads();
  int buf = 0;
  while (t >= 0) {
    const int tn = it.next();
    if (tn >= 0) load_tile(tn);
    const int j0 = t * KT;
    const bool full = (j0 + KT - 1 <= i0) && (eminb[t] >= i1) && (j0 + KT <= N);
    compute(buf, j0, !full);
    if (tn >= 0) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    t = tn;
  }

  // ---- epilogue ------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = sum_lane_pair32(lrow[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;  // a row that sees no key: O = 0
    const int i = wi0 + qb * 32 + lq;
    if (i < N) {
      bf16_t* op = o + (static_cast<size_t>(b) * N + i) * Hq * DH + static_cast<size_t>(hq) * DH;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d = db * 32 + rg * 8 + lh * 4;
          const uint32_t w0 = pack_bf16x2(oacc[qb][db][rg * 4 + 0] * inv, oacc[qb][db][rg * 4 + 1] * inv);
          const uint32_t w1 = pack_bf16x2(oacc[qb][db][rg * 4 + 2] * inv, oacc[qb][db][rg * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d) = u32x2{w0, w1};
        }
      if (lse && lh == 0)
        lse[(static_cast<size_t>(b) * Hq + hq) * N + i] = (mrow[qb] + __log2f(lt)) * KS_LN2;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 forward, D = 128 (MFMA, 8 waves)
//
// A workgroup = 8 waves = HPW query heads x 8/HPW subtiles of 32 query rows,
// so every staged 64-key tile is shared by 8 waves and each SIMD runs 2 waves
// (register budget <= 256), letting one wave's MFMAs overlap the other's
// softmax.  K and V stay in natural [key][d] layout in LDS; V^T operands are
// read with the LDS transpose instruction, so staging is a plain 16-byte copy.
// Per key tile and wave: S^T = K Q^T (16 MFMAs), masked lazily-rescaled
// softmax on 32 scores per lane, O^T += V^T P^T (16 MFMAs).
// ---------------------------------------------------------------------------
template <int HPW, bool ROPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_d128_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const TileSummary ts, bf16_t* __restrict__ o, float* __restrict__ lse, int B, int N, int Hq,
    int Hkv, int ntiles, int nqt, int total_wg, float sl2, const float2* __restrict__ rtab,
    bf16_t* __restrict__ q_rot) {
  constexpr int D = 128;
  constexpr int RS = 8 / HPW;   // 32-row subtiles per workgroup
  constexpr int BM = 32 * RS;   // query rows per workgroup
  constexpr int KT = kKeyTile;  // 64 keys per tile
  __shared__ __attribute__((aligned(16))) bf16_t S0[kKvElems];
  __shared__ __attribute__((aligned(16))) bf16_t S1[kKvElems];
  __shared__ __attribute__((aligned(16))) bf16_t S2[kKvElems];
  __shared__ __attribute__((aligned(16))) bf16_t S3[kKvElems];
  __shared__ uint16_t live[kLiveWindow];
  __shared__ int wsum[8];

  int lin = blockIdx.x;
  lin = (lin & 7) * (total_wg >> 3) + (lin >> 3);
  const int ngrp = Hq / HPW;
  if (lin >= B * ngrp * nqt) return;
  // query tiles in descending order: the first tiles of a trace see only a
  // short causal prefix, so they are the short workgroups left for the end
  const int qt = nqt - 1 - lin % nqt;
  const int grp = (lin / nqt) % ngrp;
  const int b = lin / (nqt * ngrp);
  const int G = Hq / Hkv;
  const int hq0 = grp * HPW;
  const int hkv = hq0 / G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = hq0 + (w % HPW);
  const int i0 = qt * BM;
  const int wi0 = i0 + (w / HPW) * 32;
  const int i1 = min(N, i0 + BM);
  const int lq = lane & 31, lh = lane >> 5;
  const int qi = wi0 + lq;  // this lane's query row
  const int la = tile_lane_a(lane), lt = tile_lane_t(lane);

  const int tok = Hkv * D;
  const bf16_t* kb = k + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * D;
  const bf16_t* vb = v + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * D;
  const int32_t* erb = ts.erec + static_cast<size_t>(b) * ntiles * kErec;
  const int32_t* emaxb = ts.emax + static_cast<size_t>(b) * ntiles;
  KvStager stg;
  stg.init(w, lane);

  // Q as the B operand of S^T = K Q^T: row qi, d = 16 s + 8 lh .. +8
  bf16x8 qf[8];
  {
    const bf16_t* qp = q + (static_cast<size_t>(b) * N + (qi < N ? qi : 0)) * Hq * D +
                       static_cast<size_t>(hq) * D + lh * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qp + s * 16);
      if (qi >= N) x = u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  if constexpr (ROPE) {
    // q arrives unrotated: rotate the row at its logical position (pairs
    // (d, d + 64) are fragments s and s + 4 of this lane) with the prepared
    // (cos, sin) pairs, and write the rotated row for the backward
    if (qi < N) {
      const float2* tr = rtab + (static_cast<size_t>(b) * N + qi) * (D / 2) + lh * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float2 cs[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 x = reinterpret_cast<const f32x4*>(tr + 16 * s)[u];
          cs[2 * u] = make_float2(x[0], x[1]);
          cs[2 * u + 1] = make_float2(x[2], x[3]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float x = static_cast<float>(qf[s][i]), y = static_cast<float>(qf[s + 4][i]);
          rope_rotate(x, y, cs[i]);
          qf[s][i] = static_cast<__bf16>(x);
          qf[s + 4][i] = static_cast<__bf16>(y);
        }
      }
      bf16_t* qo = q_rot + (static_cast<size_t>(b) * N + qi) * Hq * D +
                   static_cast<size_t>(hq) * D + lh * 8;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        *reinterpret_cast<u32x4*>(qo + s * 16) = __builtin_bit_cast(u32x4, qf[s]);
    }
  }
  wait_vm<0>();  // Q is in registers before the DMA stream starts
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float mrow = -1e30f, lrow = 0.f;

  // kv: staged tile t (K tile, then V tile)
  auto compute = [&](const bf16_t* kv, int t) {
    const bf16_t* Vt = kv + KT * kTileRow;
    const int j0 = t * KT;
    const int emn = __builtin_amdgcn_readfirstlane(staged_emin(kv));
    const bool partial = !((j0 + KT - 1 <= i0) && (emn >= i1) && (j0 + KT <= N));
    f32x16 sacc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kk][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        sacc[kk] = mfma32x32x16(tile_chunk(kv, la, kk * 32, 2 * s + lh), qf[s], sacc[kk]);
    }
    // scheduling: the K operand reads run four MFMAs ahead of their use
    // (0x100 = LDS reads, 0x008 = MFMA; the compiler alone issues them one
    // or two ahead and each MFMA then waits on its own read)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (p < 16 - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }

    if (partial) {  // uniform branch: element mask only on partial tiles
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int kl = kk * 32 + rg * 8 + lh * 4;
          const int4 ev = staged_e4(kv, kl >> 2);
          const int ee[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j = j0 + kl + c;
            const bool ok = j <= qi && qi < ee[c] && j < N;
            sacc[kk][rg * 4 + c] = ok ? sacc[kk][rg * 4 + c] : -INFINITY;
          }
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kk][r]);
    mx = max_lane_pair32(mx) * sl2;
    const bool need = mx > mrow + kTau;
    if (__ballot(need)) {
      const float f = need ? fast_exp2(mrow - mx) : 1.f;
      mrow = need ? mx : mrow;
      lrow *= f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= f;
    }
    bf16x8 pf[4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 pk;
#pragma unroll
        for (int vv = 0; vv < 8; ++vv)
          pk[vv] = (__bf16)fast_exp2(fmaf(sacc[kk][ks * 8 + vv], sl2, -mrow));
        pf[kk * 2 + ks] = pk;
        lrow = sum_bf16x8(pk, lrow);
      }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        oacc[db] = mfma32x32x16(tile_frag_t(Vt, lt, kk * 16, db * 32), pf[kk], oacc[db]);
    // scheduling: the V^T transpose reads (two per MFMA) run six MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (p < 16 - 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // live key tiles in windows of kLiveWindow; within a window, tile k is
  // staged into buffer k % 4 three tile computations before it is used
  const int tmax = (i1 - 1) / KT;
  for (int tw = 0; tw <= tmax; tw += kLiveWindow) {
    const int n = build_live_list(emaxb, tw, min(tmax, tw + kLiveWindow - 1), i0, live, wsum);
    if (n == 0) continue;
    auto tile = [&](int kidx) {
      return __builtin_amdgcn_readfirstlane(tw + live[min(kidx, n - 1)]);
    };
    stg.issue(lds_ptr(S0), tile(0), kb, vb, tok, erb, N);
    stg.issue(lds_ptr(S1), tile(1), kb, vb, tok, erb, N);
    stg.issue(lds_ptr(S2), tile(2), kb, vb, tok, erb, N);
    // the window's first loads land before the loop: the compiler then sees
    // no DMA in flight at the loop head and needs no waits beyond these
    wait_vm<0>();
#define KS_FWD_STEP(CUR, NXT, OFF)                          \
  {                                                         \
    const int kidx = k0 + (OFF);                            \
    wait_vm<kKvDma * 2>();                                  \
    bar_nofence();                                          \
    stg.issue(lds_ptr(NXT), tile(kidx + 3), kb, vb, tok, erb, N);\
    if (kidx < n) compute(CUR, tile(kidx));                 \
  }
    for (int k0 = 0; k0 < n; k0 += 4) {
      KS_FWD_STEP(S0, S3, 0)
      KS_FWD_STEP(S1, S0, 1)
      KS_FWD_STEP(S2, S1, 2)
      KS_FWD_STEP(S3, S2, 3)
    }
#undef KS_FWD_STEP
    wait_vm<0>();  // the window's last (re-staged) loads land before reuse
    bar_nofence();
  }

  const float ltot = sum_lane_pair32(lrow);
  if (qi < N) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;  // a row that sees no key: O = 0
    bf16_t* op = o + (static_cast<size_t>(b) * N + qi) * Hq * D + static_cast<size_t>(hq) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = db * 32 + rg * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(op + d) =
            u32x2{pack_bf16x2(oacc[db][rg * 4 + 0] * inv, oacc[db][rg * 4 + 1] * inv),
                  pack_bf16x2(oacc[db][rg * 4 + 2] * inv, oacc[db][rg * 4 + 3] * inv)};
      }
    if (lse && lh == 0)
      lse[(static_cast<size_t>(b) * Hq + hq) * N + qi] = (mrow + __log2f(ltot)) * KS_LN2;
  }
}

}  // namespace
}  // namespace ksattn

using namespace ksattn;

extern "C" size_t ks_evict_attn_fwd_workspace(int B, int N, int Hq, int Hkv, int D, int dtype) {
  (void)Hq;
  (void)Hkv;
  (void)D;
  (void)dtype;
  if (B <= 0 || N <= 0) return 0;
  return summary_bytes(B, N);
}

extern "C" ks_status ks_evict_attn_fwd(const void* q, const void* k, const void* v,
                                       const int32_t* e, void* o, float* lse, int B, int N, int Hq,
                                       int Hkv, int D, int dtype, float scale, void* ws,
                                       size_t ws_bytes, void* stream) {
  KS_REQUIRE(B >= 0 && N >= 0 && Hq > 0 && Hkv > 0, "ks_evict_attn_fwd: bad sizes");
  KS_REQUIRE(Hq % Hkv == 0, "ks_evict_attn_fwd: Hq %% Hkv != 0");
  KS_REQUIRE(dtype == KS_F32 || dtype == KS_BF16, "ks_evict_attn_fwd: dtype %d", dtype);
  KS_REQUIRE(scale > 0.f, "ks_evict_attn_fwd: scale must be positive");
  const int G = Hq / Hkv;
  if (dtype == KS_BF16 && !(D == 128 || D == 64))
    return ks_fail(KS_ERR_UNSUPPORTED, "ks_evict_attn_fwd: bf16 needs D=64 or 128 (D=%d)", D);
  if (dtype == KS_F32 && !(D == 64 || D == 128))
    return ks_fail(KS_ERR_UNSUPPORTED, "ks_evict_attn_fwd: f32 needs D=64 or 128 (D=%d)", D);
  const int hpw = ks_heads_per_wave(G);
  if (B == 0 || N == 0) return KS_OK;
  KS_REQUIRE(q && k && v && e && o, "ks_evict_attn_fwd: null pointer");
  KS_REQUIRE(ks_aligned16(q) && ks_aligned16(k) && ks_aligned16(v) && ks_aligned16(o),
             "ks_evict_attn_fwd: tensors must be 16-byte aligned");
  const size_t need = summary_bytes(B, N);
  if (!ws || ws_bytes < need)
    return ks_fail(KS_ERR_WORKSPACE, "ks_evict_attn_fwd: workspace %zu < %zu bytes", ws_bytes,
                   need);
  KS_REQUIRE(ks_aligned16(ws), "ks_evict_attn_fwd: workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  TileSummary ts;
  ks_status st = launch_summary(e, ws, B, N, s, &ts);
  if (st != KS_OK) return st;
  const int32_t* emin = ts.emin;
  const int32_t* emax = ts.emax;
  const int ntiles = (N + kKeyTile - 1) / kKeyTile;
  const float sl2 = scale * KS_LOG2E;
  if (dtype == KS_F32) {
    KS_REQUIRE(B < 65536 && Hq < 65536, "ks_evict_attn_fwd: grid too large");
    const dim3 grid((N + 63) / 64, Hq, B);
    const float* qq = static_cast<const float*>(q);
    const float* kk = static_cast<const float*>(k);
    const float* vv = static_cast<const float*>(v);
    if (D == 64)
      hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, s, qq, kk, vv, e, emin, emax,
                         static_cast<float*>(o), lse, N, Hq, Hkv, ntiles, sl2);
    else
      hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, s, qq, kk, vv, e, emin, emax,
                         static_cast<float*>(o), lse, N, Hq, Hkv, ntiles, sl2);
    return ks_check_launch("ks_evict_attn_fwd(f32)");
  }
  const int rs = 4 / hpw;
  const int nqt = (N + 64 * rs - 1) / (64 * rs);
  const long long real = static_cast<long long>(B) * (Hq / hpw) * nqt;
  const long long total = (real + 7) / 8 * 8;
  KS_REQUIRE(total < (1LL << 31), "ks_evict_attn_fwd: grid too large");
  const bf16_t* qq = static_cast<const bf16_t*>(q);
  const bf16_t* kk = static_cast<const bf16_t*>(k);
  const bf16_t* vv = static_cast<const bf16_t*>(v);
  bf16_t* oo = static_cast<bf16_t*>(o);
#define KS_FWD_LAUNCH(DH_, HPW_)                                                              \
  hipLaunchKernelGGL((fwd_bf16_kernel<DH_, HPW_>), dim3(static_cast<unsigned>(total)),        \
                     dim3(256), 0, s, qq, kk, vv, e, emin, emax, oo, lse, B, N, Hq, Hkv,      \
                     ntiles, nqt, static_cast<int>(total), sl2)
  if (D == 128) {
    const int rs8 = 8 / hpw;
    const int nqt8 = (N + 32 * rs8 - 1) / (32 * rs8);
    const long long real8 = static_cast<long long>(B) * (Hq / hpw) * nqt8;
    const long long total8 = (real8 + 7) / 8 * 8;
    KS_REQUIRE(total8 < (1LL << 31), "ks_evict_attn_fwd: grid too large");
#define KS_FWD128_LAUNCH(HPW_)                                                                 \
  hipLaunchKernelGGL((fwd_d128_kernel<HPW_, false>), dim3(static_cast<unsigned>(total8)),       \
                     dim3(512), 0, s, qq, kk, vv, ts, oo, lse, B, N, Hq, Hkv, ntiles, nqt8,       \
                     static_cast<int>(total8), sl2, nullptr, nullptr)
    if (hpw == 4) KS_FWD128_LAUNCH(4);
    else if (hpw == 2) KS_FWD128_LAUNCH(2);
    else KS_FWD128_LAUNCH(1);
#undef KS_FWD128_LAUNCH
  } else {
    if (hpw == 4) KS_FWD_LAUNCH(64, 4);
    else if (hpw == 2) KS_FWD_LAUNCH(64, 2);
    else KS_FWD_LAUNCH(64, 1);
  }
#undef KS_FWD_LAUNCH
  return ks_check_launch("ks_evict_attn_fwd(bf16)");
}

// ---------------------------------------------------------------------------
// RoPE fused into the forward: q and k arrive unrotated.  The preparation
// kernel writes the (cos, sin) table of every token's logical position and
// the rotated keys (k_rot), next to the per-tile e summary; the forward
// kernel rotates each query row in registers as it loads it and writes the
// rotated row (q_rot) for the backward.  New queries and keys continue the
// original position count (explainer, RoPE paragraph), so the caller passes
// logical positions.
// ---------------------------------------------------------------------------
extern "C" size_t ks_evict_attn_fwd_rope_workspace(int B, int N, int Hq, int Hkv, int D,
                                                   int dtype) {
  (void)Hq;
  (void)Hkv;
  (void)dtype;
  if (B <= 0 || N <= 0 || D <= 0) return 0;
  return summary_bytes(B, N) + rope_table_bytes(B, N, D);
}

extern "C" ks_status ks_evict_attn_fwd_rope(const void* q, const void* k, const void* v,
                                            const int32_t* e, const int32_t* pos, void* q_rot,
                                            void* k_rot, void* o, float* lse, int B, int N,
                                            int Hq, int Hkv, int D, int dtype, float scale,
                                            float base, void* ws, size_t ws_bytes,
                                            void* stream) {
  const char* name = "ks_evict_attn_fwd_rope";
  KS_REQUIRE(B >= 0 && N >= 0 && Hq > 0 && Hkv > 0, "%s: bad sizes", name);
  KS_REQUIRE(Hq % Hkv == 0, "%s: Hq %% Hkv != 0", name);
  KS_REQUIRE(scale > 0.f, "%s: scale must be positive", name);
  KS_REQUIRE(base > 1.0f, "%s: base must be > 1", name);
  if (dtype != KS_BF16 || D != 128)
    return ks_fail(KS_ERR_UNSUPPORTED, "%s: only bf16 with D=128 (dtype=%d D=%d)", name, dtype,
                   D);
  const int hpw = ks_heads_per_wave(Hq / Hkv);
  if (B == 0 || N == 0) return KS_OK;
  KS_REQUIRE(q && k && v && e && pos && q_rot && k_rot && o && lse, "%s: null pointer", name);
  KS_REQUIRE(ks_aligned16(q) && ks_aligned16(k) && ks_aligned16(v) && ks_aligned16(o) &&
                 ks_aligned16(q_rot) && ks_aligned16(k_rot),
             "%s: tensors must be 16-byte aligned", name);
  const size_t nq = static_cast<size_t>(B) * N * Hq * D * 2, nk = static_cast<size_t>(B) * N *
                                                                   Hkv * D * 2;
  auto overlap = [](const void* a, size_t na, const void* c, size_t nc) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(c);
    return x < y + nc && y < x + na;
  };
  KS_REQUIRE(!overlap(q, nq, q_rot, nq) && !overlap(k, nk, k_rot, nk),
             "%s: q_rot and k_rot must not alias q and k", name);
  // the keys are rotated before the attention reads q, k and v, and q_rot
  // and o are written by the same kernel: the three outputs must not touch
  // the inputs or each other
  KS_REQUIRE(!overlap(k_rot, nk, q, nq) && !overlap(k_rot, nk, v, nk) &&
                 !overlap(q_rot, nq, k, nk) && !overlap(q_rot, nq, v, nk) &&
                 !overlap(q_rot, nq, k_rot, nk) && !overlap(o, nq, q_rot, nq) &&
                 !overlap(o, nq, k_rot, nk),
             "%s: q_rot, k_rot and o must not overlap the inputs or each other", name);
  const size_t need = summary_bytes(B, N) + rope_table_bytes(B, N, D);
  if (!ws || ws_bytes < need)
    return ks_fail(KS_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", name, ws_bytes, need);
  KS_REQUIRE(ks_aligned16(ws), "%s: workspace must be 16-byte aligned", name);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* table = reinterpret_cast<float2*>(static_cast<char*>(ws) + summary_bytes(B, N));
  ks_status st = launch_rope_prep(static_cast<const bf16_t*>(k), static_cast<bf16_t*>(k_rot), pos,
                                  table, static_cast<long long>(B) * N, Hkv, D, base, s);
  if (st != KS_OK) return st;
  TileSummary ts;
  st = launch_summary(e, ws, B, N, s, &ts);
  if (st != KS_OK) return st;
  const int ntiles = (N + kKeyTile - 1) / kKeyTile;
  const float sl2 = scale * KS_LOG2E;
  const int rs8 = 8 / hpw;
  const int nqt8 = (N + 32 * rs8 - 1) / (32 * rs8);
  const long long real8 = static_cast<long long>(B) * (Hq / hpw) * nqt8;
  const long long total8 = (real8 + 7) / 8 * 8;
  KS_REQUIRE(total8 < (1LL << 31), "%s: grid too large", name);
  const bf16_t* qq = static_cast<const bf16_t*>(q);
  const bf16_t* kk = static_cast<const bf16_t*>(k_rot);
  const bf16_t* vv = static_cast<const bf16_t*>(v);
  bf16_t* oo = static_cast<bf16_t*>(o);
  bf16_t* qr = static_cast<bf16_t*>(q_rot);
#define KS_FWD128_ROPE(HPW_)                                                                  \
  hipLaunchKernelGGL((fwd_d128_kernel<HPW_, true>), dim3(static_cast<unsigned>(total8)),      \
                     dim3(512), 0, s, qq, kk, vv, ts, oo, lse, B, N, Hq, Hkv, ntiles, nqt8,     \
                     static_cast<int>(total8), sl2, table, qr)
  if (hpw == 4) KS_FWD128_ROPE(4);
  else if (hpw == 2) KS_FWD128_ROPE(2);
  else KS_FWD128_ROPE(1);
#undef KS_FWD128_ROPE
  return ks_check_launch(name);
}
