// Backward of the eviction-masked attention (bf16, D = 128).
//
// The mask replays compaction (KV-streams explainer, trainer paragraph;
// paper page, Fig. 2A); the gradients follow from the softmax calculus:
//   P = exp(S - LSE), dV = P^T dO, dP = dO V^T, D_i = rowsum(dO o O),
//   dS = P o (dP - D_i), dQ = scale dS K, dK = scale dS^T Q.
//
// Deterministic two-kernel split (no atomics, no fp32 dQ workspace), in
// launch order:
//   dq_kernel    query-tile outer, laid out like the forward:
//                S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T; its prologue
//                forms D_i of each query row and writes the (LSE, D_i)
//                records the second kernel stages.
//   dkdv_kernel  key-tile outer: a workgroup owns 256 keys of one kv head and
//                walks every query head of the group over the query rows
//                that can see them, [j0, max e_j), in 32-row chunks:
//                S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
// The pair executes 14*D flops per live (query, key, head) triple against
// the 10*D of a fused kernel, in exchange for no atomic traffic at all.
// Both run 8 waves per workgroup (2 per SIMD) on tiles staged in natural
// layout (see attn_common.h); transposed operands come from LDS transpose
// reads, and the element mask runs only on partial tiles (uniform branch).
#include "attn_common.h"

namespace ksattn {
namespace {

constexpr int D = 128;
constexpr int NSTEP = D / 16;  // k-steps over the head dimension
constexpr int NDB = D / 32;    // 32-wide d blocks
constexpr int CH = D / 8;      // 16-byte chunks per row
constexpr int BQ = 32;         // query rows per dK/dV chunk
constexpr int KW = 256;        // keys per dK/dV workgroup (8 waves x 32)
constexpr int KT = kKeyTile;   // keys per dQ tile

// ---------------------------------------------------------------------------
// Softmax records: rec[b][h][c][64] holds, for the 32-row query chunk c of
// every (batch, head), the LSE of rows 32 c .. 32 c + 31 in log2 units, then
// their D_i = sum_d dO_id O_id (fp32): 256 bytes, one DMA unit.  Rows past N
// (up to Npad = N rounded up to BQ) hold 0.  The dQ kernel forms them (it
// holds each query row's dO in registers anyway) and dK/dV, launched after
// it, stages them with its query chunks.
// ---------------------------------------------------------------------------
// dK, dV.  K stays in registers as the B operand of S = Q K^T; V of the 256
// keys stays in LDS for the whole walk (B operand of dP = dO V^T).  Query
// chunks (Q, dO, LSE, D_i of 32 rows of one head) go from global memory
// straight into LDS with LDS-DMA loads (global_load_lds_dwordx4, no
// registers), NBUF chunks in flight, so a chunk's loads are issued NBUF - 1
// chunk computations before it is used.  dO^T and Q^T come from transpose
// reads.  Workgroups are ordered key-tile major so the heavy prompt tiles
// (whose queries run to the end of the trace) start first.
//
// A staged chunk is a Q tile, a dO tile (32 rows each in the padded layout
// of attn_common.h, 544 16-byte slots each, contiguous) and the chunk's
// LSE / D_i record.  Every DMA instruction reads from one tensor: Q_j covers
// slots [64 j, 64 j + 64) (Q only, j = 0..7), M covers [512, 576) (the last
// 32 Q slots and the first 32 dO slots; each half-wave has its own base),
// O_j covers [576 + 64 j, 640 + 64 j) (dO only) and R the record.  Pad slots
// get a copy of a data chunk.  Wave w issues Q_w, O_w and, by w % 2, M or R
// (four waves write each with the same bytes): 3 DMA loads per wave.
// ---------------------------------------------------------------------------
constexpr int NBUF = 4;                       // staged chunks
constexpr int TSLOTS = BQ * (kTileRow / 8);   // 16-byte slots per 32-row tile
constexpr int RECE = 2 * TSLOTS * 8;          // element offset of the record
constexpr int CELEMS = RECE + 512;            // bf16 elements per staged chunk
constexpr int DMA_PER_WAVE = 3;

// (row, chunk) of a slot of a 32-row staged tile: bits 0..4 row, 5..8 chunk
__device__ __forceinline__ int chunk_slot_rc(int s) {
  const int p = s / 17, c = s - 17 * p;
  return tile_prow(p) | (min(c, 15) << 5);
}

// Gradients of the RoPE-fused path are with respect to the unrotated q and
// k: the fp32 gradient row (blocks acc[db], rows d = 32 db + 8 rg + 4 lh + c)
// is rotated by -theta before it is stored.  tr: the row's (cos, sin) pairs.
__device__ __forceinline__ void rotate_back(f32x16 (&acc)[NDB], const float2* tr, int lh) {
#pragma unroll
  for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4* p4 = reinterpret_cast<const f32x4*>(tr + 32 * db + 8 * rg + 4 * lh);
      const f32x4 a = p4[0], c = p4[1];
      const float2 cs[4] = {make_float2(a[0], -a[1]), make_float2(a[2], -a[3]),
                            make_float2(c[0], -c[1]), make_float2(c[2], -c[3])};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[db][rg * 4 + i], y = acc[db + 2][rg * 4 + i];
        rope_rotate(x, y, cs[i]);
        acc[db][rg * 4 + i] = x;
        acc[db + 2][rg * 4 + i] = y;
      }
    }
}

template <bool ROPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ e, const int32_t* __restrict__ emin,
    const int32_t* __restrict__ emax, const float* __restrict__ rec,
    const bf16_t* __restrict__ dout, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int B,
    int N, int Npad, int Hq, int Hkv, int ntiles, float scale, const float2* __restrict__ rtab) {
  __shared__ __attribute__((aligned(16))) bf16_t Vst[KW * kTileRow];
  __shared__ __attribute__((aligned(16))) bf16_t C0[CELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t C1[CELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t C2[CELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t C3[CELEMS];
  const int nbh = B * Hkv;
  const int kt = blockIdx.x / nbh;
  const int bh = blockIdx.x % nbh;
  const int b = bh / Hkv, hkv = bh % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, lh = lane >> 5;
  const int la = tile_lane_a(lane), lt = tile_lane_t(lane);
  const int j0 = kt * KW;
  const int kw0 = j0 + 32 * w;
  const int jl = kw0 + lq;
  const size_t tokkv = static_cast<size_t>(Hkv) * D;
  const int tokq = Hq * D;
  const float sl2 = scale * KS_LOG2E;

  int emx = static_cast<int>(0x80000000), emn = 0x7fffffff;
  {
    const int t0 = j0 / kKeyTile;
    const int t1 = min(ntiles - 1, t0 + KW / kKeyTile - 1);
    for (int t = t0; t <= t1; ++t) {
      emx = max(emx, emax[static_cast<size_t>(b) * ntiles + t]);
      emn = min(emn, emin[static_cast<size_t>(b) * ntiles + t]);
    }
  }
  // workgroup bounds, made provably uniform for the compiler
  emx = __builtin_amdgcn_readfirstlane(emx);
  emn = __builtin_amdgcn_readfirstlane(emn);
  const int qend = min(N, emx);
  const int c_begin = j0 / BQ;
  const int c_end = (qend + BQ - 1) / BQ;
  const int nc = c_end > c_begin ? c_end - c_begin : 0;
  const int nchunks = nc * G;

  // chunk order: query chunks walked backwards from the end of the range,
  // heads innermost; chunk idx = (query chunk c_end - 1 - idx / G, head
  // hkv G + idx % G), tracked with counters (no division per step)
  const int nck = Npad / BQ;
  const uint32_t rc = static_cast<uint32_t>(chunk_slot_rc(64 * w + lane)) |
                      (static_cast<uint32_t>(chunk_slot_rc(32 + 64 * w + lane)) << 9) |
                      (static_cast<uint32_t>(chunk_slot_rc(lane < 32 ? 512 + lane : lane - 32))
                       << 18);
  const bool mhi = lane >= 32;  // M: lanes 32..63 take dO slots 0..31
  const int sel = w & 1;        // 0: M, 1: R
  auto rcoff = [&](uint32_t d, int lim) {
    const int r = static_cast<int>(d & 31), c = static_cast<int>((d >> 5) & 15);
    return static_cast<uint32_t>(min(r, lim) * (tokq * 2) + c * 16);
  };
  int ih = 0, ic0 = (c_end - 1) * BQ, ij = 0;  // chunk of the next issue
  // stage the chunk (head offset hh, first row c0) into buffer dst
  auto issue = [&](lds_bf16_t* dst, int hh, int c0) {
    const int h = hkv * G + hh;
    const int lim = N - 1 - c0;  // rows past the end re-read row N - 1
    const size_t rowq = (static_cast<size_t>(b) * N + c0) * tokq + static_cast<size_t>(h) * D;
    const char* qc = reinterpret_cast<const char*>(q + rowq);
    const char* oc = reinterpret_cast<const char*>(dout + rowq);
    const char* rcb = reinterpret_cast<const char*>(
        rec + ((static_cast<size_t>(b) * Hq + h) * nck + c0 / BQ) * (2 * BQ));
    lds_dma16(qc + rcoff(rc, lim), dst + 64 * w * 8);
    lds_dma16(oc + rcoff(rc >> 9, lim), dst + (TSLOTS + 32 + 64 * w) * 8);
    const char* mb = mhi ? oc : qc;
    const uint32_t mo = rcoff(rc >> 18, lim);
    const uint32_t ro = static_cast<uint32_t>((lane & 15) * 16);
    lds_dma16((sel ? rcb : mb) + (sel ? ro : mo), dst + (sel ? RECE : 512 * 8));
  };
  auto issue_next = [&](lds_bf16_t* dst) {  // the tail re-stages the last chunk
    issue(dst, ih, ic0);
    if (ij < nchunks - 1) {
      ++ij;
      if (++ih == G) {
        ih = 0;
        ic0 -= BQ;
      }
    }
  };
  if (nchunks > 0) {
    issue_next(lds_ptr(C0));
    issue_next(lds_ptr(C1));
    issue_next(lds_ptr(C2));
  }

  bf16x8 kf[NSTEP];
  {
    const size_t off = (static_cast<size_t>(b) * N + (jl < N ? jl : 0)) * tokkv +
                       static_cast<size_t>(hkv) * D + lh * 8;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      u32x4 a = *reinterpret_cast<const u32x4*>(k + off + s * 16);
      if (jl >= N) a = u32x4{0u, 0u, 0u, 0u};
      kf[s] = __builtin_bit_cast(bf16x8, a);
    }
  }
  const int ej = jl < N ? e[static_cast<size_t>(b) * N + jl] : 0;
  for (int idx = tid; idx < KW * CH; idx += 512) {
    const int row = idx >> 4, c = idx & 15;
    const int j = j0 + row;
    const u32x4 x = j < N ? *reinterpret_cast<const u32x4*>(
                                v + (static_cast<size_t>(b) * N + j) * tokkv +
                                static_cast<size_t>(hkv) * D + c * 8)
                          : u32x4{0u, 0u, 0u, 0u};
    tile_store_chunk(Vst, row, c, x);
  }
  int wemx = jl < N ? ej : static_cast<int>(0x80000000);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) wemx = max(wemx, __shfl_xor(wemx, off));
  const int wq1 = __builtin_amdgcn_readfirstlane(min(N, wemx));
  const int kmax = min(N, j0 + KW) - 1;

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[db][r] = dva[db][r] = 0.f;

  auto compute = [&](const bf16_t* Qs, int c0) {
    if (c0 >= wq1 || c0 + BQ <= kw0) return;  // none of this wave's keys is seen
    const bf16_t* Os = Qs + BQ * kTileRow;
    const float* Rc = reinterpret_cast<const float*>(Qs + RECE);
    const bool partial = !((c0 >= kmax) && (c0 + BQ <= emn) && (c0 + BQ <= N));
    f32x16 sacc, pacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      sacc = mfma32x32x16(tile_chunk(Qs, la, 0, 2 * s + lh), kf[s], sacc);
      pacc = mfma32x32x16(tile_chunk(Os, la, 0, 2 * s + lh),
                          tile_chunk(Vst, la, 32 * w, 2 * s + lh), pacc);
    }
    // lane = key jl; accumulator row r = query c0 + 8 (r / 4) + 4 lh + r % 4;
    // LSE and D_i come from the chunk's record
    float pv[16];
    if (partial) {  // uniform branch: element mask only on partial chunks
      const int lo = jl - c0, hi = min(ej, N) - c0;  // live iff lo <= row < hi
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 l4 = *reinterpret_cast<const float4*>(Rc + rg * 8 + lh * 4);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int row = rg * 8 + lh * 4 + c;
          const float p = fast_exp2(fmaf(sacc[rg * 4 + c], sl2, -lv[c]));
          pv[rg * 4 + c] = (row >= lo && row < hi) ? p : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 l4 = *reinterpret_cast<const float4*>(Rc + rg * 8 + lh * 4);
        pv[rg * 4 + 0] = fast_exp2(fmaf(sacc[rg * 4 + 0], sl2, -l4.x));
        pv[rg * 4 + 1] = fast_exp2(fmaf(sacc[rg * 4 + 1], sl2, -l4.y));
        pv[rg * 4 + 2] = fast_exp2(fmaf(sacc[rg * 4 + 2], sl2, -l4.z));
        pv[rg * 4 + 3] = fast_exp2(fmaf(sacc[rg * 4 + 3], sl2, -l4.w));
      }
    }
    // dV MFMAs need P only: they go first, and the dS arithmetic overlaps them
    bf16x8 pf[2], sf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)pv[r];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        dva[db] = mfma32x32x16(tile_frag_t(Os, lt, 16 * ks, 32 * db), pf[ks], dva[db]);
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const float4 d4 = *reinterpret_cast<const float4*>(Rc + BQ + rg * 8 + lh * 4);
      const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = rg * 4 + c;
        sf[r >> 3][r & 7] = (__bf16)(pv[r] * (pacc[r] - dd[c]));
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        dka[db] = mfma32x32x16(tile_frag_t(Qs, lt, 16 * ks, 32 * db), sf[ks], dka[db]);
    // scheduling: the dO^T / Q^T transpose reads (two per MFMA) run three
    // MFMAs ahead (0x100 = LDS reads, 0x008 = MFMA); left alone, the compiler
    // issues them just before each MFMA, which then waits on them
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int p = 0; p < 4 * NDB; ++p) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (p < 4 * NDB - 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  __syncthreads();  // V staged
  // step: own DMA loads of chunk idx have landed (the NBUF - 2 later chunks
  // may still be in flight); after the barrier every wave's have, and the
  // buffer read at step idx - 1 is free for chunk idx + NBUF - 1
  int ch = 0, cc0 = (c_end - 1) * BQ;  // chunk of the next compute
#define KS_DKDV_STEP(CUR, NXT)                           \
  {                                                      \
    const int idx = base + (CUR##_i);                    \
    wait_vm<DMA_PER_WAVE * (NBUF - 2)>();                \
    bar_nofence();                                       \
    issue_next(lds_ptr(NXT));                            \
    if (idx < nchunks) compute(CUR, cc0);                \
    if (++ch == G) {                                     \
      ch = 0;                                            \
      cc0 -= BQ;                                         \
    }                                                    \
  }
  constexpr int C0_i = 0, C1_i = 1, C2_i = 2, C3_i = 3;
  for (int base = 0; base < nchunks; base += NBUF) {
    KS_DKDV_STEP(C0, C3)
    KS_DKDV_STEP(C1, C0)
    KS_DKDV_STEP(C2, C1)
    KS_DKDV_STEP(C3, C2)
  }
#undef KS_DKDV_STEP
  wait_vm<0>();  // no DMA write may land after the workgroup ends

  // lane holds key jl; rows of dK^T / dV^T are d = 32 db + 8 rg + 4 lh + c
  if (jl < N) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dka[db][r] *= scale;
    if constexpr (ROPE) {
      // gradient with respect to the unrotated key: rotate back by -theta
      // (pairs (d, d + 64) are blocks db and db + 2 of this lane)
      rotate_back(dka, rtab + (static_cast<size_t>(b) * N + jl) * (D / 2), lh);
    }
    const size_t off = (static_cast<size_t>(b) * N + jl) * tokkv + static_cast<size_t>(hkv) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = db * 32 + rg * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(dk + off + d) =
            u32x2{pack_bf16x2(dka[db][rg * 4], dka[db][rg * 4 + 1]),
                  pack_bf16x2(dka[db][rg * 4 + 2], dka[db][rg * 4 + 3])};
        *reinterpret_cast<u32x2*>(dv + off + d) =
            u32x2{pack_bf16x2(dva[db][rg * 4], dva[db][rg * 4 + 1]),
                  pack_bf16x2(dva[db][rg * 4 + 2], dva[db][rg * 4 + 3])};
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: laid out like the forward, 32 query rows per wave; key tiles of K and
// V staged natural, K^T operands by transpose reads.
// ---------------------------------------------------------------------------
template <int HPW, bool ROPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const TileSummary ts, float* __restrict__ rec, const bf16_t* __restrict__ o,
    const float* __restrict__ lse, const bf16_t* __restrict__ dout, bf16_t* __restrict__ dq,
    int B, int N, int Npad, int Hq, int Hkv, int ntiles, int nqt, int total_wg, float scale,
    const float2* __restrict__ rtab) {
  constexpr int RS = 8 / HPW;
  constexpr int BM = 32 * RS;
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
  const int la = tile_lane_a(lane), lt = tile_lane_t(lane);
  const int qi = wi0 + lq;
  const int tok = Hkv * D;
  const size_t tokq = static_cast<size_t>(Hq) * D;
  const bf16_t* kb = k + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * D;
  const bf16_t* vb = v + static_cast<size_t>(b) * N * tok + static_cast<size_t>(hkv) * D;
  const int32_t* erb = ts.erec + static_cast<size_t>(b) * ntiles * kErec;
  const int32_t* emaxb = ts.emax + static_cast<size_t>(b) * ntiles;
  const float sl2 = scale * KS_LOG2E;
  KvStager stg;
  stg.init(w, lane);

  // Q and dO rows in registers; D_i = sum_d dO_id O_id of this lane's row
  // from the two half rows of the lane pair (lq, lq + 32), and the row's LSE
  // in log2 units; the row's record (LSE, D_i) is also written for dK/dV,
  // which runs after this kernel (rows N .. Npad - 1 get zeros)
  bf16x8 qf[NSTEP], gf[NSTEP];
  float l2, dii;
  {
    const size_t off = (static_cast<size_t>(b) * N + (qi < N ? qi : 0)) * tokq +
                       static_cast<size_t>(hq) * D + lh * 8;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      u32x4 a = *reinterpret_cast<const u32x4*>(q + off + s * 16);
      u32x4 c = *reinterpret_cast<const u32x4*>(dout + off + s * 16);
      u32x4 ov = *reinterpret_cast<const u32x4*>(o + off + s * 16);
      if (qi >= N) a = c = ov = u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, a);
      gf[s] = __builtin_bit_cast(bf16x8, c);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc += lo_bf16(c[i]) * lo_bf16(ov[i]) + hi_bf16(c[i]) * hi_bf16(ov[i]);
    }
    acc += __shfl_xor(acc, 32);
    const float lv = qi < N ? lse[(static_cast<size_t>(b) * Hq + hq) * N + qi] * KS_LOG2E : 0.f;
    l2 = qi < N ? lv : INFINITY;
    dii = qi < N ? acc : 0.f;
    if (lh == 0 && qi < Npad) {
      float* r0 =
          rec + ((static_cast<size_t>(b) * Hq + hq) * (Npad / BQ) + qi / BQ) * (2 * BQ) + qi % BQ;
      r0[0] = qi < N ? lv : 0.f;
      r0[BQ] = dii;
    }
  }
  wait_vm<0>();  // Q, dO in registers before the DMA stream starts
  f32x16 dqa[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

  // kv: staged tile t (K tile, then V tile)
  auto compute = [&](const bf16_t* kv, int t) {
    const bf16_t* Vt = kv + KT * kTileRow;
    const int j0 = t * KT;
    const int emn = __builtin_amdgcn_readfirstlane(staged_emin(kv));
    const bool partial = !((j0 + KT - 1 <= i0) && (emn >= i1) && (j0 + KT <= N));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
      // S first: its exponentials then overlap the dP MFMAs.
      // lane = query qi; accumulator row r = key j0 + 32 kk + 8 (r / 4) + 4 lh + r % 4
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
        sacc = mfma32x32x16(tile_chunk(kv, la, kk * 32, 2 * s + lh), qf[s], sacc);
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(fmaf(sacc[r], sl2, -l2));
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
        pacc = mfma32x32x16(tile_chunk(Vt, la, kk * 32, 2 * s + lh), gf[s], pacc);
      if (partial) {  // uniform branch: element mask only on partial tiles
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int kl = kk * 32 + rg * 8 + lh * 4;
          const int4 ev = staged_e4(kv, kl >> 2);
          const int ee[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j = j0 + kl + c;
            pv[rg * 4 + c] = (j <= qi && qi < ee[c] && j < N) ? pv[rg * 4 + c] : 0.f;
          }
        }
      }
      bf16x8 sf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) sf[r >> 3][r & 7] = (__bf16)(pv[r] * (pacc[r] - dii));
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          dqa[db] = mfma32x32x16(tile_frag_t(kv, lt, kk * 32 + 16 * ks, 32 * db), sf[ks],
                                 dqa[db]);
      // scheduling: the K^T transpose reads (two per MFMA) run four MFMAs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int p = 0; p < 2 * NDB; ++p) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (p < 2 * NDB - 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
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
#define KS_DQ_STEP(CUR, NXT, OFF)                             \
  {                                                           \
    const int kidx = k0 + (OFF);                              \
    wait_vm<kKvDma * 2>();                                    \
    bar_nofence();                                            \
    stg.issue(lds_ptr(NXT), tile(kidx + 3), kb, vb, tok, erb, N);\
    if (kidx < n) compute(CUR, tile(kidx));                                 \
  }
    for (int k0 = 0; k0 < n; k0 += 4) {
      KS_DQ_STEP(S0, S3, 0)
      KS_DQ_STEP(S1, S0, 1)
      KS_DQ_STEP(S2, S1, 2)
      KS_DQ_STEP(S3, S2, 3)
    }
#undef KS_DQ_STEP
    wait_vm<0>();  // the window's last (re-staged) loads land before reuse
    bar_nofence();
  }

  if (qi < N) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqa[db][r] *= scale;
    if constexpr (ROPE)  // gradient with respect to the unrotated query
      rotate_back(dqa, rtab + (static_cast<size_t>(b) * N + qi) * (D / 2), lh);
    bf16_t* op = dq + (static_cast<size_t>(b) * N + qi) * tokq + static_cast<size_t>(hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = db * 32 + rg * 8 + lh * 4;
        const f32x16& a = dqa[db];
        *reinterpret_cast<u32x2*>(op + d) = u32x2{pack_bf16x2(a[rg * 4], a[rg * 4 + 1]),
                                                  pack_bf16x2(a[rg * 4 + 2], a[rg * 4 + 3])};
      }
  }
}

int padded_rows(int N) { return (N + BQ - 1) / BQ * BQ; }

// one of the two halves of the LSE / D_i records, [B][Hq][Npad] floats
size_t di_bytes(int B, int N, int Hq) {
  return (static_cast<size_t>(B) * Hq * padded_rows(N) * sizeof(float) + 255) &
         ~static_cast<size_t>(255);
}

}  // namespace
}  // namespace ksattn

using namespace ksattn;

extern "C" size_t ks_evict_attn_bwd_workspace(int B, int N, int Hq, int Hkv, int Dh, int dtype) {
  (void)Hkv;
  (void)Dh;
  (void)dtype;
  if (B <= 0 || N <= 0 || Hq <= 0) return 0;
  return summary_bytes(B, N) + 2 * di_bytes(B, N, Hq);
}

namespace {

// The two backward launches (dQ, then dK/dV) after the argument checks;
// rtab non-null selects the kernels that rotate the gradients back.
ks_status launch_bwd(const char* name, const bf16_t* qq, const bf16_t* kk, const bf16_t* vv,
                     const int32_t* e, const bf16_t* oo, const float* lse, const bf16_t* gg,
                     bf16_t* dq, bf16_t* dk, bf16_t* dv, int B, int N, int Hq, int Hkv,
                     float scale, void* ws, const float2* rtab, hipStream_t s) {
  const int hpw = ks_heads_per_wave(Hq / Hkv);
  TileSummary ts;
  ks_status st = launch_summary(e, ws, B, N, s, &ts);
  if (st != KS_OK) return st;
  float* rec = reinterpret_cast<float*>(static_cast<char*>(ws) + summary_bytes(B, N));
  const int Npad = padded_rows(N);
  const int ntiles = (N + kKeyTile - 1) / kKeyTile;

  // dQ first: it forms D_i and the LSE records of every row, which dK/dV reads
  const int rs = 8 / hpw;
  const int nqt = (N + 32 * rs - 1) / (32 * rs);
  const long long real_q = static_cast<long long>(B) * (Hq / hpw) * nqt;
  const long long total_q = (real_q + 7) / 8 * 8;
  KS_REQUIRE(total_q < (1LL << 31), "%s: grid too large", name);
  const int nkt = (N + KW - 1) / KW;
  const long long nkv = static_cast<long long>(B) * Hkv * nkt;
  KS_REQUIRE(nkv < (1LL << 31), "%s: grid too large", name);
#define KS_DQ_LAUNCH(HPW_, R_)                                                                 \
  hipLaunchKernelGGL((dq_kernel<HPW_, R_>), dim3(static_cast<unsigned>(total_q)), dim3(512), 0, \
                     s, qq, kk, vv, ts, rec, oo, lse, gg, dq, B, N, Npad, Hq, Hkv, ntiles, nqt, \
                     static_cast<int>(total_q), scale, rtab)
  if (rtab) {
    if (hpw == 4) KS_DQ_LAUNCH(4, true);
    else if (hpw == 2) KS_DQ_LAUNCH(2, true);
    else KS_DQ_LAUNCH(1, true);
  } else {
    if (hpw == 4) KS_DQ_LAUNCH(4, false);
    else if (hpw == 2) KS_DQ_LAUNCH(2, false);
    else KS_DQ_LAUNCH(1, false);
  }
#undef KS_DQ_LAUNCH
  st = ks_check_launch(name);
  if (st != KS_OK) return st;
  if (rtab)
    hipLaunchKernelGGL(dkdv_kernel<true>, dim3(static_cast<unsigned>(nkv)), dim3(512), 0, s, qq,
                       kk, vv, e, ts.emin, ts.emax, rec, gg, dk, dv, B, N, Npad, Hq, Hkv, ntiles,
                       scale, rtab);
  else
    hipLaunchKernelGGL(dkdv_kernel<false>, dim3(static_cast<unsigned>(nkv)), dim3(512), 0, s, qq,
                       kk, vv, e, ts.emin, ts.emax, rec, gg, dk, dv, B, N, Npad, Hq, Hkv, ntiles,
                       scale, rtab);
  return ks_check_launch(name);
}

}  // namespace

extern "C" ks_status ks_evict_attn_bwd(const void* q, const void* k, const void* v,
                                       const int32_t* e, const void* o, const float* lse,
                                       const void* dout, void* dq, void* dk, void* dv, int B,
                                       int N, int Hq, int Hkv, int Dh, int dtype, float scale,
                                       void* ws, size_t ws_bytes, void* stream) {
  KS_REQUIRE(B >= 0 && N >= 0 && Hq > 0 && Hkv > 0, "ks_evict_attn_bwd: bad sizes");
  KS_REQUIRE(Hq % Hkv == 0, "ks_evict_attn_bwd: Hq %% Hkv != 0");
  KS_REQUIRE(scale > 0.f, "ks_evict_attn_bwd: scale must be positive");
  if (dtype != KS_BF16 || Dh != D)
    return ks_fail(KS_ERR_UNSUPPORTED, "ks_evict_attn_bwd: only bf16 with D=128 (dtype=%d D=%d)",
                   dtype, Dh);
  if (B == 0 || N == 0) return KS_OK;
  KS_REQUIRE(q && k && v && e && o && lse && dout && dq && dk && dv,
             "ks_evict_attn_bwd: null pointer");
  KS_REQUIRE(ks_aligned16(q) && ks_aligned16(k) && ks_aligned16(v) && ks_aligned16(o) &&
                 ks_aligned16(dout) && ks_aligned16(dq) && ks_aligned16(dk) && ks_aligned16(dv),
             "ks_evict_attn_bwd: tensors must be 16-byte aligned");
  const size_t need = summary_bytes(B, N) + 2 * di_bytes(B, N, Hq);
  if (!ws || ws_bytes < need)
    return ks_fail(KS_ERR_WORKSPACE, "ks_evict_attn_bwd: workspace %zu < %zu bytes", ws_bytes,
                   need);
  KS_REQUIRE(ks_aligned16(ws), "ks_evict_attn_bwd: workspace must be 16-byte aligned");
  return launch_bwd("ks_evict_attn_bwd", static_cast<const bf16_t*>(q),
                    static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), e,
                    static_cast<const bf16_t*>(o), lse, static_cast<const bf16_t*>(dout),
                    static_cast<bf16_t*>(dq), static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv),
                    B, N, Hq, Hkv, scale, ws, nullptr, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Backward of the RoPE-fused forward.  The forward's rotated q and k (q_rot,
// k_rot) are the operands; the (cos, sin) table of the logical positions is
// formed again in the workspace, and dQ and dK are rotated back by -theta in
// fp32 before their bf16 store, so they are the gradients with respect to
// the unrotated projections (the rotation is orthogonal, its transpose is
// its inverse; explainer, RoPE paragraph, for the logical positions).
// ---------------------------------------------------------------------------
extern "C" size_t ks_evict_attn_bwd_rope_workspace(int B, int N, int Hq, int Hkv, int Dh,
                                                   int dtype) {
  (void)Hkv;
  (void)dtype;
  if (B <= 0 || N <= 0 || Hq <= 0 || Dh <= 0) return 0;
  return summary_bytes(B, N) + 2 * di_bytes(B, N, Hq) + rope_table_bytes(B, N, Dh);
}

extern "C" ks_status ks_evict_attn_bwd_rope(const void* q_rot, const void* k_rot, const void* v,
                                            const int32_t* e, const int32_t* pos, const void* o,
                                            const float* lse, const void* dout, void* dq,
                                            void* dk, void* dv, int B, int N, int Hq, int Hkv,
                                            int Dh, int dtype, float scale, float base, void* ws,
                                            size_t ws_bytes, void* stream) {
  const char* name = "ks_evict_attn_bwd_rope";
  KS_REQUIRE(B >= 0 && N >= 0 && Hq > 0 && Hkv > 0, "%s: bad sizes", name);
  KS_REQUIRE(Hq % Hkv == 0, "%s: Hq %% Hkv != 0", name);
  KS_REQUIRE(scale > 0.f, "%s: scale must be positive", name);
  KS_REQUIRE(base > 1.0f, "%s: base must be > 1", name);
  if (dtype != KS_BF16 || Dh != D)
    return ks_fail(KS_ERR_UNSUPPORTED, "%s: only bf16 with D=128 (dtype=%d D=%d)", name, dtype,
                   Dh);
  if (B == 0 || N == 0) return KS_OK;
  KS_REQUIRE(q_rot && k_rot && v && e && pos && o && lse && dout && dq && dk && dv,
             "%s: null pointer", name);
  KS_REQUIRE(ks_aligned16(q_rot) && ks_aligned16(k_rot) && ks_aligned16(v) && ks_aligned16(o) &&
                 ks_aligned16(dout) && ks_aligned16(dq) && ks_aligned16(dk) && ks_aligned16(dv),
             "%s: tensors must be 16-byte aligned", name);
  const size_t base_need = summary_bytes(B, N) + 2 * di_bytes(B, N, Hq);
  const size_t need = base_need + rope_table_bytes(B, N, Dh);
  if (!ws || ws_bytes < need)
    return ks_fail(KS_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", name, ws_bytes, need);
  KS_REQUIRE(ks_aligned16(ws), "%s: workspace must be 16-byte aligned", name);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* table = reinterpret_cast<float2*>(static_cast<char*>(ws) + base_need);
  ks_status st = launch_rope_prep(nullptr, nullptr, pos, table, static_cast<long long>(B) * N,
                                  Hkv, Dh, base, s);
  if (st != KS_OK) return st;
  return launch_bwd(name, static_cast<const bf16_t*>(q_rot), static_cast<const bf16_t*>(k_rot),
                    static_cast<const bf16_t*>(v), e, static_cast<const bf16_t*>(o), lse,
                    static_cast<const bf16_t*>(dout), static_cast<bf16_t*>(dq),
                    static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), B, N, Hq, Hkv, scale, ws,
                    table, s);
}
