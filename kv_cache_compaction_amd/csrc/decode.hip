// Paged GQA decode over compacted block tables.
//
// After compaction the block table lists only surviving 16-token blocks
// (KV-streams explainer, block-table paragraph), and cached keys carry the
// rotation of their logical positions (explainer, RoPE paragraph), so one
// decode step is plain softmax attention of the new query over the tokens
// reached through the table.
//
// Kernel 1 (split): one 64-lane wave per (sequence, group of HPW query heads
// of one kv head, split of 48 blocks, or 16 when the grid would be small:
// split_groups).  The split's block ids are read
// once, one per lane; each block's id is then taken with readlane.  Lane
// (t, g) = (lane % 16, lane / 16) owns token slot t of every block and the 32
// head-dim entries
// d = 32s + 8g + i (s, i < 4, 8).  Per block each lane issues four 16-byte
// loads of K and four of V at those entries, so every load instruction covers
// 64 contiguous bytes of each of the block's 16 token rows.
//   * Q K^T runs on the 16x16x32 bf16 MFMA: A = Q (rows = heads, replicated),
//     B = K^T (columns = the 16 tokens).  The result leaves S[h][t] in lane
//     (t, any g), i.e. exactly where the PV step needs it.
//   * P V is VALU work: lane (t, g) accumulates p[h][t] * v[t][d] for its
//     32 entries and HPW heads (FMA count is fixed by the problem; this
//     layout needs no cross-lane traffic in the loop).
//   * Softmax is online per lane with a lazily updated maximum: the running
//     max only moves when a score exceeds it by more than 2^kTau, so the
//     accumulator is rescaled on a handful of blocks instead of every block.
//   * At the end the 16 token slots are merged with DPP row rotations.
// Kernel 2 (reduce): merges the splits of each (sequence, head).
//
// Single-token blocks (BS = 1, the SGLang setup: explainer, paragraph on
// padding completions to whole blocks): the table lists one pool slot per
// token and the pool is [slots, Hkv, D].  The same kernels run over groups
// of 16 consecutive table entries; the split's slot ids (up to 768) are
// staged in LDS once and lane (t, g) reads the id of its own token slot t of each group, so
// every load instruction still covers 64 contiguous bytes of 16 token rows
// (now 16 separate rows of the pool).
//
// Memory: K and V of every live token are read from HBM once per step; the
// split partials add 4(D+2) bytes per (sequence, head, split).  The grid runs
// head groups fastest, so the Hkv waves reading the slices of one pool block
// (Hkv x 16 x D contiguous elements of K, and of V) run side by side, which
// keeps the DRAM accesses of concurrent waves on the same rows.  When a kv
// head has more query heads than one wave takes, its waves are placed on
// one XCD, whose L2 then serves the second read of its slices.
#include <mutex>

#include "ks_common.h"

namespace {

constexpr int D = 128;
constexpr int kSplit = 48;     // 16-token groups per split (block ids fit one wave)
static_assert(kSplit <= 64, "one block id per lane");
// Shorter splits when 48-group splits would give a small grid (fewer than
// kFewWaves waves, about two rounds of the GPU's wave slots): a step then
// spends most of its time in the last waves' full splits, while in large
// grids every extra split is extra start-up, merge and partial traffic.
constexpr int kSplitSmall = 16;
constexpr long long kFewWaves = 4096;
constexpr float kTau = 8.0f;   // lazy-rescale slack, log2 units

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// all-reduce over the 16 lanes of a DPP row
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0x128>(x);  // row_ror:8
  x += dpp<0x124>(x);  // row_ror:4
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  return x;
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0xB1>(x));
  return x;
}

struct BlockRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// BS = tokens per pool block (16, or 1: one pool slot per token).  MB = table
// entries per sequence, NB = pool blocks (slots when BS = 1).
template <int HPW, int BS>
__global__ __launch_bounds__(64) void decode_split_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kpool,
    const bf16_t* __restrict__ vpool, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_o,
    float* __restrict__ part_ml, int Hq, int Hkv, int MB, int NB, int nsplit_max, int sg,
    float sl2, const int32_t* __restrict__ qpos, double log2_base) {
  static_assert(BS == 16 || BS == 1, "block size");
  const int G = Hq / Hkv;
  // the G / HPW waves of one kv head read the same K/V slices: x = kv + Hkv *
  // sub puts them Hkv workgroups apart, and consecutive workgroups go to the
  // XCDs in turn, so with Hkv a multiple of 8 they share one XCD's L2
  const int hw = (blockIdx.x % Hkv) * (G / HPW) + blockIdx.x / Hkv;
  const int split = blockIdx.y, b = blockIdx.z;
  const int hq0 = hw * HPW;
  const int hkv = hq0 / G;
  // lengths beyond the table's capacity are clamped: nothing past a table
  // row is ever read
  const int L = min(max(seq_lens[b], 0), BS * MB);
  const int nblk = (L + 15) >> 4;     // 16-token groups
  const int blk0 = split * sg;
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + sg);
  const int lane = threadIdx.x;
  const int t = lane & 15, g = lane >> 4;

  bf16x8 qa[4];
  {
    const bf16_t* qrow = q + (static_cast<size_t>(b) * Hq + hq0 + (t % HPW)) * D + g * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = *reinterpret_cast<const bf16x8*>(qrow + s * 32);
  }
  float m[HPW], l[HPW], acc[HPW][32];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m[h] = -1e30f;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[h][i] = 0.f;
  }
  const int32_t* trow = table + static_cast<size_t>(b) * MB;
  bool bad = false;
  // BS = 16: the split's block ids, one per lane, read once; block blk's id
  // is then a wave-uniform value and its K/V loads do not wait on a table
  // load.  BS = 1: the split's slot ids (16 per group) staged in LDS.
  int pids = 0;
  __shared__ int sid[BS == 1 ? kSplit * 16 : 1];
  if constexpr (BS == 16) {
    pids = lane < blk1 - blk0 ? trow[blk0 + lane] : 0;
  } else {
    constexpr int kPerLane = kSplit * 16 / 64;
    int v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int tok = blk0 * 16 + i * 64 + lane;
      v[i] = tok < min(L, blk1 * 16) ? trow[tok] : 0;
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) sid[i * 64 + lane] = v[i];
    __syncthreads();
  }
  const size_t lane_off = static_cast<size_t>(BS == 16 ? t : 0) * D + g * 8;

  auto load = [&](int blk, BlockRegs& r) {
    const int pid = BS == 16 ? __builtin_amdgcn_readlane(pids, blk - blk0)
                             : sid[(blk - blk0) * 16 + t];
    const bool ok = static_cast<unsigned>(pid) < static_cast<unsigned>(NB);
    bad |= !ok;
    const size_t off = (static_cast<size_t>(ok ? pid : 0) * Hkv + hkv) * BS * D + lane_off;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      r.k[s] = *reinterpret_cast<const u32x4*>(kpool + off + s * 32);
      r.v[s] = *reinterpret_cast<const u32x4*>(vpool + off + s * 32);
    }
  };

  auto compute = [&](int blk, BlockRegs& r) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sacc = mfma16x16x32(qa[s], __builtin_bit_cast(bf16x8, r.k[s]), sacc);
    // The scores are read by VALU code below, on both sides of the tail-block
    // branch.  The hardware does not interlock an MFMA result with a VALU
    // read: v_mfma_f32_16x16x32_bf16 needs 8 independent wait states first
    // (the gfx950 backend's own requirement for this instruction).  They
    // are issued explicitly here, fenced so that no read can move above them,
    // instead of relying on the compiler's placement across the branch.
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
    const bool valid = blk * 16 + t < L;
    if ((blk + 1) * 16 > L) {  // tail block: slots past L may hold anything
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[s][i] = valid ? r.v[s][i] : 0u;
    }
    float sc[HPW];
    bool need_any = false;
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      sc[h] = valid ? sacc[h] * sl2 : -INFINITY;
      need_any |= sc[h] > m[h] + kTau;
    }
    if (__ballot(need_any)) {
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        const bool need = sc[h] > m[h] + kTau;
        const float f = need ? fast_exp2(m[h] - sc[h]) : 1.f;
        m[h] = need ? sc[h] : m[h];
        l[h] *= f;
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[h][i] *= f;
      }
    }
    float vf[32];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[s * 8 + 2 * i] = lo_bf16(r.v[s][i]);
        vf[s * 8 + 2 * i + 1] = hi_bf16(r.v[s][i]);
      }
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float p = fast_exp2(sc[h] - m[h]);
      l[h] += p;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[h][i] = fmaf(p, vf[i], acc[h][i]);
    }
  };

  BlockRegs r0, r1;
  load(blk0, r0);
  if (qpos) {
    // q arrives unrotated: rotate it at its logical position.  Lane k forms
    // (cos, sin) of pair k once; lane (t, g) holds d = 32 s + 8 g + i, so its
    // pairs (d, d + 64) are fragments s and s + 2 of its own registers.
    const float2 csl = rope_cos_sin(static_cast<double>(qpos[b]), lane, D, log2_base);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kk = 32 * s + 8 * g + i;
        const float2 cs = make_float2(__shfl(csl.x, kk), __shfl(csl.y, kk));
        float x = static_cast<float>(qa[s][i]), y = static_cast<float>(qa[s + 2][i]);
        rope_rotate(x, y, cs);
        qa[s][i] = static_cast<__bf16>(x);
        qa[s + 2][i] = static_cast<__bf16>(y);
      }
  }
  int blk = blk0;
  for (; blk + 1 < blk1; blk += 2) {
    load(blk + 1, r1);
    compute(blk, r0);
    if (blk + 2 < blk1) load(blk + 2, r0);
    compute(blk + 1, r1);
  }
  if (blk < blk1) compute(blk, r0);

  // with single-token blocks a bad slot id is seen by one lane only
  if (BS == 1) bad = __ballot(bad) != 0;
  // merge the 16 token slots of each lane row (lanes with equal g)
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float M = row_max16(m[h]);
    const float f = fast_exp2(m[h] - M);
    float lsum = row_sum16(l[h] * f);
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[h][i] = row_sum16(acc[h][i] * f);
    if (bad) lsum = NAN;
    if (t == 0) {
      const size_t slot = (static_cast<size_t>(b) * Hq + hq0 + h) * nsplit_max + split;
      float* po = part_o + slot * D + g * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f32x4* p4 = reinterpret_cast<f32x4*>(po + s * 32);
        p4[0] = f32x4{acc[h][s * 8 + 0], acc[h][s * 8 + 1], acc[h][s * 8 + 2], acc[h][s * 8 + 3]};
        p4[1] = f32x4{acc[h][s * 8 + 4], acc[h][s * 8 + 5], acc[h][s * 8 + 6], acc[h][s * 8 + 7]};
      }
      if (g == 0) {
        part_ml[slot * 2 + 0] = M;
        part_ml[slot * 2 + 1] = lsum;
      }
    }
  }
}

// cap = tokens one table row can reach (BS * entries)
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, bf16_t* __restrict__ out, float* __restrict__ lse,
    int Hq, int cap, int nsplit_max, int sg) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), cap);
  const int ns = (((L + 15) >> 4) + sg - 1) / sg;
  const size_t slot0 = (static_cast<size_t>(b) * Hq + h) * nsplit_max;
  // splits in groups of 16 whose loads are all issued before their use (a
  // plain loop waits for each load in turn); the sums run in split order
  constexpr int U = 16;
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += U) {
    float m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = s0 + u < ns ? part_ml[(slot0 + s0 + u) * 2] : -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, m[u]);
  }
  float den = 0.f, num = 0.f;
  for (int s0 = 0; s0 < ns; s0 += U) {
    float m[U], l[U], x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t sl = slot0 + min(s0 + u, ns - 1);
      m[u] = part_ml[sl * 2];
      l[u] = part_ml[sl * 2 + 1];
      x[u] = part_o[sl * D + d];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < ns) {
        const float f = fast_exp2(m[u] - M);
        den += l[u] * f;
        num += x[u] * f;
      }
    }
  }
  const size_t o = (static_cast<size_t>(b) * Hq + h) * D + d;
  if (ns == 0) {
    out[o] = 0;
    if (lse && d == 0) lse[static_cast<size_t>(b) * Hq + h] = -INFINITY;
    return;
  }
  out[o] = f32_to_bf16(num / den);
  if (lse && d == 0) lse[static_cast<size_t>(b) * Hq + h] = (M + __log2f(den)) * KS_LN2;
}

// ---------------------------------------------------------------------------
// append: rotate the new token's key at its logical position and write key
// and value into token slot seq_len - 1 (block table entry (seq_len - 1) / BS).
// Keys are stored already rotated, so later compaction can move blocks
// without touching their contents (explainer, RoPE paragraph).  One
// workgroup per sequence; angles in fp64 as in ks_rope_logical.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(256) void append_kernel(
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, bf16_t* __restrict__ kpool,
    bf16_t* __restrict__ vpool, int Hkv, int MB, int NB, double log2_base) {
  __shared__ float2 cs[D / 2];
  const int b = blockIdx.x;
  const int L = min(seq_lens[b], BS * MB);
  if (L < 1) return;
  const int slot = L - 1;
  const int pid = table[static_cast<size_t>(b) * MB + slot / BS];
  if (static_cast<unsigned>(pid) >= static_cast<unsigned>(NB)) return;
  for (int kk = threadIdx.x; kk < D / 2; kk += blockDim.x)
    cs[kk] = rope_cos_sin(static_cast<double>(pos[b]), kk, D, log2_base);
  __syncthreads();
  // thread = (head, 8-element chunk of the first half)
  for (int idx = threadIdx.x; idx < Hkv * (D / 16); idx += blockDim.x) {
    const int h = idx / (D / 16), ch = idx % (D / 16);
    const size_t src = (static_cast<size_t>(b) * Hkv + h) * D + ch * 8;
    const size_t dst = ((static_cast<size_t>(pid) * Hkv + h) * BS + slot % BS) * D + ch * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(k_new + src);
    const u32x4 bb = *reinterpret_cast<const u32x4*>(k_new + src + D / 2);
    u32x4 ra, rb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x0 = lo_bf16(a[i]), x1 = hi_bf16(a[i]);
      float y0 = lo_bf16(bb[i]), y1 = hi_bf16(bb[i]);
      rope_rotate(x0, y0, cs[ch * 8 + 2 * i]);
      rope_rotate(x1, y1, cs[ch * 8 + 2 * i + 1]);
      ra[i] = pack_bf16x2(x0, x1);
      rb[i] = pack_bf16x2(y0, y1);
    }
    *reinterpret_cast<u32x4*>(kpool + dst) = ra;
    *reinterpret_cast<u32x4*>(kpool + dst + D / 2) = rb;
    *reinterpret_cast<u32x4*>(vpool + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
    *reinterpret_cast<u32x4*>(vpool + dst + D / 2) =
        *reinterpret_cast<const u32x4*>(v_new + src + D / 2);
  }
}

// 16-token groups per split for B sequences of Hq query heads over table
// rows of `groups` groups: decided from the sizes alone (the workspace query
// and the launch see the same ones), with the waves counted at four query
// heads per wave
inline int split_groups(int B, int Hq, int groups) {
  const long long waves = static_cast<long long>(B) * ((Hq + 3) / 4) *
                          ((groups + kSplit - 1) / kSplit);
  return waves < kFewWaves ? kSplitSmall : kSplit;
}

// splits for a table row of `groups` 16-token groups, `sg` groups per split
inline int nsplit_for(int groups, int sg) { return (groups + sg - 1) / sg; }

inline size_t decode_workspace(int B, int Hq, int Dh, int groups) {
  if (B <= 0 || Hq <= 0 || Dh <= 0 || groups <= 0) return 0;
  const size_t slots =
      static_cast<size_t>(B) * Hq * nsplit_for(groups, split_groups(B, Hq, groups));
  return slots * (static_cast<size_t>(Dh) + 2) * sizeof(float) + 256;
}

template <int BS>
ks_status decode_impl(const char* name, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* table, const int32_t* seq_lens, void* out, float* lse, int B,
                      int Hq, int Hkv, int Dh, int max_entries, int num_pool, int dtype,
                      float scale, void* ws, size_t ws_bytes, void* stream,
                      const int32_t* qpos = nullptr, float base = 0.f) {
  KS_REQUIRE(B >= 0 && Hq > 0 && Hkv > 0 && max_entries >= 0 && num_pool >= 0,
             "%s: bad sizes", name);
  KS_REQUIRE(Hq % Hkv == 0, "%s: Hq %% Hkv != 0", name);
  if (dtype != KS_BF16 || Dh != D)
    return ks_fail(KS_ERR_UNSUPPORTED, "%s: only bf16 with D=128 (got dtype=%d D=%d)", name,
                   dtype, Dh);
  const int G = Hq / Hkv;
  const int hpw = ks_heads_per_wave(G);
  if (B == 0) return KS_OK;
  KS_REQUIRE(q && seq_lens && out, "%s: null pointer", name);
  // with no table entries nothing is read through the table, so the table
  // and the pools may be empty; otherwise an out-of-range id falls back to
  // pool block 0, which must exist
  KS_REQUIRE(max_entries == 0 || num_pool > 0, "%s: the pool has no blocks", name);
  KS_REQUIRE(max_entries == 0 || (table && k_pool && v_pool), "%s: null pointer", name);
  KS_REQUIRE(ks_aligned16(q) && ks_aligned16(k_pool) && ks_aligned16(v_pool) && ks_aligned16(out),
             "%s: tensors must be 16-byte aligned", name);
  const double log2_base = qpos ? log2(static_cast<double>(base)) : 0.0;
  KS_REQUIRE(static_cast<int64_t>(max_entries) * BS < (int64_t{1} << 31),
             "%s: table row too long", name);
  // max_entries == 0: every length clamps to 0 and no table entry is read
  const int groups = max_entries > 0 ? (max_entries * BS + 15) / 16 : 1;
  const size_t need = decode_workspace(B, Hq, Dh, groups);
  if (!ws || ws_bytes < need)
    return ks_fail(KS_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", name, ws_bytes, need);
  const int sg = split_groups(B, Hq, groups);
  const int nsplit = nsplit_for(groups, sg);
  KS_REQUIRE(nsplit < 65536 && B < 65536, "%s: grid too large", name);
  float* part_ml = static_cast<float*>(ws);
  const size_t slots = static_cast<size_t>(B) * Hq * nsplit;
  float* part_o = reinterpret_cast<float*>(
      (reinterpret_cast<uintptr_t>(part_ml + 2 * slots) + 255) & ~static_cast<uintptr_t>(255));
  const float sl2 = scale * KS_LOG2E;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // head groups fastest: the waves that read the kv-head slices of the same
  // pool blocks (contiguous in memory) are dispatched together
  const dim3 grid(Hq / hpw, nsplit, B);
  const bf16_t* qq = static_cast<const bf16_t*>(q);
  const bf16_t* kp = static_cast<const bf16_t*>(k_pool);
  const bf16_t* vp = static_cast<const bf16_t*>(v_pool);
  if (hpw == 4)
    hipLaunchKernelGGL((decode_split_kernel<4, BS>), grid, dim3(64), 0, s, qq, kp, vp, table,
                       seq_lens, part_o, part_ml, Hq, Hkv, max_entries, num_pool, nsplit, sg, sl2,
                       qpos, log2_base);
  else if (hpw == 2)
    hipLaunchKernelGGL((decode_split_kernel<2, BS>), grid, dim3(64), 0, s, qq, kp, vp, table,
                       seq_lens, part_o, part_ml, Hq, Hkv, max_entries, num_pool, nsplit, sg, sl2,
                       qpos, log2_base);
  else
    hipLaunchKernelGGL((decode_split_kernel<1, BS>), grid, dim3(64), 0, s, qq, kp, vp, table,
                       seq_lens, part_o, part_ml, Hq, Hkv, max_entries, num_pool, nsplit, sg, sl2,
                       qpos, log2_base);
  ks_status st = ks_check_launch(name);
  if (st != KS_OK) return st;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(Hq, B), dim3(D), 0, s, part_o, part_ml, seq_lens,
                     static_cast<bf16_t*>(out), lse, Hq, max_entries * BS, nsplit, sg);
  return ks_check_launch(name);
}

template <int BS>
ks_status append_impl(const char* name, const void* k_new, const void* v_new,
                      const int32_t* pos, const int32_t* table, const int32_t* seq_lens,
                      void* k_pool, void* v_pool, int B, int Hkv, int Dh, int max_entries,
                      int num_pool, int dtype, float base, void* stream) {
  KS_REQUIRE(B >= 0 && Hkv > 0 && max_entries >= 0 && num_pool >= 0, "%s: bad sizes", name);
  KS_REQUIRE(base > 1.0f, "%s: base must be > 1", name);
  if (dtype != KS_BF16 || Dh != D)
    return ks_fail(KS_ERR_UNSUPPORTED, "%s: only bf16 with D=128 (dtype=%d D=%d)", name, dtype,
                   Dh);
  if (B == 0 || max_entries == 0) return KS_OK;
  KS_REQUIRE(k_new && v_new && pos && table && seq_lens && k_pool && v_pool,
             "%s: null pointer", name);
  KS_REQUIRE(ks_aligned16(k_new) && ks_aligned16(v_new) && ks_aligned16(k_pool) &&
                 ks_aligned16(v_pool),
             "%s: tensors must be 16-byte aligned", name);
  KS_REQUIRE(static_cast<int64_t>(max_entries) * BS < (int64_t{1} << 31),
             "%s: table row too long", name);
  hipLaunchKernelGGL(append_kernel<BS>, dim3(B), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const bf16_t*>(k_new), static_cast<const bf16_t*>(v_new), pos,
                     table, seq_lens, static_cast<bf16_t*>(k_pool), static_cast<bf16_t*>(v_pool),
                     Hkv, max_entries, num_pool, log2(static_cast<double>(base)));
  return ks_check_launch(name);
}

}  // namespace

// A table row with no entries still gets the one-split workspace the launch
// asks for (every length clamps to 0 and the reduce writes the empty rows).
extern "C" size_t ks_paged_decode_workspace(int B, int Hq, int Dh, int max_blocks) {
  return decode_workspace(B, Hq, Dh, max_blocks > 0 ? max_blocks : 1);
}

extern "C" ks_status ks_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* table, const int32_t* seq_lens, void* out,
                                     float* lse, int B, int Hq, int Hkv, int Dh, int max_blocks,
                                     int num_pool_blocks, int dtype, float scale, void* ws,
                                     size_t ws_bytes, void* stream) {
  return decode_impl<16>("ks_paged_decode", q, k_pool, v_pool, table, seq_lens, out, lse, B, Hq,
                         Hkv, Dh, max_blocks, num_pool_blocks, dtype, scale, ws, ws_bytes,
                         stream);
}

extern "C" size_t ks_paged_decode_bs1_workspace(int B, int Hq, int Dh, int max_tokens) {
  return decode_workspace(B, Hq, Dh, max_tokens > 0 ? (max_tokens + 15) / 16 : 1);
}

extern "C" ks_status ks_paged_decode_bs1(const void* q, const void* k_pool, const void* v_pool,
                                         const int32_t* token_table, const int32_t* seq_lens,
                                         void* out, float* lse, int B, int Hq, int Hkv, int Dh,
                                         int max_tokens, int num_pool_tokens, int dtype,
                                         float scale, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl<1>("ks_paged_decode_bs1", q, k_pool, v_pool, token_table, seq_lens, out,
                        lse, B, Hq, Hkv, Dh, max_tokens, num_pool_tokens, dtype, scale, ws,
                        ws_bytes, stream);
}

extern "C" ks_status ks_paged_decode_rope(const void* q, const int32_t* pos, const void* k_pool,
                                          const void* v_pool, const int32_t* table,
                                          const int32_t* seq_lens, void* out, float* lse, int B,
                                          int Hq, int Hkv, int Dh, int max_entries,
                                          int num_pool, int block_size, int dtype, float scale,
                                          float base, void* ws, size_t ws_bytes, void* stream) {
  KS_REQUIRE(block_size == 16 || block_size == 1, "ks_paged_decode_rope: block_size %d",
             block_size);
  KS_REQUIRE(base > 1.0f, "ks_paged_decode_rope: base must be > 1");
  if (B > 0) KS_REQUIRE(pos, "ks_paged_decode_rope: pos is NULL");
  if (block_size == 16)
    return decode_impl<16>("ks_paged_decode_rope", q, k_pool, v_pool, table, seq_lens, out, lse,
                           B, Hq, Hkv, Dh, max_entries, num_pool, dtype, scale, ws, ws_bytes,
                           stream, pos, base);
  return decode_impl<1>("ks_paged_decode_rope", q, k_pool, v_pool, table, seq_lens, out, lse, B,
                        Hq, Hkv, Dh, max_entries, num_pool, dtype, scale, ws, ws_bytes, stream,
                        pos, base);
}

extern "C" ks_status ks_append_kv(const void* k_new, const void* v_new, const int32_t* pos,
                                  const int32_t* table, const int32_t* seq_lens, void* k_pool,
                                  void* v_pool, int B, int Hkv, int Dh, int max_blocks,
                                  int num_pool_blocks, int dtype, float base, void* stream) {
  return append_impl<16>("ks_append_kv", k_new, v_new, pos, table, seq_lens, k_pool, v_pool, B,
                         Hkv, Dh, max_blocks, num_pool_blocks, dtype, base, stream);
}

extern "C" ks_status ks_append_kv_bs1(const void* k_new, const void* v_new, const int32_t* pos,
                                      const int32_t* token_table, const int32_t* seq_lens,
                                      void* k_pool, void* v_pool, int B, int Hkv, int Dh,
                                      int max_tokens, int num_pool_tokens, int dtype, float base,
                                      void* stream) {
  return append_impl<1>("ks_append_kv_bs1", k_new, v_new, pos, token_table, seq_lens, k_pool,
                        v_pool, B, Hkv, Dh, max_tokens, num_pool_tokens, dtype, base, stream);
}

// ---------------------------------------------------------------------------
// ks_paged_decode_noalloc: ks_paged_decode with its split partials kept in a
// device array the library owns, for callers that cannot allocate.  The
// array lives for the whole process on every GPU the library runs on; one
// copy per device, found once per device with hipGetSymbolAddress (in host
// code `scratch` names a host-side stand-in, never the device memory).
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t{96} << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// the device address of this device's scratch array (looked up on the first
// call on that device, with that device current)
static ks_status scratch_on(hipStream_t stream, const char* name, void** out) {
  int dev = -1;
  hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (err != hipSuccess)
    return ks_fail(KS_ERR_HIP, "%s: device of the stream: %s", name, hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return ks_fail(KS_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", name,
                   dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = -1;
    err = hipGetDevice(&cur);
    if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
    void* p = nullptr;
    if (err == hipSuccess) err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    if (err != hipSuccess || !p)
      return ks_fail(KS_ERR_HIP, "%s: scratch address on device %d: %s", name, dev,
                     hipGetErrorString(err));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return KS_OK;
}

extern "C" size_t ks_paged_decode_noalloc_max_scratch(void) { return kScratchBytes; }

extern "C" ks_status ks_paged_decode_noalloc(const void* q, const void* k_pool,
                                             const void* v_pool, const int32_t* table,
                                             const int32_t* seq_lens, void* out, float* lse,
                                             int B, int Hq, int Hkv, int Dh, int max_blocks,
                                             int num_pool_blocks, int dtype, float scale,
                                             void* stream) {
  const char* name = "ks_paged_decode_noalloc";
  if (B > 0 && Hq > 0 && Dh > 0) {
    const size_t need = decode_workspace(B, Hq, Dh, max_blocks > 0 ? max_blocks : 1);
    if (need > kScratchBytes)
      return ks_fail(KS_ERR_WORKSPACE,
                     "%s: needs %zu bytes of split partials (B=%d, Hq=%d, max_blocks=%d), "
                     "more than its %zu-byte scratch; use ks_paged_decode with a workspace",
                     name, need, B, Hq, max_blocks, kScratchBytes);
  }
  void* ws = nullptr;
  if (B > 0) {
    const ks_status st = scratch_on(static_cast<hipStream_t>(stream), name, &ws);
    if (st != KS_OK) return st;
  }
  return decode_impl<16>(name, q, k_pool, v_pool, table, seq_lens, out, lse, B, Hq, Hkv, Dh,
                         max_blocks, num_pool_blocks, dtype, scale, ws, kScratchBytes, stream);
}
