/*
 * ks.h -- C ABI of libks.so, the KV-streams hot path for AMD MI355X (gfx950).
 *
 * KV-streams ("KV-streams for Efficient Compaction in Agentic Reinforcement
 * Learning", Penaloza et al.) compacts an agent's live KV cache by splicing
 * evicted turns out of it instead of re-prefilling a shorter sequence.  The
 * trainer then replays the recorded compaction events as an attention mask
 * over the continuous trace.  This library provides the GPU kernels of both
 * sides: RoPE at logical positions, eviction-masked attention forward and
 * backward, block-table compaction and paged GQA decode.
 *
 * Citations in these sources name two web pages about the method: "the
 * explainer" is the wqu.guru article "KV-streams: accelerating agentic RL
 * training by operating on the KV cache directly" (its paragraphs on RoPE,
 * 16-token blocks and the block table, padding, turn-level eviction and the
 * trainer), and "the paper page" is the thelatestinai.com summary of the
 * paper above (abstract, Fig. 2A, Fig. 3, Tables 1-2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory      Every tensor pointer is DEVICE memory owned by the caller.  The
 *             library never allocates: scratch space comes from a caller
 *             workspace whose size is given by the matching *_workspace()
 *             query.  Pointers must be 16-byte aligned.
 * Layouts     Row-major and contiguous.  Trace tensors are [B, N, H, D]
 *             ("BSHD"); the paged pool is [num_blocks, Hkv, 16, D].
 * Streams     `stream` is a hipStream_t (NULL = the null stream).  Every call
 *             is asynchronous on that stream; nothing synchronises the host.
 * GQA         Hq % Hkv == 0; query head h reads kv head h / (Hq / Hkv).
 * Errors      Arguments are validated before anything is launched.  A non-OK
 *             status means nothing was written.  A launch failure returns
 *             KS_ERR_HIP.  ks_last_error() gives a message for the last
 *             non-OK status of the calling thread.  Nothing is printed,
 *             thrown or aborted across the ABI.  All entry points are
 *             reentrant; calls that share output or workspace buffers on
 *             different streams race.
 */
#ifndef KS_H
#define KS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int ks_status;
#define KS_OK 0
#define KS_ERR_INVALID_ARG 1
#define KS_ERR_UNSUPPORTED 2
#define KS_ERR_HIP 3
#define KS_ERR_WORKSPACE 4

/* element types */
#define KS_F32 0
#define KS_BF16 1

/* e_j of a token that is never evicted */
#define KS_NEVER 0x7fffffff
/* tokens per paged KV block */
#define KS_BLOCK 16

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ks_last_error(void);

/* Library version string. */
const char* ks_version(void);

/*
 * ks_rope_logical -- rotate queries and keys by their LOGICAL position.
 *
 * After compaction a retained key may sit in a different physical slot, but
 * it keeps the rotation of its original position, and new queries and keys
 * continue the original position count (KV-streams explainer on wqu.guru,
 * the paragraph on RoPE and the one that separates physical storage from
 * logical position).
 *
 * Rotate-half (NeoX) pairing: for k < D/2, theta = pos * base^(-2k/D),
 *   x[k]       <- x[k] cos(theta) - x[k + D/2] sin(theta)
 *   x[k + D/2] <- x[k + D/2] cos(theta) + x[k] sin(theta).
 * The angle is formed and reduced in fp64; the rotation runs in fp32 and is
 * rounded once to the storage type.  inverse != 0 rotates by -theta (the
 * transpose, i.e. the backward of the rotation).
 *
 * q    [B, N, Hq, D]  in place (may be NULL when Hq == 0 or q is not wanted)
 * k    [B, N, Hkv, D] in place (may be NULL likewise)
 * pos  int32 [B, N]   logical positions (device)
 * dtype KS_F32 or KS_BF16; D even, 2 <= D <= 256, D % 16 == 0.
 */
ks_status ks_rope_logical(void* q, void* k, const int32_t* pos, int B, int N,
                          int Hq, int Hkv, int D, int dtype, float base,
                          int inverse, void* stream);

/*
 * ks_evict_attn_fwd -- attention over a continuous trace under the eviction
 * mask that reproduces compaction.
 *
 * Training replays the logged compaction events: every surviving entry is
 * the one computed when its token was generated, and a token evicted at an
 * event is invisible to every later query (explainer, trainer paragraph;
 * paper page, Fig. 2A, where the mask stands for the eviction).  With e_j the
 * trace index of the event that evicted token j (KS_NEVER if never):
 *   M_ij = [j <= i] and [i < e_j]
 *   LSE_i = log sum_{j: M_ij} exp(scale q_i.k_j)
 *   O_i   = sum_{j: M_ij} exp(scale q_i.k_j - LSE_i) v_j
 * Key tiles that no query of a tile can see are skipped using the per-tile
 * minimum and maximum of e.
 *
 * q    [B, N, Hq, D]   (rotated; dtype)
 * k, v [B, N, Hkv, D]  (k rotated; dtype)
 * e    int32 [B, N]    must satisfy e_j > j; any value >= N means "never".
 *                      (If it does not, token j is seen by no query; a row
 *                      that sees no key gets O = 0 and LSE = -inf, and no
 *                      gradient flows through it.)
 * o    [B, N, Hq, D]   output (dtype)
 * lse  float [B, Hq, N] output, natural log, may be NULL
 * dtype KS_BF16 (D = 128 or 64, fp32 accumulation) or KS_F32 (D <= 128,
 *       D % 16 == 0).
 * ws   workspace of at least ks_evict_attn_fwd_workspace() bytes.
 */
size_t ks_evict_attn_fwd_workspace(int B, int N, int Hq, int Hkv, int D,
                                   int dtype);
ks_status ks_evict_attn_fwd(const void* q, const void* k, const void* v,
                            const int32_t* e, void* o, float* lse, int B,
                            int N, int Hq, int Hkv, int D, int dtype,
                            float scale, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * ks_evict_attn_bwd -- gradients of ks_evict_attn_fwd.
 *
 * Softmax backward over the same mask (the pages state none; this is the
 * calculus of the forward above):
 *   P = exp(S - LSE), dV_j = sum_i P_ij dO_i, dP_ij = dO_i.v_j,
 *   D_i = sum_j P_ij dP_ij = dO_i.O_i, dS = P (dP - D_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
 * dK and dV sum over the query heads that share a kv head.  Gradients are
 * with respect to the rotated q and k (apply ks_rope_logical with inverse=1
 * to obtain gradients of the raw projections).  Deterministic: no atomics.
 *
 * o, lse  outputs of the forward on the same inputs (lse required)
 * dout    [B, N, Hq, D] upstream gradient (dtype)
 * dq      [B, N, Hq, D], dk, dv [B, N, Hkv, D] outputs (dtype)
 * dtype   KS_BF16 with D = 128.
 */
size_t ks_evict_attn_bwd_workspace(int B, int N, int Hq, int Hkv, int D,
                                   int dtype);
ks_status ks_evict_attn_bwd(const void* q, const void* k, const void* v,
                            const int32_t* e, const void* o, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv,
                            int B, int N, int Hq, int Hkv, int D, int dtype,
                            float scale, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * ks_evict_attn_fwd_rope -- ks_rope_logical and ks_evict_attn_fwd in one
 * call, for the training step.
 *
 * Queries and keys arrive UNROTATED; every token is rotated at its logical
 * position pos (explainer, the RoPE paragraph; same angles and rounding as
 * ks_rope_logical, so q_rot, k_rot, o and lse are bit-identical to
 * ks_rope_logical followed by ks_evict_attn_fwd).  The keys are rotated
 * once, out of place, into k_rot; each query row is rotated in registers by
 * the attention kernel, which also stores it to q_rot.  q and k are not
 * modified.  q_rot and k_rot are what ks_evict_attn_bwd_rope takes.
 *
 * q      [B, N, Hq, D] unrotated queries;  k, v [B, N, Hkv, D]
 * e      int32 [B, N] as in ks_evict_attn_fwd; pos int32 [B, N] (device)
 * q_rot  [B, N, Hq, D], k_rot [B, N, Hkv, D] outputs; q_rot, k_rot and o
 *        must not overlap q, k, v or each other (KS_ERR_INVALID_ARG)
 * o, lse outputs as in ks_evict_attn_fwd (lse required)
 * dtype  KS_BF16 with D = 128 (else KS_ERR_UNSUPPORTED); base > 1.
 * ws     workspace of at least ks_evict_attn_fwd_rope_workspace() bytes
 *        (the tile summary and a [B*N][D/2] (cos, sin) table).
 */
size_t ks_evict_attn_fwd_rope_workspace(int B, int N, int Hq, int Hkv, int D,
                                        int dtype);
ks_status ks_evict_attn_fwd_rope(const void* q, const void* k, const void* v,
                                 const int32_t* e, const int32_t* pos,
                                 void* q_rot, void* k_rot, void* o, float* lse,
                                 int B, int N, int Hq, int Hkv, int D,
                                 int dtype, float scale, float base, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * ks_evict_attn_bwd_rope -- gradients of ks_evict_attn_fwd_rope with
 * respect to the UNROTATED q and k (and v).
 *
 * The softmax backward of ks_evict_attn_bwd on the rotated operands; dQ and
 * dK are then rotated by -theta in fp32 before their single rounding to
 * bf16 (the rotation is orthogonal, so its backward is its transpose).  This
 * replaces ks_evict_attn_bwd followed by ks_rope_logical(inverse=1) and
 * skips that second rounding, so dq and dk agree with it to one bf16 ulp,
 * not bit for bit; dv is bit-identical.
 *
 * q_rot, k_rot  the rotated operands written by ks_evict_attn_fwd_rope
 * pos, base     the logical positions and base given to the forward
 * other arguments as in ks_evict_attn_bwd; dtype KS_BF16 with D = 128.
 * ws            at least ks_evict_attn_bwd_rope_workspace() bytes.
 */
size_t ks_evict_attn_bwd_rope_workspace(int B, int N, int Hq, int Hkv, int D,
                                        int dtype);
ks_status ks_evict_attn_bwd_rope(const void* q_rot, const void* k_rot,
                                 const void* v, const int32_t* e,
                                 const int32_t* pos, const void* o,
                                 const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, int B, int N, int Hq,
                                 int Hkv, int D, int dtype, float scale,
                                 float base, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * ks_compact_block_table -- splice evicted blocks out of paged block tables.
 *
 * The table may not keep empty slots, so complete blocks are removed and the
 * remaining block references are joined, order preserved (explainer, the
 * paragraph on vLLM's 16-token blocks and the block table):
 *   out_b = [table_b[x] for x < nblk_in_b if keep_b[x]],  nblk_out_b = |out_b|,
 *   out_b[x] = -1 for x >= nblk_out_b.
 * If pos_in is given, the same selection is applied to it (e.g. the logical
 * index of each block) into pos_out.
 *
 * table_in, table_out  int32 [B, max_blocks] (device; must not alias)
 * nblk_in, nblk_out    int32 [B] (device; may alias each other); entries of
 *                      nblk_in are clamped to [0, max_blocks]
 * keep                 uint8 [B, max_blocks], nonzero = keep
 * pos_in, pos_out      int32 [B, max_blocks] or both NULL
 * With max_blocks = 0 only the lengths are touched (nblk_out = 0) and the
 * table, keep and pos pointers may be NULL.
 *
 * With single-token blocks (the SGLang setup: explainer, paragraph on padding
 * completions to whole blocks) the same call compacts token tables: entries
 * are pool slots, one per token, and max_blocks is the row length in tokens.
 * Rows longer than 4096 entries are split over several workgroups.
 */
ks_status ks_compact_block_table(const int32_t* table_in,
                                 const int32_t* nblk_in, const uint8_t* keep,
                                 int32_t* table_out, int32_t* nblk_out,
                                 const int32_t* pos_in, int32_t* pos_out,
                                 int B, int max_blocks, void* stream);

/*
 * ks_compact_block_table_rounds -- several compaction events in one launch.
 *
 * Same result as `rounds` successive ks_compact_block_table calls, where
 * event r applies keep[r] to the table left by events 0 .. r-1 (each event
 * is the splice above; a decoder that has several pending events before its
 * next step applies them together).  Intermediate tables are never written.
 *
 * keep      uint8 [rounds, B, max_blocks]; keep[r][b][x] refers to entry x of
 *           sequence b's table after r events
 * rounds    0 .. KS_MAX_ROUNDS; rounds = 0 copies the table (clamped length,
 *           -1 past it)
 * max_blocks at most KS_MAX_ROUND_BLOCKS: rows of up to 4096 entries are held
 *           on chip; longer rows (token tables of single-token blocks) keep
 *           one survival bit per entry on chip and read the row once at the
 *           end
 * other arguments and aliasing rules as for ks_compact_block_table.
 * Errors: KS_ERR_INVALID_ARG for rounds or max_blocks out of range.
 */
#define KS_MAX_ROUNDS 64
#define KS_MAX_ROUND_BLOCKS 65536
ks_status ks_compact_block_table_rounds(const int32_t* table_in,
                                        const int32_t* nblk_in,
                                        const uint8_t* keep, int rounds,
                                        int32_t* table_out, int32_t* nblk_out,
                                        const int32_t* pos_in, int32_t* pos_out,
                                        int B, int max_blocks, void* stream);

/*
 * ks_paged_decode -- one GQA decode step over compacted paged caches.
 *
 * Each sequence attends the first seq_lens[b] tokens reached through its
 * block table.  Keys in the pool were rotated at their own logical positions
 * when written, and q was rotated at the decoded token's logical position, so
 * attention over the spliced table equals the trainer's masked attention row
 * for that token (explainer: RoPE and block-table paragraphs).
 *
 * q        [B, Hq, D] bf16 (rotated)
 * k_pool,
 * v_pool   [num_pool_blocks, Hkv, 16, D] bf16
 * table    int32 [B, max_blocks]; entries < ceil(seq_lens[b] / 16) must be
 *          valid pool indices; an out-of-range id makes that sequence's
 *          output NaN (nothing outside the pool is read).  With
 *          max_blocks = 0 nothing is read: table and pools may be NULL and
 *          every output row is 0 (lse -inf); otherwise num_pool_blocks >= 1
 *          (KS_ERR_INVALID_ARG if not)
 * seq_lens int32 [B], 0 <= seq_lens[b] <= 16 * max_blocks; a zero-length
 *          sequence yields a zero output and lse = -inf
 * out      [B, Hq, D] bf16;  lse float [B, Hq] natural log, may be NULL
 * dtype    KS_BF16; D = 128.
 * ws       at least ks_paged_decode_workspace(B, Hq, D, max_blocks) bytes
 *          (split partials); with max_blocks = 0 the query returns the size
 *          of one split, which the call still needs.
 */
size_t ks_paged_decode_workspace(int B, int Hq, int D, int max_blocks);
ks_status ks_paged_decode(const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* table,
                          const int32_t* seq_lens, void* out, float* lse,
                          int B, int Hq, int Hkv, int D, int max_blocks,
                          int num_pool_blocks, int dtype, float scale,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * ks_append_kv -- write the newly generated token of every sequence into its
 * paged cache: the key rotated at its LOGICAL position, and the value.
 *
 * Keys are stored already rotated, so compaction can move or splice blocks
 * without touching them, and the next token continues the original position
 * count (explainer, RoPE paragraph).  The token goes to slot
 * s = seq_lens[b] - 1, i.e. block table[b][s / 16], row s % 16.
 *
 * k_new, v_new  [B, Hkv, D] bf16 (k_new unrotated; neither is modified)
 * pos           int32 [B]   logical position of the new token
 * table         int32 [B, max_blocks], seq_lens int32 [B] (already counting
 *               the new token; sequences with seq_lens[b] < 1 are skipped)
 * k_pool, v_pool [num_pool_blocks, Hkv, 16, D] bf16, written in place;
 *               a table entry outside [0, num_pool_blocks) skips that
 *               sequence (nothing outside the pool is written)
 * dtype KS_BF16, D = 128; RoPE base as in ks_rope_logical.
 */
ks_status ks_append_kv(const void* k_new, const void* v_new, const int32_t* pos,
                       const int32_t* table, const int32_t* seq_lens, void* k_pool,
                       void* v_pool, int B, int Hkv, int D, int max_blocks,
                       int num_pool_blocks, int dtype, float base, void* stream);

/*
 * ks_paged_decode_bs1 -- ks_paged_decode with single-token blocks.
 *
 * The SGLang setup stores one token per block, so turns need no padding to
 * 16 and compaction can splice any token run (explainer, paragraph on
 * padding completions to whole blocks).  The table lists one pool slot per
 * token; everything else is as for ks_paged_decode.
 *
 * q           [B, Hq, D] bf16 (rotated)
 * k_pool,
 * v_pool      [num_pool_tokens, Hkv, D] bf16 (keys rotated when written)
 * token_table int32 [B, max_tokens]; entries < seq_lens[b] must be valid
 *             slots; an out-of-range slot makes that sequence's output NaN
 *             (nothing outside the pool is read)
 * seq_lens    int32 [B], 0 <= seq_lens[b] <= max_tokens (clamped); a
 *             zero-length sequence yields a zero output and lse = -inf
 * out, lse, dtype, D, scale, workspace and errors as for ks_paged_decode.
 */
size_t ks_paged_decode_bs1_workspace(int B, int Hq, int D, int max_tokens);
ks_status ks_paged_decode_bs1(const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* token_table,
                              const int32_t* seq_lens, void* out, float* lse,
                              int B, int Hq, int Hkv, int D, int max_tokens,
                              int num_pool_tokens, int dtype, float scale,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * ks_paged_decode_rope -- paged decode with the query's RoPE fused into the
 * kernel's prologue.
 *
 * New queries continue the original position count (explainer, RoPE
 * paragraph); here the unrotated query is rotated at its logical position
 * inside the decode kernel instead of by a separate ks_rope_logical call.
 * The rotation is bit-identical to ks_rope_logical's, so the result equals
 * ks_rope_logical (on a copy of q) followed by ks_paged_decode.
 *
 * q           [B, Hq, D] bf16, UNROTATED (not modified)
 * pos         int32 [B] logical position of each sequence's query
 * block_size  16: pools [num_pool, Hkv, 16, D], table of block ids,
 *                 workspace ks_paged_decode_workspace(B, Hq, D, max_entries);
 *             1:  pools [num_pool, Hkv, D], table of token slots,
 *                 workspace ks_paged_decode_bs1_workspace(B, Hq, D, max_entries)
 * base        RoPE base (> 1)
 * other arguments, outputs and errors as for ks_paged_decode.
 */
ks_status ks_paged_decode_rope(const void* q, const int32_t* pos,
                               const void* k_pool, const void* v_pool,
                               const int32_t* table, const int32_t* seq_lens,
                               void* out, float* lse, int B, int Hq, int Hkv,
                               int D, int max_entries, int num_pool,
                               int block_size, int dtype, float scale,
                               float base, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * ks_paged_decode_noalloc -- ks_paged_decode for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  No workspace argument: the split partials live in a
 * device array owned by the library, ks_paged_decode_noalloc_max_scratch()
 * bytes (96 MiB) per GPU, kept until the process ends.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *
 * Limit   the call's split partials, ks_paged_decode_workspace(B, Hq, D,
 *         max_blocks) bytes (B * Hq * ceil(max_blocks / S) split slots of
 *         (D + 2) floats, S = 48 groups per split, or 16 when 48-group
 *         splits would make fewer than 4096 waves), must fit the array (e.g.
 *         64 sequences x 32 query heads over tables of 4,096 blocks); larger
 *         calls return KS_ERR_WORKSPACE before any launch -- use
 *         ks_paged_decode with a workspace for those.
 * Sharing Every call on one GPU uses that GPU's single array, which keeps the
 *         last call's contents (each call writes every entry it reads).
 *         Calls that overlap in time on one GPU -- on different streams or
 *         from different host threads -- RACE and may return wrong results;
 *         serialize them (one stream, or events between streams).
 * The first call on a device looks up that device's array (the device of
 * `stream`, or the current device for the null stream); a failure there
 * returns KS_ERR_HIP.  Arguments, outputs and other errors as for
 * ks_paged_decode; results are bit-identical to it.
 */
size_t ks_paged_decode_noalloc_max_scratch(void);
ks_status ks_paged_decode_noalloc(const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* table,
                                  const int32_t* seq_lens, void* out, float* lse,
                                  int B, int Hq, int Hkv, int D, int max_blocks,
                                  int num_pool_blocks, int dtype, float scale,
                                  void* stream);

/*
 * ks_append_kv_bs1 -- ks_append_kv with single-token blocks: the new token's
 * rotated key and its value go to pool slot token_table[b][seq_lens[b] - 1].
 *
 * k_pool, v_pool [num_pool_tokens, Hkv, D] bf16; token_table int32
 * [B, max_tokens]; other arguments, skips and errors as for ks_append_kv.
 */
ks_status ks_append_kv_bs1(const void* k_new, const void* v_new,
                           const int32_t* pos, const int32_t* token_table,
                           const int32_t* seq_lens, void* k_pool, void* v_pool,
                           int B, int Hkv, int D, int max_tokens,
                           int num_pool_tokens, int dtype, float base,
                           void* stream);

/*
 * Input checks (a debugging aid; nothing on the hot path depends on them).
 *
 * The kernels stay inside their buffers when the preconditions below are
 * broken: a token with e_j <= j is seen by no query, and a table entry
 * outside the pool makes that sequence's decode output NaN.  These calls
 * count the violations instead, one int32 per sequence written to `bad`
 * (device memory, [B]); a count of 0 means the input meets the
 * preconditions.  Asynchronous on `stream` like every other call.
 *
 * ks_check_eviction_record  bad[b] = #{ j < N : e[b][j] <= j } for the
 *     eviction record e int32 [B, N] of ks_evict_attn_fwd / _bwd.
 * ks_check_block_table  bad[b] = #{ x < ceil(L_b / block_size) :
 *     table[b][x] outside [0, num_pool_blocks) } + (1 if L_b < 0 or
 *     L_b > block_size * max_blocks), with L_b = seq_lens[b] (clamped to
 *     the row for the count); table int32 [B, max_blocks], block_size 16
 *     (ks_paged_decode) or 1 (ks_paged_decode_bs1).
 */
ks_status ks_check_eviction_record(const int32_t* e, int B, int N, int32_t* bad,
                                   void* stream);
ks_status ks_check_block_table(const int32_t* table, const int32_t* seq_lens,
                               int B, int max_blocks, int num_pool_blocks,
                               int block_size, int32_t* bad, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KS_H */
