/*
 * maskattn.h -- C ABI of the masked attention backward library for AMD MI355X (gfx950).
 *
 * Two masked forms of the FlashAttention-style attention backward pass:
 *
 *  (A) GQA attention with a learnable per-head sink logit and a sliding-window causal
 *      mask, BHSD layout.  Defined on the page "[Example] Add GQA Sink Backward BHSD with
 *      robustness improvements" (tilelang-ascend PR 1): "Files Added" (forward with
 *      online softmax + sink + sliding window; backward producing dSinks) and the commit
 *      message of the 4->2 kernel revision (Phase0 Delta = sum(O*dO), a KV loop of five
 *      GEMMs with softmax and dS, Phase5 dSink; outputs O, Delta, dQ, dK, dV, dSinks).
 *
 *  (B) Block-sparse MHA driven by a uint8 block mask [B, N, ceil(Sq/bx), ceil(Skv/by)],
 *      BNSD layout, D = 128.  Defined on the page "knowledge(triton) ... #174"
 *      (cannbot-knowledge PR 174), BlockSparseAttentionGrad runbook: "task features"
 *      (inputs dO, O and the softmax statistics; outputs dQ, dK, dV), "optimisation 1"
 *      (the host only checks shapes, allocates and views; the mask transpose and the
 *      selection tables are built on the device; no token-level dense mask), and the
 *      precision recipe (p = exp(s - lse), ds = p * (dp - delta), a row with no selected
 *      block gets zero).
 *
 * Mathematical contract (fp64 statement; the library computes it with fp16/bf16 MFMA
 * operands and fp32 accumulation):
 *   s_ij   = scale * q_i . k_j                    (scale multiplies q.k; natural log domain)
 *   vis    (A) 0 <= i - j < window;  window >= S is plain causal
 *          (B) block_mask[b, n, i / bx, j / by] != 0
 *   lse_i  = log(exp(sink_h) + sum_{j vis} exp(s_ij))          (A; the sink is not scaled)
 *          = log(sum_{j vis} exp(s_ij)), -inf for an empty row (B)
 *   P_ij   = vis ? exp(s_ij - lse_i) : 0,   O_i = sum_j P_ij v_j
 *   D_i    = dO_i . O_i
 *   dS_ij  = P_ij (dO_i . v_j - D_i)
 *   dQ_i   = scale sum_j dS_ij k_j
 *   dK_j   = scale sum_{h in group(kvh)} sum_i dS_ij q_i
 *   dV_j   = sum_{h in group(kvh)} sum_i P_ij dO_i
 *   dsink_h = - sum_b sum_i exp(sink_h - lse_i) D_i            (A only)
 * GQA groups are contiguous: query head h uses key/value head h / (Hq / Hkv).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer.  Tensors are dense, row-major, in the
 *     layouts given per argument, 16-byte aligned.  Outputs must not alias inputs.
 *   - dtype selects the element type of q, k, v, o, dout, dq, dk, dv: MA_F16 (IEEE
 *     half) or MA_BF16 (bfloat16).  lse, sink, dsink and the workspace are fp32.
 *   - stream is a hipStream_t (NULL = the null stream).  Every call only enqueues work
 *     on that stream and returns; there is no host synchronisation inside.
 *   - The caller owns every buffer.  The library allocates no memory and keeps no state
 *     between calls; concurrent calls on different streams with different buffers are safe.
 *   - Validation reads only the scalar arguments and pointer values (never device data).
 *     On any error nothing is enqueued and the status says why.
 *   - Every element of every output is written, including exact zeros for rows that no
 *     visible pair touches.
 *   - Supported: D = 128 only; S >= 1 (any length, ragged tails allowed); window >= 1;
 *     bx, by multiples of 16 in [16, 128].
 */
#ifndef MASKATTN_H
#define MASKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MA_OK = 0,            /* enqueued */
  MA_EINVAL = 1,        /* null/misaligned pointer, non-positive size, Hq % Hkv != 0, window < 1, ... */
  MA_EUNSUPPORTED = 2,  /* D != 128, bx/by not a multiple of 16 or > 128, unknown dtype */
  MA_EWORKSPACE = 3,    /* workspace smaller than the matching *_workspace_bytes() query */
  MA_ELAUNCH = 4,       /* the HIP runtime reported an error while enqueueing */
  MA_ESCRATCH = 5       /* attn_sink_bwd_noalloc: the problem needs more than its static scratch */
};

/* Element types of the activation tensors. */
enum { MA_F16 = 0, MA_BF16 = 1 };

/* Human-readable text for a status code (static storage, never NULL). */
const char* maskattn_strerror(int status);

/* ---------------------------------------------------------------------------------
 * (A) attn_sink_fwd: forward pass with sink and sliding window (support call; it
 * produces the O and lse the backward consumes).  Page 1, "Files Added" (online
 * softmax with attention sink + sliding window mask) and the 4->2 revision (forward
 * -> O, lse).
 *   q     [B, Hq,  S, D]  dtype          k, v [B, Hkv, S, D] dtype
 *   sink  [Hq]            fp32 logits (may be -inf: no sink)
 *   o     [B, Hq,  S, D]  dtype  (out)   lse  [B, Hq, S]      fp32, natural log (out)
 *   Hq % Hkv == 0, D == 128, window >= 1, scale > 0 (finite).
 * --------------------------------------------------------------------------------- */
int attn_sink_fwd(const void* q, const void* k, const void* v, const float* sink,
                  void* o, float* lse,
                  int B, int Hq, int Hkv, int S, int D, int window, float scale,
                  int dtype, void* stream);

/* Workspace bytes attn_sink_bwd needs (0 on invalid sizes).  Layout (offsets in bytes),
 * with Sp = 64*ceil(S/64) and R = align256(4*B*Hq*Sp):
 *   0:   Delta [B, Hq, Sp] fp32  (Delta_i = dO_i . O_i; readable after the call; rows >= S
 *        hold 0)
 *   R:   lse * log2(e) [B, Hq, Sp] fp32 (rows >= S and rows with lse = -inf hold +inf)
 *   2R:  dsink partials [B, Hq, ceil(S/64)] fp32 */
size_t attn_sink_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D);

/* Workspace bytes that select attn_sink_bwd's dS-bank path (0 on invalid sizes or window <
 * 1): attn_sink_bwd_workspace_bytes() followed, at that offset, by the dS bank, 2048 bytes
 * for every 32 x 32 (query block, key block) pair holding a visible (i, j) of each (batch,
 * query head): B * Hq * sum_a (min(a, kb) + 1) blocks, a over ceil(S/32) query blocks, kb =
 * ceil((min(window, S) - 1) / 32).  For window = S that is the lower triangle: 4.3 GB at
 * B = 1, Hq = 64, S = 8192.
 * When the key tiles give too few dK/dV workgroups to fill the GPU (W = min(window, S): W >=
 * 256, key tiles of 128 rows, B * Hkv * ceil(ceil(S/128) / 2) < 256 tile pairs; W < 256, key
 * tiles of 64 rows, B * Hkv * ceil(S/64) < 512), the bank is followed (at the next 256-byte
 * boundary) by the fp32 partial dK and dV of a head split of the dK/dV work, 2 * B * Hkv * M *
 * Sp * D * 4 bytes.  Key tile p's visits (its query heads times the 64-row query tiles of rows
 * [bc p, min(S, bc p + bc - 1 + W)), bc the key tile rows) go to min(group, ceil(visits /
 * target)) workgroups of whole query heads, target = max(1, ceil(all tiles' visits * B * Hkv /
 * 1024)), M the largest such count (none when M = 1); the partial sums are added in chunk
 * order (deterministic).  268 MB at B = 1, Hq = 64, Hkv = 8, S = window = 4096 (M = 8; the key
 * tiles near the start see up to twice the average work).  Dense calls only: the
 * packed-sequence entry points do not split. */
size_t attn_sink_bwd_ds_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int window);

/* ---------------------------------------------------------------------------------
 * (A) attn_sink_bwd: backward pass with sink and sliding window.
 *   q, o, dout [B, Hq, S, D] dtype;  k, v [B, Hkv, S, D] dtype
 *   lse [B, Hq, S] fp32 (as produced by the forward: includes the sink)
 *   sink [Hq] fp32
 *   dq [B, Hq, S, D], dk/dv [B, Hkv, S, D] dtype (out); dsink [Hq] fp32 (out)
 *   workspace: device buffer of >= attn_sink_bwd_workspace_bytes() bytes, 256-aligned.
 *   With >= attn_sink_bwd_ds_workspace_bytes() bytes the dK/dV kernel also stores dS (in
 *   the element type) and dQ is one GEMM per stored block; with less, the dQ kernel
 *   recomputes S and dP.  The two paths round dS at different points, so their dQ may
 *   differ in the last bits; both meet the same tolerance.
 * Results are deterministic: no atomics; every reduction has a fixed order.
 * --------------------------------------------------------------------------------- */
int attn_sink_bwd(const void* q, const void* k, const void* v,
                  const void* o, const void* dout, const float* lse, const float* sink,
                  void* dq, void* dk, void* dv, float* dsink,
                  void* workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int S, int D, int window, float scale,
                  int dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * attn_sink_bwd_noalloc: attn_sink_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as attn_sink_bwd given exactly
 * attn_sink_bwd_workspace_bytes() of workspace (the path where dQ recomputes S and dP),
 * without the workspace argument: its scratch (Delta, lse * log2 e, dsink partials; the
 * attn_sink_bwd workspace layout) lives in
 * a static device array of MA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * from the first call on that GPU until the process ends; its device address is looked up
 * once per device.  The call allocates nothing and enqueues no memset (every scratch byte
 * it reads is written earlier in the same call).
 *   - MA_ESCRATCH when attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D) exceeds
 *     MA_NOALLOC_SCRATCH_BYTES (nothing is enqueued).
 *   - Every call on one GPU shares that GPU's array and leaves its contents behind: calls
 *     that overlap on one GPU (concurrent streams, or host threads) race and must be
 *     serialised by the caller.
 * --------------------------------------------------------------------------------- */
#define MA_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_sink_bwd_noalloc(const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse, const float* sink,
                          void* dq, void* dk, void* dv, float* dsink,
                          int B, int Hq, int Hkv, int S, int D, int window, float scale,
                          int dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * (B) blocksparse_build_tables: device-side mask transpose and selection tables.
 * Page 2, "optimisation 1" and "optimisation 2" (transpose bit-equal to
 * mask.permute(0,1,3,2); compaction by exclusive prefix count, so entries ascend).
 *   block_mask [B, N, nqb, nkb] uint8 (nonzero = keep)
 *   mask_t     [B, N, nkb, nqb] uint8 (out)
 *   sel_q      [B, N, nqb, nkb] int32 (out): row i lists the kept key blocks, ascending,
 *                                            then -1;  cnt_q [B, N, nqb] int32 (out)
 *   sel_k      [B, N, nkb, nqb] int32 (out): row j lists the kept query blocks,
 *                                            ascending, then -1;  cnt_k [B, N, nkb] (out)
 * The outputs are bit-exact functions of the mask.
 * --------------------------------------------------------------------------------- */
int blocksparse_build_tables(const uint8_t* block_mask, int B, int N, int nqb, int nkb,
                             uint8_t* mask_t, int32_t* sel_q, int32_t* cnt_q,
                             int32_t* sel_k, int32_t* cnt_k, void* stream);

/* (B) blocksparse_attn_fwd: block-sparse forward (support call producing O and lse;
 * empty rows get O = 0 and lse = -inf).  Layouts as blocksparse_attn_bwd; the workspace
 * (same size query and layout as the backward) receives the mask tables it iterates. */
int blocksparse_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                         void* o, float* lse, void* workspace, size_t workspace_bytes,
                         int B, int N, int Sq, int Skv, int D, int bx, int by, float scale,
                         int dtype, void* stream);

/* Workspace bytes blocksparse_attn_bwd needs (0 on invalid sizes).  Layout, each
 * region starting at a 256-byte boundary, in this order:
 *   Delta [B, N, Sqp] fp32, lse * log2(e) [B, N, Sqp] fp32 (Sqp = 64*ceil(Sq/64); +inf for
 *   padding rows and rows with lse = -inf),
 *   mask_t [B, N, nkb, nqb] u8,
 *   sel_q [B, N, nqb, nkb] i32, cnt_q [B, N, nqb] i32, sel_k [B, N, nkb, nqb] i32,
 *   cnt_k [B, N, nkb] i32,
 *   when N * nqb > 64: fp32 partial dK and dV of key blocks selected by more than 32 query
 *   blocks (summed over a GQA group's query heads), which the backward splits over several
 *   workgroups and adds back in a fixed order: 2 x B x floor(N * (nqb + 31) / 32) slots of
 *   [Skvp, D] (Skvp = 64*ceil(Skv/64)), a bound that holds for every Hkv dividing N.  A call
 *   whose group * nqb is at most 64 splits nothing (one workgroup walks each key block).
 * The block-sparse forward calls take the same workspace. */
size_t blocksparse_attn_bwd_workspace_bytes(int B, int N, int Sq, int Skv, int D, int bx, int by);

/* Workspace that also holds the block path's dS bank: blocksparse_attn_bwd_workspace_bytes()
 * plus 2048 bytes per entry of a grid of 32 x 32 blocks of every (batch, query head): 32-row
 * query blocks (rows 32 i ..) by nka key sub-blocks, where nka = ceil(Skv/32) when by is a
 * multiple of 32 (the dense 32-row key grid) and ceil(Skv/by) * ceil(by/32) otherwise (the
 * sub-blocks of 32 rows starting at each mask block's first key row, the last one of a block
 * partly past it):  B * N * ceil(Sq/32) * nka * 2048 bytes at the end of the workspace
 * (256-byte aligned), provided a head's grid has fewer than 2^30 entries; otherwise equal to
 * blocksparse_attn_bwd_workspace_bytes().  Passing at least this many bytes to
 * blocksparse_attn_bwd(_gqa) makes the dK/dV kernel store the 16-bit dS of every 32 x 32 block
 * holding a selected (query, key) pair and the dQ kernel read it back, one GEMM per block,
 * instead of recomputing S and dP: the second pass of the five-GEMM scheme that the
 * block-sparse page's handbook lists among its next optimisations (a single pass computing the
 * five products, partial sums in a workspace, then a reduce), with dS rather than fp32 dQ
 * partials as the intermediate.  Rows and key columns of an entry outside the selected mask
 * blocks hold exact zeros.  Results are deterministic either way (fixed key order).  Only
 * entries touching selected mask blocks are written or read. */
size_t blocksparse_attn_bwd_ds_workspace_bytes(int B, int N, int Sq, int Skv, int D, int bx, int by);

/* ---------------------------------------------------------------------------------
 * (B) blocksparse_attn_bwd: block-sparse MHA backward.
 *   q, o, dout [B, N, Sq, D] dtype;  k, v [B, N, Skv, D] dtype;  lse [B, N, Sq] fp32
 *   block_mask [B, N, ceil(Sq/bx), ceil(Skv/by)] uint8
 *   dq [B, N, Sq, D], dk/dv [B, N, Skv, D] dtype (out)
 * Builds the tables (as blocksparse_build_tables) into the workspace, then Delta, dK/dV
 * (iterating each key block's kept query blocks) and dQ (iterating each query block's
 * kept key blocks).  Deterministic.
 * --------------------------------------------------------------------------------- */
int blocksparse_attn_bwd(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         const uint8_t* block_mask,
                         void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         int B, int N, int Sq, int Skv, int D, int bx, int by, float scale,
                         int dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * (B') Block-sparse attention with grouped K/V heads (GQA).  The block-sparse page is MHA;
 * these apply the sink page's grouping (contiguous groups: query head h reads K/V head
 * h / (Hq / Hkv)) to it, with the block mask per query head:
 *   q, o, dout [B, Hq, Sq, D];  k, v [B, Hkv, Skv, D];  lse [B, Hq, Sq] fp32
 *   block_mask [B, Hq, ceil(Sq/bx), ceil(Skv/by)] uint8
 *   dq [B, Hq, Sq, D], dk/dv [B, Hkv, Skv, D] (out; dK/dV summed over the group)
 * Workspace: blocksparse_attn_bwd_workspace_bytes(B, Hq, Sq, Skv, D, bx, by), same layout.
 * Errors as blocksparse_attn_fwd / blocksparse_attn_bwd, plus MA_EINVAL when Hkv < 1 or
 * Hq % Hkv != 0.  With Hkv = Hq they are blocksparse_attn_fwd / blocksparse_attn_bwd.
 * --------------------------------------------------------------------------------- */
int blocksparse_attn_fwd_gqa(const void* q, const void* k, const void* v, const uint8_t* block_mask,
                             void* o, float* lse, void* workspace, size_t workspace_bytes,
                             int B, int Hq, int Hkv, int Sq, int Skv, int D, int bx, int by, float scale,
                             int dtype, void* stream);
int blocksparse_attn_bwd_gqa(const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             const uint8_t* block_mask,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             int B, int Hq, int Hkv, int Sq, int Skv, int D, int bx, int by, float scale,
                             int dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * (A') Sink attention over packed variable-length sequences.  Page 1's kernel table lists a
 * "GQA Sink Backward VarLen" (and forward) workload: a batch of sequences of different
 * lengths, each attending only to itself, with the same sink and sliding-window mask as
 * attn_sink_fwd / attn_sink_bwd.  The pages give no layout; these calls take sequences packed
 * along the row axis of every head:
 *   q, o, dout, dq [Hq, total, D] dtype;  k, v, dk, dv [Hkv, total, D] dtype
 *   lse [Hq, total] fp32 (natural log, includes the sink)
 *   cu_seqlens [B + 1] int32, DEVICE memory: sequence b is rows cu_seqlens[b] ..
 *     cu_seqlens[b + 1] - 1 of every head; contract: cu_seqlens[0] = 0, non-decreasing,
 *     cu_seqlens[B] = total, every length <= max_seqlen (empty sequences allowed).
 *   window counts within a sequence (window >= max_seqlen: causal within each sequence).
 *   dsink [Hq] fp32 (out): summed over all sequences.
 * Workspace: attn_sink_bwd_workspace_bytes(B, Hq, Hkv, max_seqlen, D), same layout with S =
 * max_seqlen, per (sequence, head) (Delta row i of sequence b, head h at [b, h, i]);
 * attn_sink_bwd_ds_workspace_bytes(B, Hq, Hkv, max_seqlen, D, window) selects the dS-bank
 * path as for attn_sink_bwd (bank entries per (sequence, head) sized for max_seqlen).
 * The offsets are device data and are not validated; the kernels clamp them to [0, total]
 * and each length to max_seqlen, so a table that breaks the contract gives unspecified
 * values but never an access outside the tensors.  Rows outside every sequence are not
 * written.  Errors as attn_sink_fwd / attn_sink_bwd, plus MA_EINVAL for a null or
 * misaligned cu_seqlens, total < 1, max_seqlen < 1 or max_seqlen > total.  With B equal
 * lengths S and a tensor relaid [B, H, S, D] -> [H, B*S, D] the results are attn_sink_fwd's
 * and attn_sink_bwd's, bit for bit wherever attn_sink_bwd does not split its key tiles by
 * query heads (Hq = Hkv, or its minimum workspace); a split dense call sums dK and dV in
 * another order (the packed entry points never split).
 * --------------------------------------------------------------------------------- */
int attn_sink_fwd_varlen(const void* q, const void* k, const void* v, const float* sink,
                         const int* cu_seqlens, void* o, float* lse,
                         int B, int total, int max_seqlen, int Hq, int Hkv, int D, int window,
                         float scale, int dtype, void* stream);
int attn_sink_bwd_varlen(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse, const float* sink,
                         const int* cu_seqlens,
                         void* dq, void* dk, void* dv, float* dsink,
                         void* workspace, size_t workspace_bytes,
                         int B, int total, int max_seqlen, int Hq, int Hkv, int D, int window,
                         float scale, int dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * Profiling variants: identical work and results to attn_sink_bwd / blocksparse_attn_bwd,
 * and additionally record caller-created HIP events (hipEvent_t, passed as void*) on
 * `stream` between the stages, so per-stage device time can be read with
 * hipEventElapsedTime without a profiler:
 *   events[0] before the first kernel            events[1] after preprocess (+ tables)
 *   events[2] after the dK/dV kernel (and the dsink reduce its first workgroup does, or the
 *             block path's chunk reduce)         events[3] after the dQ kernel
 * events must point to 4 valid events (MA_EINVAL if events is NULL).
 * --------------------------------------------------------------------------------- */
int attn_sink_bwd_timed(const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse, const float* sink,
                        void* dq, void* dk, void* dv, float* dsink,
                        void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int S, int D, int window, float scale,
                        int dtype, void* stream, void* const* events);

int blocksparse_attn_bwd_timed(const void* q, const void* k, const void* v,
                               const void* o, const void* dout, const float* lse,
                               const uint8_t* block_mask,
                               void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes,
                               int B, int N, int Sq, int Skv, int D, int bx, int by, float scale,
                               int dtype, void* stream, void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* MASKATTN_H */
