/*
 * cpattn.h - C ABI of the MI355X (gfx950) context-parallel attention library.
 *
 * The library computes exact causal softmax attention over a sequence that is
 * partitioned into context-parallel (CP) chunks, the way the CP section of
 * "Scaling LLM Inference: Innovations in Tensor Parallelism, Context
 * Parallelism, and Expert Parallelism" describes it (techreport.ngo rewrite,
 * section "Context Parallelism for Million-Token Contexts"): the sequence is
 * divided among the CP ranks, every rank produces Q, K and V for its own
 * tokens, and then either its K/V (Pass-KV) or its Q (Pass-Q) moves from rank
 * to rank until each query has met the whole context.  The reader notes on
 * the same article (soumitrasaha.com, "The communication bottleneck across
 * all three axes") add that the K/V pieces circulate on a ring and the
 * per-step results are combined into the full-context output.  One GPU plays
 * every rank in turn; the ring exchange becomes a choice of chunk pointers.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are described by cpattn_tensor: a device pointer plus sizes and
 *    element strides of a [B, S, H, D] view whose last (D) axis is contiguous.
 *    Q/K/V/O use that layout; an LSE tensor uses it with D = 1 ([B, S, H]).
 *  - Scores are scaled by 1/sqrt(D).  Query head h reads KV head
 *    h / (Hq / Hkv) (grouped-query attention; Hq must be a multiple of Hkv).
 *  - Causal visibility: key row j of a K/V block whose first row sits at
 *    global position kv_offset is visible to query row i of a Q block whose
 *    first row sits at q_offset iff kv_offset + j <= q_offset + i (the
 *    diagonal is visible).
 *  - LSE is the natural log of the sum of exp(scaled score) over visible keys.
 *    A row that sees no key gets LSE = -inf and an all-zero output row.
 *  - Supported: D in {64, 128}; Q/K/V all BF16 (bf16 MFMA, fp32 accumulate)
 *    or all F32 (fp32 vector arithmetic).  Partial outputs and LSE are F32.
 *    Sequence lengths below 2^30; B and H below 2^31; K and V token strides
 *    (stride_s) of at most 2^24 elements (CPATTN_ERR_UNSUPPORTED beyond).
 *  - Alignment: Q/K/V/O data pointers 16-byte aligned and their strides
 *    (stride_b, stride_s, stride_h) multiples of 16 bytes' worth of elements
 *    (8 for BF16, 4 for F32); LSE data pointers 4-byte aligned, LSE strides
 *    unconstrained.  Workspaces 16-byte aligned.
 *  - Ownership: the caller owns every buffer and the stream.  The library
 *    allocates no device memory and keeps no pointer after a call returns;
 *    the drivers use only the caller's workspace.  Outputs must not alias
 *    inputs or each other.
 *  - Errors: all argument checks run before any HIP call.  On a non-OK
 *    status nothing has been enqueued or written and cpattn_last_error()
 *    (thread-local) describes the problem.  CPATTN_OK means the work is
 *    enqueued on `stream` (a hipStream_t; NULL is the default stream);
 *    execution errors surface at the caller's next synchronisation.
 *  - Results are deterministic: no atomics on any accumulation path, and a
 *    fixed reduction order, so repeated calls give bitwise-identical output.
 *  - Graph capture: a call enqueues kernel launches only (no allocation, copy
 *    or memset on the stream), so calls may be recorded into a HIP graph; a
 *    replay reuses the buffers and sizes of the recorded call.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPATTN_MAX_MERGE 64   /* most partials one cpattn_merge call accepts */

typedef enum cpattn_status {
  CPATTN_OK = 0,
  CPATTN_ERR_INVALID_ARG = 1,   /* null pointer, shape/stride/alignment mismatch, bad count */
  CPATTN_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels implement (e.g. D) */
  CPATTN_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the size query returned */
  CPATTN_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} cpattn_status;

typedef enum cpattn_dtype { CPATTN_BF16 = 0, CPATTN_F32 = 1 } cpattn_dtype;

/* Ring order.  CPATTN_ORDER_AUTO picks, per call, the order that moves fewer
 * bytes between ranks (cpattn_ring_select_order).  Calls take the order as an
 * int holding one of these values; any other value is CPATTN_ERR_INVALID_ARG. */
typedef enum cpattn_order { CPATTN_PASS_KV = 0, CPATTN_PASS_Q = 1, CPATTN_ORDER_AUTO = 2 } cpattn_order;

typedef struct cpattn_tensor {
  void* data;        /* device pointer (may be NULL only when the tensor is empty) */
  int32_t dtype;     /* cpattn_dtype */
  int32_t reserved;  /* must be 0 */
  int64_t B, S, H, D;                   /* sizes; D = 1 for LSE tensors */
  int64_t stride_b, stride_s, stride_h; /* element strides; the D axis has stride 1 */
} cpattn_tensor;

/*
 * cpattn_partial - attention of one local Q block against one K/V block.
 *
 * The unit of work of one ring step: a rank's local queries against the K/V
 * chunk it holds at that step (techreport.ngo rewrite, "Context Parallelism
 * for Million-Token Contexts", Pass-KV and Pass-Q bullets).
 *   q   [B, Sq, Hq, D]   BF16 or F32, rows at global positions q_offset + i
 *   k,v [B, Sk, Hkv, D]  same dtype as q, rows at kv_offset + j
 *   out [B, Sq, Hq, D]   F32: softmax(scale * q k^T, masked) v, normalised by
 *                        this block's own denominator
 *   lse [B, Sq, Hq]      F32 (D = 1): natural-log LSE of this block's scores
 * q_offset, kv_offset >= 0; causal is 0 or 1.  Rows that see no key of this
 * block (possible under the causal mask) get out = 0 and lse = -inf.
 * A BF16 call with Sq = 1, D in {64, 128} and Hq / Hkv <= 64 (a decode-shaped
 * block) runs on the split-KV decode kernel, whose query heads share each
 * K/V read; the result is the same up to rounding.
 */
cpattn_status cpattn_partial(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                             int64_t q_offset, int64_t kv_offset, int causal,
                             cpattn_tensor* out, cpattn_tensor* lse, void* stream);

/*
 * cpattn_merge - combine n partial (O, LSE) results of the same rows.
 *
 * The step that turns the pieces gathered around the ring into the
 * full-context result (soumitrasaha.com reader notes, "The communication
 * bottleneck across all three axes"), done by the exact log-sum-exp rule:
 *   M = max_c lse_c,  w_c = exp(lse_c - M),
 *   out = sum_c w_c O_c / sum_c w_c,  out_lse = M + ln(sum_c w_c);
 * rows whose partials all have lse = -inf give out = 0, out_lse = -inf.
 *   partials[c] [B, S, H, D] F32, c = 0..n-1, all with the same sizes and
 *               strides (host array of n descriptors)
 *   lses[c]     [B, S, H] F32, all with the same strides
 *   out         [B, S, H, D] F32 or BF16 (rounded to nearest even)
 *   out_lse     [B, S, H] F32, or NULL to skip
 * 1 <= n <= CPATTN_MAX_MERGE.  Sums run in the array order, so the result is
 * bitwise reproducible for a given order (any order is correct up to
 * rounding).
 */
cpattn_status cpattn_merge(const cpattn_tensor* partials, const cpattn_tensor* lses, int n,
                           cpattn_tensor* out, cpattn_tensor* out_lse, void* stream);

/*
 * Ring layout shared by the ring calls below.
 *
 * q [B, Sq, Hq, D] and k, v [B, Skv, Hkv, D] with Sq <= Skv: the queries are
 * the last Sq positions of the sequence whose keys and values k and v hold
 * (Sq = Skv is a full prefill; Sq < Skv is new tokens against a cached
 * context).  Both are cut into n_chunks = P equal contiguous chunks, one per
 * simulated CP rank (techreport.ngo rewrite, "Context Parallelism for
 * Million-Token Contexts": the sequence is divided among the ranks): Q chunk
 * i holds Cq = Sq / P queries at positions Skv - Sq + i Cq + [0, Cq), K/V
 * chunk j holds Ckv = Skv / P keys at positions j Ckv + [0, Ckv).  Ring step
 * s gives rank r the pair (Q chunk r, K/V chunk (r - s) mod P) under
 * CPATTN_PASS_KV, or (Q chunk (r - s) mod P, K/V chunk r) under
 * CPATTN_PASS_Q (the same section: the two variants differ only in whether
 * K/V or Q moves between ranks).  Under the causal mask a pair whose first key
 * lies after its last query sees nothing and is skipped.  Each Q chunk's
 * partials are merged in the order they reached its owner (Pass-KV: own
 * chunk, then (i - s) mod P for s = 1, 2, ...; Pass-Q: own chunk, then
 * (i + s) mod P), skipping the pairs that were skipped.
 * 1 <= n_chunks <= CPATTN_MAX_MERGE must divide Sq and Skv.
 */

/*
 * cpattn_ring_prefill_workspace_size - bytes of workspace cpattn_ring_prefill,
 * cpattn_ring_step and cpattn_ring_merge need for this q, K/V length, chunk
 * count and mask: one fp32 O and LSE slot per visible (Q chunk, K/V chunk)
 * pair.  k may be NULL for K/V as long as q.  Returns 0 if the arguments are
 * invalid (cpattn_last_error() then says why).
 */
size_t cpattn_ring_prefill_workspace_size(const cpattn_tensor* q, const cpattn_tensor* k, int n_chunks, int causal);

/*
 * cpattn_ring_select_order - the ring order that moves fewer bytes between
 * ranks for this shape, and the bytes of each.
 *
 * The pages present Pass-KV and Pass-Q side by side without a rule
 * ("Context Parallelism for Million-Token Contexts").  The rule here counts
 * what a P-rank ring would move: every chunk makes P - 1 hops (K and V of a
 * chunk under Pass-KV, 2 Ckv Hkv D elements per hop and batch row; a Q chunk
 * under Pass-Q, Cq Hq D elements), and under Pass-Q every visible pair
 * computed away from its Q chunk's owner also returns its partial, fp32 O
 * and LSE (Cq Hq (D + 1) floats).  Elements are q's dtype.  Pass-KV wins
 * ties.  On return *order is CPATTN_PASS_KV or CPATTN_PASS_Q; the byte counts
 * are written where the pointers are not NULL.  No device call is made.
 */
cpattn_status cpattn_ring_select_order(const cpattn_tensor* q, const cpattn_tensor* k, int n_chunks, int causal,
                                       int* order, uint64_t* bytes_pass_kv, uint64_t* bytes_pass_q);

/*
 * cpattn_ring_prefill - attention of every query over the whole sequence by a
 * simulated CP ring (layout above).
 *
 * All ranks' partials of every step go out together (on one device the pairs
 * are independent), each into its workspace slot; then every Q chunk's
 * partials are merged in arrival order.  The result equals, bit for bit,
 * cpattn_ring_step for every step followed by cpattn_ring_merge (with BF16
 * K/V chunks of a multiple of 64 tokens, at most 16384, and at least two
 * owner query tiles per compute unit, a query tile walks its visible chunks
 * and merges its own partials as soon as it has written them, with the same
 * arithmetic).
 *   q [B, Sq, Hq, D], k/v [B, Skv, Hkv, D]  BF16 or F32
 *   order              CPATTN_PASS_KV, CPATTN_PASS_Q or CPATTN_ORDER_AUTO
 *   out [B, Sq, Hq, D] F32 or BF16
 *   lse [B, Sq, Hq]    F32, or NULL
 *   workspace          device buffer of at least
 *                      cpattn_ring_prefill_workspace_size(q, k, n_chunks, causal) bytes;
 *                      scratch of this call (its contents afterwards are unspecified:
 *                      the walk keeps a query tile's own-chunk partial in registers
 *                      when it is the last one the tile computes)
 */
cpattn_status cpattn_ring_prefill(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                  int n_chunks, int order /* cpattn_order */, int causal,
                                  cpattn_tensor* out, cpattn_tensor* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * cpattn_ring_step - the partial-attention work of one ring step for every
 * simulated rank: the pairs that step s assigns are computed in one launch
 * into their workspace slots.  Running steps 0 .. n_chunks-1 and then
 * cpattn_ring_merge on the same workspace is exactly cpattn_ring_prefill; on
 * a real CP ring this is what a rank does between two K/V (or Q) exchanges
 * ("Context Parallelism for Million-Token Contexts").  Arguments as in
 * cpattn_ring_prefill; 0 <= step < n_chunks.  A step with no visible pair
 * enqueues nothing.
 */
cpattn_status cpattn_ring_step(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                               int n_chunks, int order /* cpattn_order */, int causal, int step,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * cpattn_ring_step_accumulate - one ring step whose partials are merged into
 * the running result as they arrive, with no workspace and no separate merge:
 * the kernel that computes a pair's partial (O, LSE) combines it with the
 * owner's rows already in out/lse by the exact LSE merge (soumitrasaha.com
 * reader notes, "The communication bottleneck across all three axes": the
 * pieces passed around the ring are accumulated into the full result).
 * Step 0 gives every owner its first pair (its own chunk) and writes those
 * rows; each later step merges the pair it assigns into them.  Running steps
 * 0 .. n_chunks-1 in order on one stream leaves the full attention in out and
 * lse, merged in arrival order; rows of an owner with no pair at a step are
 * not touched.
 *   q, k, v, n_chunks, order, causal, step  as in cpattn_ring_step
 *   out [B, Sq, Hq, D]  F32 (read and written from step 1 on)
 *   lse [B, Sq, Hq]     F32, required (the running LSE)
 * Steps after 0 read out/lse as left by the earlier steps of the same ring:
 * calls for one ring must not overlap, and nothing else may write out/lse in
 * between.
 */
cpattn_status cpattn_ring_step_accumulate(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                          int n_chunks, int order /* cpattn_order */, int causal, int step,
                                          cpattn_tensor* out, cpattn_tensor* lse, void* stream);

/*
 * cpattn_ring_merge - merge every Q chunk's partials from a workspace filled
 * by cpattn_ring_step (all steps), in the order they reached the chunk's
 * owner, into out [B, Sq, Hq, D] (F32 or BF16) and lse [B, Sq, Hq] (F32, or
 * NULL).  The query shapes come from out; kv_len is the K/V length Skv the
 * steps ran with.  n_chunks, causal and the order must match the steps that
 * filled the workspace; the order must be CPATTN_PASS_KV or CPATTN_PASS_Q
 * (for steps run with CPATTN_ORDER_AUTO, the order
 * cpattn_ring_select_order returns).
 */
cpattn_status cpattn_ring_merge(int n_chunks, int order /* cpattn_order */, int causal, int64_t kv_len,
                                const void* workspace, size_t workspace_bytes,
                                cpattn_tensor* out, cpattn_tensor* lse, void* stream);

/*
 * cpattn_ring_prefill_fused - the ring prefill with the merge done online.
 *
 * Every Q chunk's partials are accumulated into one running (O, LSE) as the
 * K/V chunks reach it, instead of being stored and merged afterwards (the
 * pieces gathered around the ring accumulated into the full result: "The
 * communication bottleneck across all three axes", soumitrasaha.com reader
 * notes).  On one device the owner of Q chunk i sees the keys up to its last
 * query (all of them without the causal mask) in one pass, in position order;
 * any order of the same keys is exact up to rounding, so the result equals
 * cpattn_ring_prefill's within rounding.  No workspace, one launch.
 *   q, k, v  as for cpattn_ring_prefill (Sq <= Skv)
 *   out      [B, Sq, Hq, D] F32
 *   lse      [B, Sq, Hq] F32, or NULL to skip
 * Errors as for cpattn_ring_prefill (out must be F32).
 */
cpattn_status cpattn_ring_prefill_fused(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                        int n_chunks, int causal, cpattn_tensor* out, cpattn_tensor* lse,
                                        void* stream);

/*
 * cpattn_splitkv_decode_workspace_size - bytes of workspace
 * cpattn_splitkv_decode needs (0 if the arguments are invalid).
 */
size_t cpattn_splitkv_decode_workspace_size(const cpattn_tensor* q, const cpattn_tensor* k, int n_chunks);

/*
 * cpattn_splitkv_decode - one new token per sequence against a cached K/V
 * that is split into n_chunks equal chunks.
 *
 * Decode reads the KV cache and is memory-bandwidth bound (techreport.ngo
 * rewrite, "Why Parallelism Defines LLM Serving Cost"; reader notes, "The
 * communication bottleneck across all three axes"); the cache grows
 * linearly with context ("Context Parallelism for Million-Token Contexts").
 * Each chunk (further cut into sub-splits chosen by the library) yields a
 * partial (O, LSE) that is merged into the result.  The new token sits at
 * position Skv - 1 and sees every cached key.
 *   q   [B, 1, Hq, D]    BF16
 *   k,v [B, Skv, Hkv, D] BF16
 *   out [B, 1, Hq, D]    F32 or BF16
 *   lse [B, 1, Hq]       F32, or NULL
 * n_chunks >= 1 must divide Skv; Hq / Hkv <= 64.
 */
cpattn_status cpattn_splitkv_decode(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                    int n_chunks, cpattn_tensor* out, cpattn_tensor* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * cpattn_splitkv_decode_noalloc - cpattn_splitkv_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Same arguments, result and kernels as cpattn_splitkv_decode, but the
 * partials live in a fixed scratch array inside the library (64 MiB per GPU,
 * held until the process ends) instead of a caller's workspace; the call
 * allocates and frees nothing.  A decode whose partials need more than the
 * scratch holds (cpattn_splitkv_decode_workspace_size() > 64 MiB) returns
 * CPATTN_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller.  Nothing in the
 * scratch needs to start at zero: every partial the merge reads is written
 * by the same call first.
 */
cpattn_status cpattn_splitkv_decode_noalloc(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                            int n_chunks, cpattn_tensor* out, cpattn_tensor* lse, void* stream);

/*
 * cpattn_kv_cache_write - the prefill's K/V, chunk by chunk, into the KV-cache
 * shards of the CP ranks.
 *
 * The prefill constructs the KV cache of every transformer layer and decode
 * then reads and extends it (techreport.ngo rewrite, "Why Parallelism Defines
 * LLM Serving Cost"); with the sequence divided among CP ranks ("Context
 * Parallelism for Million-Token Contexts"), rank r keeps its own chunk's keys
 * and values.  Rows [0, C) of shard r receive rows [r C, (r+1) C) of k and v
 * (C = S / n_chunks); the other shard rows are not touched.
 *   k, v                 [B, S, Hkv, D] BF16 or F32
 *   k_shards, v_shards   host arrays of n_chunks descriptors [B, cap, Hkv, D]
 *                        (same dtype, shape and strides; only the pointers
 *                        differ), cap >= C
 * 1 <= n_chunks <= CPATTN_MAX_MERGE must divide S.  A byte copy.
 */
cpattn_status cpattn_kv_cache_write(const cpattn_tensor* k, const cpattn_tensor* v, int n_chunks,
                                    const cpattn_tensor* k_shards, const cpattn_tensor* v_shards, void* stream);

/*
 * cpattn_kv_cache_append - new tokens' keys and values into rows
 * [row, row + T) of one shard (the cache growing by decode, same sections).
 *   k_new, v_new       [B, T, Hkv, D]
 *   k_shard, v_shard   [B, cap, Hkv, D], same dtype; 0 <= row, row + T <= cap
 * A byte copy.
 */
cpattn_status cpattn_kv_cache_append(const cpattn_tensor* k_new, const cpattn_tensor* v_new,
                                     const cpattn_tensor* k_shard, const cpattn_tensor* v_shard, int64_t row,
                                     void* stream);

/*
 * cpattn_cp_decode_workspace_size - bytes of workspace cpattn_cp_decode needs
 * for this q and these shards (sized by the shards' capacity, so it does not
 * change as they fill); 0 if the arguments are invalid.
 */
size_t cpattn_cp_decode_workspace_size(const cpattn_tensor* q, const cpattn_tensor* k_shards, int n_shards);

/*
 * cpattn_cp_decode - one new token per sequence against a KV cache sharded
 * across CP ranks.
 *
 * Decode reads the KV cache and is memory-bandwidth bound ("Why Parallelism
 * Defines LLM Serving Cost"); with the cache divided among the ranks, each
 * rank attends the new query against its own shard and the per-rank partials
 * are merged by the exact LSE rule.  The new token comes after every cached
 * key, so it sees all of them.  Shard r contributes its rows
 * [0, shard_len[r]); shards are merged in index order.
 *   q                    [B, 1, Hq, D] BF16
 *   k_shards, v_shards   host arrays of n_shards descriptors [B, cap, Hkv, D]
 *                        BF16 (same shape and strides), Hq / Hkv <= 64
 *   shard_len            host array of n_shards lengths, 0 <= len <= cap
 *   out [B, 1, Hq, D]    F32 or BF16;  lse [B, 1, Hq] F32, or NULL
 *   workspace            >= cpattn_cp_decode_workspace_size(q, k_shards, n_shards)
 * 1 <= n_shards <= CPATTN_MAX_MERGE.  A row whose shards are all empty gets
 * out = 0 and lse = -inf.
 */
cpattn_status cpattn_cp_decode(const cpattn_tensor* q, const cpattn_tensor* k_shards, const cpattn_tensor* v_shards,
                               const int64_t* shard_len, int n_shards, cpattn_tensor* out, cpattn_tensor* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* cpattn_last_error(void);

/* Library version string, e.g. "cpattn 0.2.0 gfx950". */
const char* cpattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
