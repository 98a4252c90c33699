/*
 * fe.h -- C ABI of libfe.so: paged grouped-query attention over a
 * block-allocated KV cache, hand-written HIP for MI355X (gfx950).
 *
 * The operations are the per-layer attention step of the prefill-then-decode
 * loop that "Make the Engine Talk" (inference-engine book, chapter 1) walks
 * through in sections 1.2 and 1.3: one pass over the prompt primes the cache,
 * then one pass per generated token, and grouped-query attention is one of
 * the forward pass's mechanisms.  The ForgeEngine README
 * (github.com/marcoharuni/forge-engine), table "What it implements", gives
 * the cache as a paged block allocator and the kernels as a CUDA paged GQA
 * kernel plus a restricted prefill lab; its architecture flowchart has the
 * prefill/decode step both write to and read from the paged cache.
 *
 * Shapes and layout (the pages fix none of them; these are this library's):
 *   D  = head_dim            -- must be 128
 *   BS = KV block size       -- must be 16 tokens
 *   Hq query heads, Hkv KV heads, Hq % Hkv == 0, G = Hq / Hkv in 1..8;
 *   query head h reads KV head h / G (contiguous groups).
 *   K and V pools: bf16 [num_blocks][Hkv][BS][D] each, so every
 *     (block, KV head) tile is one contiguous 4 KiB run.
 *   slot = block * BS + offset_in_block (int32).
 *   block_tables: int32 [B][max_blocks_per_seq], row b lists sequence b's
 *     blocks in token order; token t of sequence b lives in block
 *     block_tables[b][t / BS] at offset t % BS.
 *   context_lens[b] (int32) counts every token sequence b attends over,
 *     including the ones appended this step.
 *   Attention is softmax(scale * q . k_t) v over tokens t < L, accumulated in
 *   fp32; out is rounded to bf16 (nearest even); lse is the natural-log
 *   log-sum-exp  log sum_t exp(scale * q . k_t)  in fp32.
 *
 * Conventions:
 *   - Every pointer argument is DEVICE memory owned by the caller, except
 *     where marked (the allocator calls take host memory).  The GPU calls
 *     allocate nothing, device or host, and the library keeps no mutable
 *     global state; calls on different streams touching disjoint buffers are
 *     independent.  The only host allocation is a KV block allocator's own
 *     state, made by fe_kv_allocator_create and freed by
 *     fe_kv_allocator_destroy.
 *   - Every call is asynchronous on `stream` (0 = the null stream).  One
 *     stream orders an append before the attention that reads it.
 *   - Tensor pointers must be 16-byte aligned (FE_ERR_INVALID_ARG otherwise);
 *     the kernels move 16-byte units.
 *   - Return value: FE_OK (0), or a negative fe_status.  Argument errors are
 *     detected on the host before anything is enqueued, so outputs are
 *     untouched on error.  A failed launch returns FE_ERR_HIP.
 *     fe_last_error() then gives a per-thread message.  No C++ exception
 *     crosses this boundary.
 *   - Device-array contents are not checked on the host (that would need a
 *     synchronisation).  Kernels clamp instead of faulting: block ids are
 *     clamped into [0, num_blocks), context lengths into
 *     [0, min(max_context_len, max_blocks_per_seq * BS)], query rows named
 *     by query_start_loc into [0, total_q), and append slots outside
 *     [0, num_blocks * BS) are skipped.  Out-of-contract contents
 *     thus give unspecified results, never an out-of-bounds access.
 *   - Defined edge cases: a context length of 0 gives out = 0 and
 *     lse = -inf; block-table entries past ceil(L / BS) and pool slots past
 *     token L - 1 of a sequence's last block are never used (their contents,
 *     NaN included, cannot reach the output).
 */
#ifndef FE_H_
#define FE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FE_OK = 0,
  FE_ERR_NULL = -1,         /* a required pointer is NULL */
  FE_ERR_INVALID_ARG = -2,  /* negative/zero size, Hq % Hkv != 0, non-finite scale, ... */
  FE_ERR_UNSUPPORTED = -3,  /* a valid shape the library has no kernel for (D != 128, BS != 16, G > 8) */
  FE_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than the size query returns */
  FE_ERR_HIP = -5,          /* the HIP runtime reported an error at launch */
  FE_ERR_INTERNAL = -6,
  FE_ERR_CAPACITY = -7      /* the KV block allocator has too few free blocks (or a sequence's limit is reached) */
} fe_status;

/*
 * KV append: scatter new K/V rows into their cache slots.
 *   For every i in [0, T) with s = slot_mapping[i] in [0, num_blocks * BS):
 *     k_cache[s / BS][g][s % BS][:] = k_new[i][g][:]  for every KV head g,
 *     and the same for v.  A negative slot is padding and is skipped.
 *   This is a bit-exact copy; no other byte of the pools changes.
 *   k_new, v_new   bf16 [T][Hkv][D]
 *   slot_mapping   int32 [T]; slots must be distinct within one call
 *   k_cache, v_cache  bf16 [num_blocks][Hkv][BS][D], updated in place
 *   T == 0 is a valid no-op (pointers may then be NULL).
 * Source: ForgeEngine README, "What it implements" (paged KV cache) and the
 * architecture flowchart's write edge from prefill/decode into the cache.
 */
int fe_paged_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, void* k_cache,
                       void* v_cache, int T, int num_blocks, int Hkv, int D, int BS, hipStream_t stream);

/*
 * Bytes of device workspace fe_paged_gqa_decode needs for these sizes and
 * this num_partitions (0 = the automatic choice, which depends only on the
 * arguments here).  Host-only; returns 0 when no workspace is needed
 * (single partition) and (size_t)-1 for invalid sizes.  Hkv is an argument
 * because the automatic choice fills the GPU with (sequence, KV head,
 * partition) work items, whose count depends on it.
 * Source: ForgeLM README, "Core Principles" 1 (a small hot path with
 * controlled allocation: the caller sizes and owns the scratch memory); the
 * workspace holds the split-K partials of fe_paged_gqa_decode.
 */
size_t fe_paged_gqa_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_context_len,
                                          int num_partitions);

/*
 * Number of KV partitions fe_paged_gqa_decode uses for these arguments
 * (num_partitions 0 = automatic).  Host-only; -1 for invalid sizes.
 * Source: as fe_paged_gqa_decode_workspace_size.
 */
int fe_paged_gqa_decode_num_partitions(int B, int Hq, int Hkv, int D, int max_context_len,
                                       int num_partitions);

/*
 * Paged GQA decode: one query token per sequence over its block table.
 *   out           bf16 [B][Hq][D]
 *   lse           fp32 [B][Hq] natural log, or NULL
 *   q             bf16 [B][Hq][D]
 *   k_cache, v_cache  bf16 [num_blocks][Hkv][BS][D]
 *   block_tables  int32 [B][max_blocks_per_seq]
 *   context_lens  int32 [B]
 *   max_context_len  host-side upper bound of context_lens (sizes the grid)
 *   scale         softmax scale (usually fp32(1/sqrt(D))), must be finite
 *   num_partitions  split-K factor: the longest context is cut into this
 *                 many block-aligned ranges of equal size; each is reduced
 *                 to a normalised fp32 partial and an LSE, and a second
 *                 kernel merges them by log-sum-exp.  0 = automatic, 1 = one
 *                 pass with no workspace.  A range holds at most 256 blocks
 *                 (4096 tokens): a smaller value is raised to meet that, and
 *                 a value above the longest context's block count is lowered
 *                 (fe_paged_gqa_decode_num_partitions returns the value used).
 *   workspace     device scratch of at least
 *                 fe_paged_gqa_decode_workspace_size(...) bytes (may be NULL
 *                 when that size is 0), owned by the caller; contents are
 *                 clobbered and need no initialisation.  Calls that may
 *                 overlap in time (different streams) need different
 *                 workspaces.
 * Source: ForgeEngine README, "What it implements" (CUDA paged GQA kernel);
 * "Make the Engine Talk" section 1.2 (one pass per generated token) and
 * section 1.3 (grouped-query attention).
 */
int fe_paged_gqa_decode(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                        int B, int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len,
                        float scale, int num_partitions, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * fe_paged_gqa_decode without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *   Every argument, the result and the errors are those of
 *   fe_paged_gqa_decode (same kernels, same partitioning, bit-identical
 *   results), except that the split-K partials live in a device array of
 *   32 MiB inside the library: one copy per GPU, created with the code
 *   object and held until the process ends.  Its address on a device is
 *   looked up once (with that device current) on the first call for it.
 *   Sizes whose workspace (fe_paged_gqa_decode_workspace_size) exceeds
 *   32 MiB return FE_ERR_WORKSPACE before anything is enqueued; lower
 *   num_partitions or use fe_paged_gqa_decode.  Single-partition calls use
 *   no scratch at all.
 *   Every call on one GPU shares that GPU's array, and a call leaves its
 *   partials there: two calls that may overlap in time on one GPU (different
 *   streams, or graphs replayed concurrently) race on it and give
 *   unspecified results.  Calls ordered on one stream are safe.  The array
 *   needs no initialisation (every partial is written before it is read).
 *   A failed device lookup returns FE_ERR_HIP.
 * For callers that cannot allocate; the operation is that of
 * fe_paged_gqa_decode.
 */
int fe_paged_gqa_decode_noalloc(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                                int B, int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len,
                                float scale, int num_partitions, hipStream_t stream);

/*
 * fe_paged_kv_append of one new token per sequence fused into
 * fe_paged_gqa_decode: one launch instead of two for the per-token step
 * (append the token's K/V, then attend over the context that ends with it).
 *   k_new, v_new  bf16 [B][Hkv][D]: sequence b's new K and V rows
 *   slot_mapping  int32 [B]: the cache slot (block * BS + offset) of b's new
 *                 token, which is position context_lens[b] - 1, the last of
 *                 its context; a slot < 0 or >= num_blocks * BS is skipped
 *                 (nothing written) and that position is read from the cache
 *   k_cache, v_cache  written at those slots (bit copies), read as in
 *                 fe_paged_gqa_decode
 *   every other argument as fe_paged_gqa_decode (same workspace size)
 * The result equals fe_paged_kv_append(k_new, v_new, slot_mapping, ..., T = B)
 * followed by fe_paged_gqa_decode on the same arguments: the workgroup that
 * holds b's last block writes the row and attends to it from registers.
 * Preconditions (not checked): slot_mapping[b], when in range, is the slot of
 * position context_lens[b] - 1 in b's block table (a slot anywhere else in a
 * sequence's visible context makes that sequence's result unspecified);
 * slots are distinct; with context_lens[b] = 0 nothing is written for b.
 * Errors as fe_paged_gqa_decode, plus FE_ERR_NULL for NULL k_new, v_new or
 * slot_mapping and FE_ERR_INVALID_ARG for k_new or v_new not 16-byte aligned.
 * Source: ForgeEngine README, "What it implements" (paged KV cache written by
 * the engine, CUDA paged GQA kernel); "Make the Engine Talk" section 1.2 (each
 * generated token extends the cache, then one attention pass per token).
 */
int fe_paged_gqa_decode_append(void* out, float* lse, const void* q, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, void* k_cache, void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                               int B, int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len,
                               float scale, int num_partitions, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * The whole per-token attention step of a layer in one launch: the
 * per-head QK-RMSNorm + rotary embedding of fe_qk_norm_rope_append applied to
 * q and to the new k rows, the append of the new K/V rows, and decode.
 *   q             bf16 [B][Hq][D]: the projected (not yet normalised) queries
 *   k_new, v_new  bf16 [B][Hkv][D]: the projected new K and V rows
 *   q_norm_w, k_norm_w, cos_sin, max_pos, positions (int32 [B]), eps: as in
 *                 fe_qk_norm_rope_append (positions[b] is usually
 *                 context_lens[b] - 1)
 *   slot_mapping  int32 [B], with the preconditions of
 *                 fe_paged_gqa_decode_append
 *   every other argument as fe_paged_gqa_decode_append (same workspace size)
 * The result equals fe_qk_norm_rope_append(q_out, q, k_new, v_new, ...,
 * slot_mapping, k_cache, v_cache, T = B) followed by fe_paged_gqa_decode on
 * q_out (the same normalisation and rotation arithmetic, rounded to bf16 at
 * the same point), with no q_out written: each workgroup normalises and
 * rotates the q rows of its KV head itself, and the workgroup that holds b's
 * last block does the same to the new k row before it writes and attends to
 * it.  Errors as fe_paged_gqa_decode_append, plus FE_ERR_INVALID_ARG for
 * max_pos <= 0, an eps that is negative or not finite, or norm weights or
 * cos_sin not 16-byte aligned, and FE_ERR_NULL for a NULL q_norm_w, k_norm_w,
 * cos_sin or positions when B > 0.
 * Source: "Make the Engine Talk" sections 1.2-1.3 (each generated token
 * extends the cache and is attended to, after RMSNorm and rotary embedding);
 * ForgeEngine README, "What it implements" (RMSNorm kernel, paged KV cache,
 * CUDA paged GQA kernel).
 */
int fe_paged_gqa_decode_norm_rope_append(void* out, float* lse, const void* q, const void* k_new, const void* v_new,
                                         const void* q_norm_w, const void* k_norm_w, const float* cos_sin,
                                         int max_pos, const int32_t* positions, const int32_t* slot_mapping,
                                         void* k_cache, void* v_cache, const int32_t* block_tables,
                                         int max_blocks_per_seq, const int32_t* context_lens, int B, int Hq, int Hkv,
                                         int D, int BS, int num_blocks, int max_context_len, float scale, float eps,
                                         int num_partitions, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * Paged GQA prefill of a causal query chunk against the cached prefix.
 *   q              bf16 [total_q][Hq][D], sequences packed back to back
 *   query_start_loc  int32 [B + 1] DEVICE array; sequence b owns packed rows
 *                  query_start_loc[b] .. query_start_loc[b+1] - 1 (C_b rows)
 *   context_lens   int32 [B]: prefix + chunk; the chunk's K/V must already
 *                  be in the cache (fe_paged_kv_append on the same stream)
 *   Row query_start_loc[b] + i sits at position L_b - C_b + i and attends to
 *   tokens 0 .. L_b - C_b + i (bottom-right causal alignment).
 *   out            bf16 [total_q][Hq][D]
 *   lse            fp32 [total_q][Hq] natural log, or NULL
 *   max_q_len      host-side upper bound of every C_b (sizes the grid)
 *   max_context_len  host-side upper bound of context_lens
 *   QK^T and PV run on the bf16 MFMA units with fp32 accumulation; the
 *   softmax weights are rounded to bf16 for the PV product.
 * Source: ForgeEngine README, "What it implements" (restricted prefill lab)
 * and "Scheduling" (token-budgeted batching, which cuts prompts into
 * chunks); "Make the Engine Talk" section 1.2 (the prefill pass).
 */
int fe_paged_gqa_prefill_chunk(void* out, float* lse, const void* q, const int32_t* query_start_loc,
                               const void* k_cache, const void* v_cache, const int32_t* block_tables,
                               int max_blocks_per_seq, const int32_t* context_lens, int B, int total_q,
                               int max_q_len, int Hq, int Hkv, int D, int BS, int num_blocks,
                               int max_context_len, float scale, hipStream_t stream);

/*
 * fe_paged_gqa_prefill_chunk with the kernel's tile shape and the precision
 * of the softmax weights in the PV product chosen by the caller; every other
 * argument, the result's definition and the errors are the same.
 *   key_groups     0 = automatic (what fe_paged_gqa_prefill_chunk does);
 *                  1 = each workgroup walks its keys with one group of waves
 *                  (two workgroups fit on a compute unit);
 *                  2 = two wave groups split the keys and merge by
 *                  log-sum-exp (one workgroup per compute unit);
 *                  3 = two wave groups take two consecutive query tiles over
 *                  one shared stream of K/V tiles (one workgroup per
 *                  compute unit, half as many workgroups);
 *                  2 is valid only for Hq/Hkv <= 4 and 3 only for Hq/Hkv in
 *                  {1, 2, 4}, else FE_ERR_UNSUPPORTED.  Other values:
 *                  FE_ERR_INVALID_ARG.
 * The automatic choice takes 2 when the launch has at most one workgroup
 * per compute unit, 3 above that (1 when a chunk has a single query tile or
 * Hq/Hkv = 3), and 1 for Hq/Hkv > 4.  The shapes differ only in the order of fp32
 * additions, so results agree within rounding, not bit for bit.
 *   split_weights  0 = each softmax weight enters the PV product rounded to
 *                  bf16 (what fe_paged_gqa_prefill_chunk does: at most 2^-8
 *                  relative per weight); 1 = as two bf16 parts, the rounded
 *                  weight and its rounded remainder (at most 2^-16 relative),
 *                  which doubles the PV product's MFMA work (30-40% more
 *                  time).  On a row dominated by two or three keys with
 *                  output values near 2-4, the error of 0 plus the output's
 *                  own bf16 rounding can exceed 1e-2; with 1 what remains
 *                  is essentially the output's own rounding.  Other values:
 *                  FE_ERR_INVALID_ARG.
 * Source: as fe_paged_gqa_prefill_chunk.
 */
int fe_paged_gqa_prefill_chunk_ex(void* out, float* lse, const void* q, const int32_t* query_start_loc,
                                  const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* context_lens, int B, int total_q,
                                  int max_q_len, int Hq, int Hkv, int D, int BS, int num_blocks,
                                  int max_context_len, float scale, int key_groups, int split_weights,
                                  hipStream_t stream);

/*
 * Bytes of device workspace fe_paged_gqa_mixed needs for these sizes
 * (num_partitions 0 = automatic).  Host-only; 0 when no decode sequence is
 * split, (size_t)-1 for invalid sizes.
 * Source: ForgeLM README, "Core Principles" 1 (controlled allocation); the
 * workspace holds the arrival counters and partials of fe_paged_gqa_mixed.
 */
size_t fe_paged_gqa_mixed_workspace_size(int num_decode, int Hq, int Hkv, int D, int max_context_len,
                                         int num_partitions);

/*
 * Mixed batch in ONE kernel launch: decode rows and prefill chunks together,
 * the step a token-budgeted continuous batcher produces.
 *   Sequences b in [0, num_decode) are decode rows: each owns exactly one
 *   packed query row, query_start_loc[b], and attends over its whole context
 *   (as fe_paged_gqa_decode).  Sequences b in [num_decode, B) are prefill
 *   chunks (as fe_paged_gqa_prefill_chunk: bottom-right causal).  A decode
 *   row is thus the chunk of length one of its sequence; results equal those
 *   of the two separate calls within their tolerances.
 *   out, lse, q, query_start_loc, k_cache, v_cache, block_tables,
 *   context_lens, total_q, max_context_len, scale: as in
 *   fe_paged_gqa_prefill_chunk, over all B sequences.
 *   max_q_len      host-side upper bound of the prefill chunks' lengths
 *   num_partitions split-K factor of the decode rows (0 = automatic: ranges
 *                  of at least 64 blocks, and no more than about 6 decode
 *                  items (sequence, KV head, partition) per compute unit),
 *                  at most 256 blocks per range as in decode
 *   workspace      device scratch of at least
 *                  fe_paged_gqa_mixed_workspace_size(...) bytes (NULL when
 *                  that is 0), owned by the caller.  It must be zero-filled
 *                  once before its first use: it starts with num_decode * Hkv
 *                  arrival counters (the last partition of a split decode
 *                  row to finish merges the partials in the same launch),
 *                  which every completed call leaves at zero again; the rest
 *                  is clobbered.  Calls that may overlap in time need
 *                  different workspaces.
 *   Preconditions on device contents (not checked): query_start_loc[b] = b
 *   and query_start_loc[b + 1] - query_start_loc[b] = 1 for b < num_decode.
 * Source: ForgeEngine README, "Scheduling" (continuous, token-budgeted
 * batching) and "What it implements" (paged GQA kernel, restricted prefill
 * lab); "Make the Engine Talk" section 1.2.
 */
int fe_paged_gqa_mixed(void* out, float* lse, const void* q, const int32_t* query_start_loc, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, int B, int num_decode, int total_q, int max_q_len, int Hq,
                       int Hkv, int D, int BS, int num_blocks, int max_context_len, float scale, int num_partitions,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fused per-head QK-RMSNorm + rotary embedding + KV append: the step just
 * before attention, done in one pass so the normed and rotated k does not
 * make a round trip through HBM before it is appended.
 *   For every token i in [0, T), in fp32, rounded once to bf16 (nearest even):
 *     each q head row x = q[i][h] and k head row x = k[i][g]:
 *       y = x * w / sqrt(mean_d(x[d]^2) + eps)   (w = q_norm_w or k_norm_w)
 *       with p = positions[i] clamped into [0, max_pos), for d < D/2:
 *         c = cos_sin[p][d], s = cos_sin[p][D/2 + d]
 *         out[d] = y[d] c - y[D/2 + d] s,  out[D/2 + d] = y[D/2 + d] c + y[d] s
 *     q_out[i][h] = out of q head h;
 *     with s = slot_mapping[i] in [0, num_blocks * BS): the cache slot s of KV
 *     head g gets out of k head g (k_cache) and v[i][g] bit for bit (v_cache);
 *     other slots are skipped (q_out is still written).
 *   q, q_out       bf16 [T][Hq][D]; q_out may be q itself (in place)
 *   k, v           bf16 [T][Hkv][D]
 *   q_norm_w, k_norm_w  bf16 [D]
 *   cos_sin        fp32 [max_pos][D]: the cosines of the D/2 angles of a
 *                  position, then their sines (the caller's rotary table)
 *   positions      int32 [T]
 *   slot_mapping, k_cache, v_cache: as in fe_paged_kv_append
 *   eps            finite, >= 0
 *   All tensor pointers 16-byte aligned.  T == 0 is a no-op.
 * Source: "Make the Engine Talk" section 1.3 (RMSNorm and rotary position
 * embeddings among the forward pass's mechanisms); ForgeEngine README, "What
 * it implements" (RMSNorm kernel, paged KV cache).  The formulas are this
 * library's reading: the pages name the mechanisms only.
 */
int fe_qk_norm_rope_append(void* q_out, const void* q, const void* k, const void* v, const void* q_norm_w,
                           const void* k_norm_w, const float* cos_sin, int max_pos, const int32_t* positions,
                           const int32_t* slot_mapping, void* k_cache, void* v_cache, int T, int Hq, int Hkv, int D,
                           int BS, int num_blocks, float eps, hipStream_t stream);

/*
 * Bytes of device workspace fe_sampler_softmax_argmax needs for B rows of
 * V logits (host-only; (size_t)-1 for invalid sizes).
 * Source: ForgeLM README, "Core Principles" 1 (controlled allocation); the
 * workspace holds the per-range partials of fe_sampler_softmax_argmax.
 */
size_t fe_sampler_workspace_size(int B, int V);

/*
 * The sampler's hot step over each row b of bf16 logits [B][V], at inverse
 * temperature s = inv_temperature[b] (NULL: 1), in fp32:
 *   probs[b][i] = exp(s x_i - m) / sum_j exp(s x_j - m),  m = max_j s x_j
 *   lse[b]      = m + log sum_j exp(s x_j - m)            (natural log)
 *   argmax[b]   = the lowest i with x_i = max_j x_j       (greedy token, exact)
 *   -inf logits are masked tokens (probability 0); a row of only -inf gives
 *   probabilities 0, lse = -inf and argmax 0.
 *   probs          fp32 [B][V], or NULL (argmax / lse only)
 *   lse            fp32 [B], or NULL
 *   argmax         int32 [B]
 *   logits         bf16 [B][V]; V must be a multiple of 8 (FE_ERR_UNSUPPORTED)
 *   inv_temperature  fp32 [B] (> 0, finite; not checked) or NULL
 *   workspace      device scratch of fe_sampler_workspace_size(B, V) bytes,
 *                  clobbered (required; the one-workgroup-per-row form
 *                  leaves it untouched)
 * Runs the form fe_sampler_softmax_argmax_ex picks with form 0.
 * Source: "Make the Engine Talk" section 1.3 (the sampler: greedy,
 * temperature and top-p decoding, with its softmax in fp32 over a vocabulary
 * this wide); ForgeEngine README, "What it implements" (sampling policies).
 */
int fe_sampler_softmax_argmax(float* probs, float* lse, int32_t* argmax, const void* logits,
                              const float* inv_temperature, int B, int V, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * fe_sampler_softmax_argmax with the kernel form chosen by the caller; the
 * results are the same up to fp32 summation order.
 *   form 0  automatic: form 2 when V <= 163,840 and B >= 160 with B mod 256
 *           either 0 or at least 160 (every round of 256 workgroups, one per
 *           CU, holds at least 160 rows), else form 1
 *   form 1  ranges: each row cut into ranges over about 1024 workgroups, a
 *           pass for the ranges' partials and a pass that merges them and
 *           writes (two launches; the logits are read twice)
 *   form 2  one workgroup of 1024 threads per row, the row held in registers
 *           (one launch, the logits read once; a CU streams one row at a few
 *           tens of GB/s, so it pays only when the rows cover the CUs);
 *           FE_ERR_UNSUPPORTED when V > 163,840
 *   other   FE_ERR_INVALID_ARG
 * Other arguments and errors as fe_sampler_softmax_argmax.
 * Source: as fe_sampler_softmax_argmax.
 */
int fe_sampler_softmax_argmax_ex(float* probs, float* lse, int32_t* argmax, const void* logits,
                                 const float* inv_temperature, int B, int V, int form, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * The form (1 or 2) that form 0 of fe_sampler_softmax_argmax_ex runs for B
 * rows of V logits (host-only; -1 for invalid sizes).
 * Source: as fe_sampler_softmax_argmax.
 */
int fe_sampler_form(int B, int V);

/*
 * Paged KV block allocator (host memory, host calls only): hands out the
 * cache blocks whose slots fe_paged_kv_append fills and whose ids the
 * attention calls read through block_tables.
 *   The free blocks form a stack that starts as 0, 1, 2, ... from the top.
 *   fe_kv_allocator_append pops the blocks a sequence's new tokens need;
 *   fe_kv_allocator_release pushes all of a sequence's blocks back in reverse
 *   token order (its first block on top).  Which blocks a call receives
 *   therefore depends only on the sequence of calls (deterministic cleanup:
 *   after every sequence is finished or cancelled and released,
 *   fe_kv_allocator_num_allocated is 0).
 *   Sequences are ids 0 .. max_seqs - 1, chosen by the caller; each holds at
 *   most max_blocks_per_seq blocks.  One thread owns an allocator (the
 *   scheduler): calls on one allocator must not overlap.
 * Source: ForgeEngine README, "What it implements" (paged block allocator
 * with deterministic cleanup), "Loading" (one worker owns KV-cache mutation)
 * and its measurements table (final allocated KV blocks: 0 after finished and
 * cancelled requests).
 */
typedef struct fe_kv_allocator fe_kv_allocator;

/* NULL for non-positive sizes, num_blocks * block_size (or a sequence's
 * token limit) beyond INT32_MAX, or failed host allocation. */
fe_kv_allocator* fe_kv_allocator_create(int num_blocks, int block_size, int max_seqs, int max_blocks_per_seq);
void fe_kv_allocator_destroy(fe_kv_allocator* a);

/* Reserve slots for n new tokens at the end of sequence seq and write them
 * to slots_out (host int32[n]; slot = block * block_size + offset).  All or
 * nothing: FE_ERR_CAPACITY when the free blocks or the sequence's block limit
 * do not suffice (nothing changes); n == 0 is a no-op. */
int fe_kv_allocator_append(fe_kv_allocator* a, int seq, int n, int32_t* slots_out);

/* Release every block of sequence seq (finished or cancelled); its length
 * becomes 0.  Releasing an empty sequence is a no-op. */
int fe_kv_allocator_release(fe_kv_allocator* a, int seq);

/* Tokens held by sequence seq (>= 0), or a negative status. */
int fe_kv_allocator_seq_len(const fe_kv_allocator* a, int seq);
int fe_kv_allocator_num_free(const fe_kv_allocator* a);
int fe_kv_allocator_num_allocated(const fe_kv_allocator* a);

/* Attention inputs for a batch of sequences (host arrays): row i of
 * block_tables ([n][row_len]) lists seqs[i]'s blocks in token order, padded
 * with pad_block; context_lens[i] is its length.  FE_ERR_CAPACITY when a
 * sequence holds more than row_len blocks. */
int fe_kv_allocator_batch(const fe_kv_allocator* a, const int* seqs, int n, int32_t* block_tables, int row_len,
                          int32_t pad_block, int32_t* context_lens);

/*
 * Measurement helper, not part of the attention path: the HBM read ceiling
 * of the decode kernel's load form, for benchmarks to report beside the
 * kernels' rates.  Reads the n whole 4 KiB tiles base[tile_ids[i] * 4096 ..
 * + 4095] (i < n), each with one wave's four 1 KiB runs of non-temporal
 * 16-byte buffer loads, 16 tiles per wave, and XOR-folds each wave's data
 * into sink[i / 16] (sink: uint32 [ceil(n / 16)], device, overwritten).
 *   base       device buffer of num_tiles * 4096 bytes, 16-byte aligned
 *   tile_ids   int32 [n] device; ids outside [0, num_tiles) are skipped
 *              (never read)
 * Asynchronous on `stream`; n == 0 is a no-op.  Errors: FE_ERR_NULL,
 * FE_ERR_INVALID_ARG (num_tiles <= 0, n < 0, misaligned base), FE_ERR_HIP.
 * Source: ForgeLM README, "Tooling and Benchmarks" (performance claims need
 * reproducible measurement) and "Documentation" ("Measured optimization over
 * speculative abstraction").
 */
int fe_hbm_read_probe(const void* base, int64_t num_tiles, const int32_t* tile_ids, int n, uint32_t* sink,
                      hipStream_t stream);

/*
 * Measurement helper, not part of the attention path: the bf16 MFMA rate the
 * device sustains with the prefill tile's instruction
 * (v_mfma_f32_32x32x16_bf16, 32 x 32 x 16, 32768 flop each).  Launches
 * `workgroups` workgroups of 8 waves (two per SIMD, as the prefill tile
 * runs); wave i loads 8 A and 8 B operands per lane from `operands`
 * (16-byte entries ((i * 16 + k) * 64 + lane) mod n_ops, k < 16), then issues
 * rounds * 64 MFMAs on 8 independent accumulators (round r, step j pairs
 * accumulator k with A[(j + k) mod 8] and B[k]) and writes the sum of its
 * accumulators to sink[i].  Flops of a call:
 * workgroups * 8 * rounds * 64 * 32768.
 *   operands    device, n_ops 16-byte entries of bf16 pairs, 16-byte aligned
 *   sink        fp32 [workgroups * 8], device, overwritten
 * Asynchronous on `stream`; workgroups == 0 is a no-op.  Errors: FE_ERR_NULL,
 * FE_ERR_INVALID_ARG (n_ops <= 0, workgroups or rounds < 0, misaligned
 * operands), FE_ERR_UNSUPPORTED (a grid of 2^31 threads or more), FE_ERR_HIP.
 * Source: ForgeLM README, "Tooling and Benchmarks" (performance claims need
 * reproducible measurement) and "Documentation" ("Measured optimization over
 * speculative abstraction").
 */
int fe_mfma_rate_probe(const void* operands, int n_ops, int workgroups, int rounds, float* sink, hipStream_t stream);

/*
 * Static description of a status code (never NULL; "FE_ERR_UNKNOWN" for a
 * value that is not an fe_status).
 * Source: ForgeLM README, "Proposed Stack" (a C/C++ native backend reached
 * through FFI bindings, across which errors travel as status codes, not
 * exceptions); ForgeEngine README, "Verified L4 results" (parameter
 * validation is part of what its tests check).
 */
const char* fe_status_string(int status);

/*
 * Detail of the most recent failure on the calling thread ("" if none): the
 * function, the argument or size that failed a check, or the HIP error text.
 * Valid until the next failing call on the same thread.
 * Source: as fe_status_string.
 */
const char* fe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FE_H_ */
