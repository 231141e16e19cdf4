/*
 * pkv.h -- C ABI of libpkv, attention over a block-paged KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * The operations are those of a single-GPU continuous-batching inference
 * engine described on the pages "Inference Server" (project README mirror,
 * section "The engine"; GitHub README, section "What's inside") and
 * "Inference Server -- Architecture Map" (section "How a single request flows
 * through the system"):
 *   - a block-paged, per-layer K/V cache in the vLLM/PagedAttention layout,
 *     with refcounted (shared) blocks and window-aware sliding layers;
 *   - paged decode and prefill attention reading K/V through per-sequence
 *     block tables, with a split-K decode variant;
 *   - chunked prefill: a chunk of new tokens is appended to the cache, then
 *     attends causally over the cached prefix and the chunk;
 *   - one batched decode per engine tick over all active sequences, one new
 *     token each; GQA and tanh logit softcapping (Gemma-style models).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer to caller-owned memory,
 *   16-byte aligned, dense and row-major in the shape given.  The library
 *   never allocates or frees memory and keeps no pointer after it returns.
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *   enqueue work and return; buffers must stay alive until the stream has
 *   executed it.  No call synchronises.
 * dtype.  PKV_BF16 or PKV_F32; q, out, new K/V rows and both pools share it.
 *   Accumulation is always fp32; bf16 results are rounded to nearest even.
 * Block pool (vLLM/PagedAttention layout), X = 16 / sizeof(element):
 *     k_pool [num_blocks, num_kv_heads, head_dim / X, 16, X]
 *     v_pool [num_blocks, num_kv_heads, head_dim, 16]
 *   Token t of sequence b lives in block block_tables[b * max_blocks_per_seq
 *   + t / 16] at offset t % 16.  Block size is fixed at 16.
 * Lengths.  context_lens[b] counts all cached tokens of sequence b, the token
 *   just appended included.  A decode query sits at position
 *   context_lens[b] - 1.
 * GQA.  num_q_heads = gqa_group * num_kv_heads; query head h reads kv head
 *   h / gqa_group.
 * Window.  window > 0 keeps key t for a query at q_pos iff q_pos - t < window
 *   (the last `window` tokens, the query's own included); <= 0 disables it.
 * Softcap.  softcap > 0 replaces each logit s = scale * q.k by
 *   softcap * tanh(s / softcap); <= 0 disables it.
 * Errors.  Every `int` function returns PKV_OK (0) or a negative code; the
 *   message of the calling thread's last failure is pkv_last_error().
 *   Validation reads only the scalar arguments, never device memory; a failed
 *   call enqueues nothing.  Device contents are the caller's contract
 *   (0 <= block id < num_blocks, 0 <= context_lens[b] <=
 *   max_blocks_per_seq * 16, distinct non-negative slots); the kernels clamp
 *   lengths and skip out-of-range block ids and slots instead of touching
 *   memory outside the pools, but results are then unspecified.
 * Reentrancy.  Calls are thread-safe.  Calls that share a workspace must not
 *   overlap in time (use one workspace per stream in flight).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* = hipStream_t */

enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1 };

enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = -1,       /* null pointer, negative size, inconsistent shape     */
  PKV_EUNSUPPORTED = -2, /* dtype, head_dim not in {64,128,256}, block_size != 16,
                            gqa_group outside what the entry point supports,
                            partition_size not a positive multiple of 16        */
  PKV_EWORKSPACE = -3,   /* workspace null or smaller than the size query says  */
  PKV_EHIP = -4,         /* the HIP runtime reported an error at launch         */
  PKV_ENOMEM = -5        /* the block allocator has too few free blocks, or the
                            host is out of memory                               */
};

#define PKV_BLOCK_SIZE 16

/*
 * paged_kv_append -- write new K/V rows into their cache slots.
 * The KV cache is paged in fixed-size blocks (page "Inference Server", section
 * "The engine"): the K/V of every new token is copied into the slot the host reserved for it;
 * a chunk of a long prompt is appended this way before it attends (chunked
 * prefill, page "Inference Server -- Architecture Map", section "How a single
 * request flows through the system"), and so is each decode token.
 *
 *   k_new, v_new  [num_tokens, num_kv_heads, head_dim]   rows to write
 *   slot_mapping  int32 [num_tokens]: slot = block * 16 + offset; a negative
 *                 slot skips the token (padding).  Slots must be distinct.
 *   k_pool, v_pool  the pools above, updated in place.
 * The copy is bit-exact.  num_tokens == 0 is a no-op.
 */
int paged_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    int32_t num_tokens, void* k_pool, void* v_pool, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                    struct ihipStream_t* stream);

/*
 * paged_kv_copy_blocks -- copy-on-write block copies inside the pools.  The
 * cache is block-paged with refcounted blocks (page "Inference Server",
 * section "The engine"): sequences that share a prefix hold the same
 * physical blocks, and a sequence about to write into a shared block first
 * gets a private copy of it.  This copies, for each pair i, the whole block
 * src_ids[i] to block dst_ids[i] in both pools (every kv head, all 16 slots).
 *
 *   k_pool, v_pool  the pools (paged_kv_append's layout), updated in place
 *   src_ids, dst_ids  int32 [num_pairs] device arrays
 * A pair with an id outside [0, num_blocks), or with src == dst, is skipped.
 * The destinations must be distinct and none may be a source of another
 * pair (otherwise the result depends on the order of the copies).  The copy
 * is bit-exact.  num_pairs == 0 is a no-op.
 */
int paged_kv_copy_blocks(void* k_pool, void* v_pool, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, const int32_t* src_ids,
                         const int32_t* dst_ids, int32_t num_pairs, int32_t dtype,
                         struct ihipStream_t* stream);

/*
 * pkv_check_paged_metadata -- check, on the device, the caller's side of the
 * contract every other entry point trusts: the block tables and context
 * lengths (page "Inference Server", section "The engine": K/V in fixed-size
 * blocks reached through per-sequence block tables) and an append's slot
 * mapping.  The attention and append kernels never read or write outside
 * the pools when these arrays are wrong, but their results are then
 * unspecified; this call reports the mistake instead.
 *
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]   (null if num_seqs == 0)
 *   context_lens  int32 [num_seqs]                       (null if num_seqs == 0)
 *   slot_mapping  int32 [num_slots]                      (null if num_slots == 0)
 *   flags         uint32 [1] device word: cleared, then the OR of
 *     PKV_CHECK_BAD_CONTEXT_LEN  some context_lens[b] < 0 or > max_blocks_per_seq * 16
 *     PKV_CHECK_BAD_BLOCK_ID     some entry block_tables[b][j] with j * 16 < context_lens[b]
 *                                (an entry the sequence reads) outside [0, num_blocks)
 *     PKV_CHECK_BAD_SLOT         some slot >= num_blocks * 16 (negative slots are skips)
 *     PKV_CHECK_DUPLICATE_SLOT   two rows share a non-negative slot
 * Entries past a sequence's length are not checked.  The word is valid once
 * the stream reaches the call.  The duplicate test compares every pair of
 * slots (num_slots^2 reads): a debugging aid, not for the serving loop.
 * Calls sharing one flags word must not overlap in time.
 */
#define PKV_CHECK_BAD_CONTEXT_LEN 1u
#define PKV_CHECK_BAD_BLOCK_ID 2u
#define PKV_CHECK_BAD_SLOT 4u
#define PKV_CHECK_DUPLICATE_SLOT 8u
int pkv_check_paged_metadata(const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                             const int32_t* slot_mapping, int32_t num_slots, uint32_t* flags,
                             struct ihipStream_t* stream);

/*
 * pkv_block_allocator -- the host side of refcounted blocks (page "Inference
 * Server", section "The engine"): hands out block ids, counts the block
 * tables holding each block, and prepares copy-on-write before a sequence
 * writes into blocks it shares.  Host memory only, no HIP calls; every
 * function locks the allocator, so calls from several threads are safe.
 *
 *   create: an allocator of num_blocks ids, all free (handed out 0, 1, ...).
 *   alloc: n fresh ids (refcount 1) into ids[0..n); all or nothing
 *     (PKV_ENOMEM if fewer than n are free).
 *   share: one more holder for each listed id (a table that now also holds
 *     it, e.g. a forked prefix); every id must be allocated.
 *   release: one holder fewer for each listed id (repeats count); a block
 *     whose count reaches 0 is free again.  All or nothing.
 *   prepare_write: a sequence is about to write into logical blocks
 *     [first, last] of its table row (host memory).  Every such block held
 *     by more than one table is replaced in table_row by a fresh private
 *     block; the pair (old, new) is written to src_ids / dst_ids (room for
 *     last - first + 1 pairs) and counted in *num_copies; the old block loses
 *     this holder.  The caller then copies the pairs with
 *     paged_kv_copy_blocks before writing.  All or nothing (PKV_ENOMEM if
 *     too few blocks are free).
 *   num_free, refcount: -1 for a null allocator or an out-of-range id.
 */
typedef struct pkv_block_allocator pkv_block_allocator;
int pkv_allocator_create(pkv_block_allocator** allocator, int32_t num_blocks);
void pkv_allocator_destroy(pkv_block_allocator* allocator);
int pkv_allocator_alloc(pkv_block_allocator* allocator, int32_t n, int32_t* ids);
int pkv_allocator_share(pkv_block_allocator* allocator, const int32_t* ids, int32_t n);
int pkv_allocator_release(pkv_block_allocator* allocator, const int32_t* ids, int32_t n);
int pkv_allocator_prepare_write(pkv_block_allocator* allocator, int32_t* table_row, int32_t first,
                                int32_t last, int32_t* src_ids, int32_t* dst_ids,
                                int32_t* num_copies);
int32_t pkv_allocator_num_free(pkv_block_allocator* allocator);
int32_t pkv_allocator_refcount(pkv_block_allocator* allocator, int32_t block);

/*
 * paged_attn_decode_workspace_size -- bytes of device workspace that
 * paged_attn_decode (partition_size == 0) or paged_attn_decode_splitk
 * (partition_size > 0) needs for these sizes.  Depends on the arguments only.
 * Returns 0 for invalid sizes.
 *
 * The workspace holds one counter per (sequence, kv head) (a fixed 256 KiB
 * region at its start: num_seqs * num_kv_heads <= 65536, else
 * PKV_EUNSUPPORTED) and the partial results.  It must be zero-filled once,
 * before its first use; every call leaves the counters at zero again, so
 * the same workspace serves any number of calls in a row (with any sizes it
 * is large enough for) without being cleared.  The caller must not write it
 * between calls.
 */
size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t gqa_group, int32_t head_dim,
                                        int32_t max_context_len, int32_t partition_size);

/*
 * paged_attn_decode -- batched one-token decode over the block-paged cache.
 * The engine's decode kernel reads K/V through per-sequence block tables (page
 * "Inference Server", section "The engine"); one batched decode per tick over every
 * active request (page "Inference Server -- Architecture Map", section "How a
 * single request flows through the system").
 *
 *   out           [num_seqs, num_kv_heads * gqa_group, head_dim]
 *   lse           optional fp32 [num_seqs, num_q_heads], natural-log
 *                 log-sum-exp of each row's logits (NULL: not written)
 *   q             [num_seqs, num_q_heads, head_dim]
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]
 *   context_lens  int32 [num_seqs];  max_context_len >= every entry and
 *                 <= max_blocks_per_seq * 16
 *   gqa_group     1 .. 16
 *   workspace     >= paged_attn_decode_workspace_size(..., 0) bytes
 * The work over all (sequence, kv head, block) triples is split evenly across
 * the GPU in one launch; the partial results of a split (sequence, kv head)
 * are merged by log-sum-exp by the workgroup that finishes its last piece.
 * A sequence with context length 0 gets out = 0 and lse = -inf.
 */
int paged_attn_decode(void* out, float* lse, const void* q, const void* k_pool,
                      const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                      int32_t gqa_group, int32_t head_dim, int32_t block_size, float scale,
                      float softcap, int32_t window, void* workspace, size_t workspace_bytes,
                      int32_t dtype, struct ihipStream_t* stream);

/*
 * paged_attn_decode_splitk -- the split-K decode variant (page "Inference
 * Server", section "The engine").  Sequence b's tokens are cut into
 * partitions [p * partition_size, (p + 1) * partition_size), anchored at
 * token 0; each partition's (max logit, sum of exponentials, partial output)
 * enters a log-sum-exp merge.  The partitions are the units of work: each
 * workgroup (one per compute unit) takes a run of consecutive partitions,
 * folds those of one sequence and kv head as their blocks stream (the online
 * softmax over a run is the log-sum-exp merge of its partitions' partials)
 * and stores one partial per run; the runs are merged by log-sum-exp in the
 * same launch.  (Where that form's LDS does not fit -- bf16 with a GQA group
 * of 8 or more at head_dim 256, or 16 at head_dim 128 -- and for fp32, each
 * partition is a workgroup of its own.)  The result equals the
 * partition-by-partition merge up to rounding order.  Arguments as
 * paged_attn_decode, plus
 *   partition_size  tokens per partition, a positive multiple of 16
 *   workspace       >= paged_attn_decode_workspace_size(..., partition_size)
 */
int paged_attn_decode_splitk(void* out, float* lse, const void* q, const void* k_pool,
                             const void* v_pool, int32_t num_blocks,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len,
                             int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                             int32_t head_dim, int32_t block_size, float scale, float softcap,
                             int32_t window, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, int32_t dtype, struct ihipStream_t* stream);

/*
 * paged_attn_decode_no_alloc -- paged_attn_decode (partition_size == 0) or
 * paged_attn_decode_splitk (partition_size > 0) without a caller workspace
 * and without any allocation, for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments and results as those two
 * entry points, minus the workspace.
 *
 * The workspace is a static device array of the library, 32.5 MiB per GPU
 * (the largest balanced-split workspace: gqa_group 16, head_dim 256), held
 * from the first call on a GPU until the process ends.  Sizes whose
 * workspace would exceed it (paged_attn_decode_workspace_size) are rejected
 * with PKV_EWORKSPACE; the balanced split (partition_size == 0) always fits.
 * The first call on each GPU also enqueues, on `stream`, a small kernel that
 * clears the array's counters; every completed call leaves them at zero.
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU (other streams, other threads, the first call included) race and give
 * wrong results.  No hipMalloc, hipFree or other allocation is made.
 */
int paged_attn_decode_no_alloc(void* out, float* lse, const void* q, const void* k_pool,
                               const void* v_pool, int32_t num_blocks,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len,
                               int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                               int32_t head_dim, int32_t block_size, float scale, float softcap,
                               int32_t window, int32_t partition_size, int32_t dtype,
                               struct ihipStream_t* stream);

/*
 * paged_attn_decode_append -- one decode tick in one launch: the append of
 * every sequence's newest token and the batched decode that attends to it.
 * Each tick appends the token every active request just produced and runs
 * one batched decode over all of them (page "Inference Server --
 * Architecture Map", section "How a single request flows through the
 * system"); the append writes into the block-paged pool (page "Inference
 * Server", section "The engine").
 *
 * Arguments as paged_attn_decode (partition_size == 0) or
 * paged_attn_decode_splitk (partition_size > 0), plus
 *   k_new, v_new  [num_seqs, num_kv_heads, head_dim], the pool's dtype,
 *                 16-byte aligned: the newest token's K and V rows
 *   k_pool, v_pool  written as well as read
 * Sequence b's newest token is position L_b - 1, L_b = min(context_lens[b],
 * max_context_len, max_blocks_per_seq * 16) (so context_lens counts it); it
 * goes to slot block_tables[b][(L_b - 1) / 16] * 16 + (L_b - 1) % 16 of every
 * kv head, exactly as paged_kv_append with those slots would write it, and
 * the outputs equal those of paged_kv_append followed by paged_attn_decode
 * (or _splitk).  Sequences with L_b == 0, with context_lens[b] >
 * max_context_len (a caller error: the clamped position holds an older
 * token, which is left alone), or whose entry for that block is outside
 * [0, num_blocks), append nothing.  Within one call, no block that
 * receives a token may be read by another sequence (a block shared by
 * several sequences is copied before it is appended to).
 * Errors as paged_attn_decode; PKV_EINVAL also for a missing or misaligned
 * k_new / v_new.
 */
int paged_attn_decode_append(void* out, float* lse, const void* q, const void* k_new,
                             const void* v_new, void* k_pool, void* v_pool, int32_t num_blocks,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len,
                             int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                             int32_t head_dim, int32_t block_size, float scale, float softcap,
                             int32_t window, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, int32_t dtype, struct ihipStream_t* stream);

/*
 * paged_attn_decode_sink_h2o -- the decode variants behind two of the
 * engine's eviction policies, AttentionSink and H2O (page "Inference
 * Server", GitHub README, section "What's inside"), on the balanced split of
 * paged_attn_decode.  Arguments as paged_attn_decode, plus
 *   sink_tokens   with window > 0, tokens [0, sink_tokens) stay visible
 *                 beside the window (the attention sinks); 0: plain window.
 *                 Ignored without a window (every token is visible then).
 *   scores        NULL, or fp32 [num_seqs, num_q_heads, score_stride],
 *                 16-byte aligned: receives the natural-log logits of every
 *                 token of the blocks the decode reads (-inf where not
 *                 visible); other entries are left alone
 *   column_mass   NULL, or fp32 [num_seqs, num_kv_heads, score_stride]:
 *                 mass[b, g, t] = sum over the group's query heads h of the
 *                 softmax weight of token t, exp(logit - lse); 0 for tokens
 *                 not visible (the whole row is written).  Needs scores and
 *                 lse.
 *   score_stride  a multiple of 16, >= max_context_len (when column_mass)
 * Errors as paged_attn_decode; PKV_EINVAL for a negative sink_tokens,
 * scores without column_mass (or the reverse), column_mass without lse, or a
 * bad score_stride / alignment.  With column_mass, two kernels run (the
 * decode writes logits and lse, a second one forms the mass).
 */
int paged_attn_decode_sink_h2o(void* out, float* lse, const void* q, const void* k_pool,
                               const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                               int32_t gqa_group, int32_t head_dim, int32_t block_size,
                               float scale, float softcap, int32_t window, int32_t sink_tokens,
                               float* scores, float* column_mass, int32_t score_stride,
                               void* workspace, size_t workspace_bytes, int32_t dtype,
                               struct ihipStream_t* stream);

/*
 * pkv_decode_graph -- a decode tick (paged_attn_decode_append) captured once
 * into a HIP graph for one batch-size bucket and replayed every tick: the
 * engine replays decode steps captured per batch-size bucket (page
 * "Inference Server", section "The engine"), one batched decode per tick
 * (page "Inference Server -- Architecture Map", section "How a single
 * request flows through the system").
 *
 * pkv_decode_graph_create takes paged_attn_decode_append's arguments, minus
 * the workspace and stream, for a bucket of num_seqs >= 1 rows.  Every
 * pointer is bound into the graph: the caller keeps those buffers alive and
 * in place until pkv_decode_graph_destroy, and before each launch writes the
 * tick's q, k_new, v_new, block_tables and context_lens into them (rows the
 * tick does not use: context_lens 0; they append nothing and output 0).
 * max_context_len bounds every length of every tick.  The graph owns its
 * decode workspace (allocated and zero-filled here, freed by destroy), so
 * create allocates device memory and synchronises; launch does neither.
 * Launches of one graph must not overlap (they share its workspace and
 * buffers): launch on one stream, or order them.
 *
 * create: *graph = the new graph, or NULL on error (errors as
 * paged_attn_decode_append, PKV_EHIP for a failed allocation or capture).
 * launch: enqueues one replay on `stream`.  destroy: NULL is a no-op.
 */
typedef struct pkv_decode_graph pkv_decode_graph;
int pkv_decode_graph_create(pkv_decode_graph** graph, void* out, float* lse, const void* q,
                            const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                            int32_t num_blocks, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                            int32_t gqa_group, int32_t head_dim, int32_t block_size, float scale,
                            float softcap, int32_t window, int32_t partition_size, int32_t dtype);
int pkv_decode_graph_launch(pkv_decode_graph* graph, struct ihipStream_t* stream);
void pkv_decode_graph_destroy(pkv_decode_graph* graph);

/*
 * paged_attn_prefill -- causal attention of a chunk of new tokens over the
 * cached prefix plus the chunk (chunked / batched prefill, page "Inference
 * Server", section "The engine", where the prefill kernels also read K/V
 * through the block tables).  The chunk's K/V must already be in the pool
 * (paged_kv_append); prefix blocks may be shared between sequences.
 *
 *   out           [num_q_tokens, num_q_heads, head_dim]
 *   lse           optional fp32 [num_q_tokens, num_q_heads] (NULL: not written)
 *   q             [num_q_tokens, num_q_heads, head_dim]; rows of sequence b
 *                 are cu_q_lens[b] .. cu_q_lens[b+1]-1
 *   cu_q_lens     int32 [num_seqs + 1], non-decreasing, cu_q_lens[0] = 0,
 *                 cu_q_lens[num_seqs] = num_q_tokens
 *   max_q_len     >= every n_b = cu_q_lens[b+1] - cu_q_lens[b]
 *   context_lens  int32 [num_seqs], L_b >= n_b; query row j of sequence b
 *                 sits at position L_b - n_b + j and sees keys t <= position
 *                 (rows at negative positions, L_b < n_b, a caller error,
 *                 see no key: out = 0 and lse = -inf)
 *   gqa_group     1, 2, 4, 8 or 16
 */
int paged_attn_prefill(void* out, float* lse, const void* q, const int32_t* cu_q_lens,
                       int32_t num_q_tokens, int32_t max_q_len, const void* k_pool,
                       const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                       int32_t gqa_group, int32_t head_dim, int32_t block_size, float scale,
                       float softcap, int32_t window, int32_t dtype, struct ihipStream_t* stream);

/*
 * paged_attn_mixed -- one call for a batch that mixes prefill chunks with
 * decode rows: the engine interleaves chunked prefill with the decode of the
 * other active requests, tick by tick (page "Inference Server -- Architecture
 * Map", section "How a single request flows through the system").
 *
 * Sequences [0, num_prefill_seqs) are chunks: their rows are
 * cu_q_lens[b] .. cu_q_lens[b+1]-1 of q / out (cu_q_lens has
 * num_prefill_seqs + 1 entries, the last = num_prefill_tokens), as in
 * paged_attn_prefill.  Sequences [num_prefill_seqs, num_seqs) are decode
 * rows: one query each, rows num_prefill_tokens + (b - num_prefill_seqs).
 * block_tables / context_lens cover all num_seqs sequences in that order.
 * The result is that of paged_attn_prefill over the whole batch (a decode row
 * is a one-row chunk), but the chunks run through the matrix-core prefill and
 * the decode rows through the balanced decode split, which spreads a long row
 * over several compute units.  For bf16 with both parts present this is one
 * launch on `stream`: the chunks' workgroups first in the grid, the decode
 * rows' after them, sized to the compute units the chunks leave free; fp32,
 * or a batch with only one part, runs that part's own kernel.
 *   out, q, lse   [num_prefill_tokens + num_seqs - num_prefill_seqs, Hq, D]
 *   workspace     >= paged_attn_decode_workspace_size(num_seqs -
 *                 num_prefill_seqs, ..., 0) bytes when there are decode rows
 * Errors as paged_attn_prefill and paged_attn_decode; PKV_EINVAL for counts
 * that do not fit.
 */
int paged_attn_mixed(void* out, float* lse, const void* q, const int32_t* cu_q_lens,
                     int32_t num_prefill_seqs, int32_t num_prefill_tokens, int32_t max_q_len,
                     const void* k_pool, const void* v_pool, int32_t num_blocks,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                     int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                     int32_t block_size, float scale, float softcap, int32_t window,
                     void* workspace, size_t workspace_bytes, int32_t dtype,
                     struct ihipStream_t* stream);

/*
 * pkv_hbm_read_probe -- a measurement aid, not part of the attention path: a
 * plain read of `bytes` (a multiple of 16) at device pointer `buf` by
 * `num_wgs` workgroups of 256 lanes (16-byte loads, four in flight per lane),
 * each writing one folded word to device array out [num_wgs].  Timed around
 * a buffer larger than the 256 MB Infinity Cache, it gives the HBM read rate
 * a kernel reaches on this GPU, the practical ceiling of the bandwidth-bound
 * decode (which the page "Inference Server", section "The engine", runs
 * over the block-paged cache every tick).  bytes == 0 is a no-op.
 */
int pkv_hbm_read_probe(const void* buf, size_t bytes, uint32_t* out, int32_t num_wgs,
                       struct ihipStream_t* stream);

/*
 * pkv_hbm_gather_probe -- a measurement aid beside pkv_hbm_read_probe: a read
 * of whole blocks in a given order, block order[i] of each of two device
 * buffers k and v (block_bytes each, a multiple of 4096), the access pattern
 * of the decode over a shuffled block pool (a block's K tile and V tile,
 * blocks scattered over the pool); num_blocks is the buffers' block count,
 * and an order entry outside [0, num_blocks) reads block 0.  num_wgs workgroups of 256 lanes each take a contiguous
 * range of the order, two blocks in flight, and write one folded word to
 * out [num_wgs].  n == 0 is a no-op.
 */
int pkv_hbm_gather_probe(const void* k, const void* v, size_t block_bytes, int32_t num_blocks,
                         const int32_t* order, int32_t n, uint32_t* out, int32_t num_wgs,
                         struct ihipStream_t* stream);

/*
 * pkv_mfma_rate_probe -- a measurement aid beside the prefill: num_wgs
 * workgroups of four waves (one per SIMD when num_wgs equals the CU count)
 * each run iters x 8 back-to-back bf16 32x32x16 matrix-core products (32768
 * flops per product per wave) with no memory access, and lane 0 writes four
 * counters to stamps[4 w .. 4 w + 3] (caller-owned device memory, 8-byte
 * aligned): the shader-clock counter before and after the loop, then the
 * constant-rate (100 MHz) counter before and after.  From them: cycles per
 * product, the clock the SIMDs ran at, and the sustained product rate.
 * PKV_EINVAL for a null or misaligned buffer, iters outside [1, 2^24] or
 * num_wgs outside [1, 2^20].
 */
int pkv_mfma_rate_probe(unsigned long long* stamps, int32_t iters, int32_t num_wgs,
                        struct ihipStream_t* stream);

/* Message describing the calling thread's last failed call ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
