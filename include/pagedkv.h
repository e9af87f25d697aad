/*
 * pagedkv.h — C ABI of a gfx950 (MI355X) library for attention over a paged
 * KV cache: storing new K/V into cache blocks, decode attention (one query
 * token per sequence, split-K with the partials merged in the same launch,
 * optional sliding window)
 * and variable-length causal prefill over a partly cached prefix.
 *
 * Sources.  nano-vllm-rs README, "Run Inference" (the KV-cache block size is a
 * user knob) and "GGUF Models" (the cache is paged); lunaryes/nano-vllm
 * diagram, "Components" and "Connections" (a KV block manager allocates cached
 * blocks; the model runner sets an execution context that the layers read);
 * nano-vllm-sansho README, "Key Features" (prefix caching) and "Sansho Serving
 * Roofline Anchors" (q=1 decode; a sliding-window-256 model).  The pages do
 * not write the attention formula; the library computes textbook scaled-dot-
 * product softmax attention, described with each call below.
 *
 * Conventions for every call
 *  - Tensors are device pointers to contiguous row-major arrays.  bf16 is the
 *    IEEE bfloat16 bit layout; index arrays are int32.
 *  - KV cache layout: [num_blocks, block_size, num_kv_heads, head_dim] bf16.
 *    A slot s is row (s % block_size) of block (s / block_size).
 *  - Logical position j of sequence b lives in slot
 *      block_tables[b * max_blocks_per_seq + j / block_size] * block_size
 *        + j % block_size.
 *  - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *  - Supported shapes: head_dim == 128; num_q_heads / num_kv_heads in
 *    {1, 2, 4, 8}; block_size a multiple of 16 in [16, 1024].
 *  - The caller owns every buffer.  The library allocates and frees no device
 *    memory.  Workspace, where needed, is caller-provided after a size query.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *    default stream) and returns; results are visible to later work on the
 *    same stream.  Calls are thread-safe.
 *  - Host-side argument checks never touch device memory.  A non-OK status
 *    means nothing was launched; pk_last_error_message() then describes the
 *    problem (thread-local).  No C++ exception crosses this ABI.
 *  - Indices read from device memory (slots, block-table entries) are
 *    bounds-checked in the kernels: an out-of-range slot is not stored and an
 *    out-of-range block-table entry contributes no keys, so a bad table can
 *    give a wrong answer but never an out-of-bounds access.
 *  - `out` must not alias any input; `key`/`value` must not alias the caches.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pk_status {
  PK_OK = 0,
  PK_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent sizes */
  PK_ERR_UNSUPPORTED = 2,   /* a shape the library does not implement          */
  PK_ERR_WORKSPACE = 3,     /* decode workspace missing or too small           */
  PK_ERR_LAUNCH = 4,        /* the HIP runtime rejected a kernel launch        */
  PK_ERR_INDEX = 5          /* checked mode: index arrays violate a contract   */
} pk_status;

/* Library version string, e.g. "pagedkv 0.1.0 gfx950". */
const char* pk_version(void);
/* Name of a status code; never NULL. */
const char* pk_status_string(pk_status s);
/* Detail for the last non-OK status returned on this thread ("" if none). */
const char* pk_last_error_message(void);

/*
 * pk_kv_store — store the K/V rows of new tokens into the paged cache.
 * (the slot_mapping scatter: each new token's K/V go to the slot the block
 * manager gave it; nano-vllm-rs README "GGUF Models", lunaryes/nano-vllm
 * "Connections": the scheduler's block manager allocates cached blocks.)
 *
 *   key, value    bf16 [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping  int32 [num_tokens]; slot of token i, or -1 to skip token i
 *                 (padding).  Slots >= num_blocks * block_size are skipped too.
 *                 Valid slots must be distinct (otherwise which write lands is
 *                 unspecified).
 *   k_cache, v_cache  bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *
 * The copy is bit-exact.  num_tokens == 0 is a no-op.
 */
pk_status pk_kv_store(const void* key, const void* value,
                      const int32_t* slot_mapping, int32_t num_tokens,
                      void* k_cache, void* v_cache,
                      int32_t num_blocks, int32_t block_size,
                      int32_t num_kv_heads, int32_t head_dim, void* stream);

/*
 * Decode split planning.  Decode work for one (sequence, KV head) is cut into
 * partitions of `partition_size` tokens (a multiple of 64) starting at its
 * first admitted key (with a sliding window W: ceil(min(L, W) / partition_size)
 * partitions); each partition is
 * reduced by one workgroup to a partial softmax state, and the partials are
 * merged (split-K / flash-decoding).  The merge happens in the same launch:
 * each (sequence, KV head) counts its finished partitions on a device-scope
 * counter, and the partition that finishes last merges them.  The counters
 * come from a pool of 2^20 that the library holds on every GPU it runs on
 * (zero when the library loads; every merge leaves its counter at zero); each
 * split call takes the next num_seqs * num_kv_heads of them when it is made
 * (wrapping at the end of the pool; a call captured into a graph keeps its
 * counters for every replay).  Two launches that may run at the same time on
 * one GPU therefore use distinct counters unless 2^20 or more pairs' worth of
 * split calls were made between them, e.g. a graph replayed on one stream
 * while that many calls went through another.  The first split call on a
 * device looks up the pool's device address (hipGetSymbolAddress): make one
 * call per device before capturing a graph.  When the stream's device is not
 * the current one, or a
 * call has more pairs than the pool, a second (combine) launch merges instead,
 * with the same arithmetic.  When every sequence fits one partition the
 * partition kernel writes the output directly.
 *
 * pk_paged_decode_plan: the partition size and the number of partition slots
 * per sequence that pk_paged_decode will use for these arguments.
 * `partition_size_request` 0 asks for the built-in choice; otherwise it must
 * be a positive multiple of 64, at most 2^30 (PK_ERR_INVALID_ARG otherwise).
 * The built-in choice is a power of two from 64 to 2^30.
 */
pk_status pk_paged_decode_plan(int32_t num_seqs, int32_t num_kv_heads,
                               int32_t max_context_len, int32_t sliding_window,
                               int32_t partition_size_request,
                               int32_t* partition_size_out,
                               int32_t* num_partitions_out);

/* Workspace bytes pk_paged_decode needs for the same arguments (0 when the
 * plan has a single partition), or 0 with the status set if the arguments are
 * invalid. */
size_t pk_paged_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len,
                                      int32_t sliding_window,
                                      int32_t partition_size_request);

/*
 * pk_paged_decode — attention for one query token per sequence over the
 * paged cache (the q=1 decode step; nano-vllm-sansho README "Sansho Serving
 * Roofline Anchors"), with an optional sliding window (its SWA-256 model).
 *
 *   out           bf16 [num_seqs, num_q_heads, head_dim]
 *   q             bf16 [num_seqs, num_q_heads, head_dim]
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; only the entries of
 *                 a sequence's admitted range address cache rows.  Other
 *                 entries of the row may be read (e.g. ahead of the length),
 *                 but their values are never used as block ids, so they may
 *                 hold anything (padding such as -1 or INT32_MAX)
 *   context_lens  int32 [num_seqs]; L_b keys, including the new token, which
 *                 is the query (it must already be stored, e.g. by
 *                 pk_kv_store earlier on the same stream).  Values are clamped
 *                 to [0, max_blocks_per_seq * block_size]; a table row may
 *                 address at most 2^31 - 1 tokens (PK_ERR_UNSUPPORTED
 *                 otherwise).
 *   num_seqs      at most 65535 per call (PK_ERR_UNSUPPORTED otherwise)
 *   max_context_len  host-side upper bound of context_lens, used to plan the
 *                 split; keys of a sequence beyond it are not attended.
 *   scale         softmax scale applied to q.k (1/sqrt(head_dim) usually)
 *   sliding_window  0: attend keys 0..L-1; W > 0: keys max(0, L-W)..L-1
 *   workspace     fp32 scratch of at least pk_paged_decode_workspace_size()
 *                 bytes (may be NULL when that size is 0); its contents are
 *                 dead after the call's kernels finish
 *
 * out[b, h] = sum_j softmax_j(scale * q[b,h] . K_j) V_j over the admitted j,
 * computed with fp32 accumulation and rounded to bf16 (nearest even).  A
 * sequence with L_b == 0 gets a zero row.
 */
pk_status pk_paged_decode(void* out, const void* q,
                          const void* k_cache, const void* v_cache,
                          int32_t num_blocks, int32_t block_size,
                          int32_t num_kv_heads, int32_t head_dim,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t max_context_len,
                          float scale, int32_t sliding_window,
                          int32_t partition_size_request,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * pk_paged_decode_noalloc — pk_paged_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It allocates nothing (no hipMalloc, no hipFree, no
 * allocating library call) and takes no workspace: the split-K partials go to
 * a static device array of PK_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.
 *   - Arguments, results and errors as pk_paged_decode, without the workspace.
 *     The output is bit-identical to pk_paged_decode's.
 *   - A plan whose partials exceed PK_NOALLOC_SCRATCH_BYTES (what
 *     pk_paged_decode_workspace_size reports for the same arguments) returns
 *     PK_ERR_WORKSPACE and launches nothing; a single-partition plan needs no
 *     scratch at all.
 *   - The device that is current on the calling thread must be the stream's
 *     device (PK_ERR_INVALID_ARG otherwise).  The first call on a device looks
 *     up the array's device address (hipGetSymbolAddress); make one call per
 *     device before capturing a graph.
 *   - Every call on a GPU shares that GPU's array, and the array keeps the
 *     last call's contents (nothing in it needs clearing: every partial is
 *     written before it is read).  Calls whose kernels overlap on one GPU
 *     (different streams without ordering between them) race on the array:
 *     order them, e.g. issue them on one stream.
 */
#define PK_NOALLOC_SCRATCH_BYTES (8u << 20)
pk_status pk_paged_decode_noalloc(void* out, const void* q,
                                  const void* k_cache, const void* v_cache,
                                  int32_t num_blocks, int32_t block_size,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len,
                                  float scale, int32_t sliding_window,
                                  int32_t partition_size_request, void* stream);

/*
 * pk_paged_decode_store — the decode step's store and attention in one
 * launch: for every sequence b with L_b = context_lens[b] > 0, the new token's
 * K/V rows k_new[b], v_new[b] (bf16 [num_seqs, num_kv_heads, head_dim]) are
 * written to the cache slot of position L_b - 1 (found through block_tables,
 * as the block manager allocated it), and attention is computed exactly as
 * pk_paged_decode over positions lo..L_b-1 with position L_b - 1 taken from
 * k_new / v_new.  Results and caches are bit-identical to pk_kv_store with
 * slot_mapping[b] = slot of position L_b - 1 followed by pk_paged_decode.
 * L_b is the caller's context length, not clamped: when L_b exceeds
 * max_context_len, the row is still stored at position L_b - 1 (if the table
 * has an entry for it) but attention covers only the clamped range, as it
 * would after pk_kv_store; when L_b - 1 lies beyond the table row, nothing is
 * stored (no slot exists for it).
 * (The fused kernel the nano-vllm-sansho README names as an optimization
 * target, "Sansho Serving Roofline Anchors".)  Other arguments, workspace
 * sizing and errors as pk_paged_decode.  A block-table entry outside the cache
 * for position L_b - 1 means nothing is stored for that sequence.
 */
pk_status pk_paged_decode_store(void* out, const void* q,
                                const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache,
                                int32_t num_blocks, int32_t block_size,
                                int32_t num_kv_heads, int32_t head_dim,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_context_len,
                                float scale, int32_t sliding_window,
                                int32_t partition_size_request,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * pk_paged_prefill — variable-length causal attention for the new tokens of
 * several sequences whose prefix may already be cached (prefix caching:
 * nano-vllm-sansho README "Key Features"; prefill and decode as separate
 * phases: lunaryes/nano-vllm introduction).
 *
 *   out           bf16 [total_q, num_q_heads, head_dim]
 *   q             bf16 [total_q, num_q_heads, head_dim]; sequence b owns rows
 *                 cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   cu_seqlens_q  int32 [num_seqs + 1], non-decreasing, cu_seqlens_q[0] == 0,
 *                 cu_seqlens_q[num_seqs] == total_q
 *   cu_seqlens_k  int32 [num_seqs + 1]; Lk_b = cu_seqlens_k[b+1] -
 *                 cu_seqlens_k[b] keys of sequence b are in the cache (prefix
 *                 and new tokens; store the new ones first with pk_kv_store)
 *   max_seqlen_q  host-side upper bound of the per-sequence query counts;
 *                 queries beyond it are not computed
 *   max_blocks_per_seq  at most 2048 (the touched table entries are staged
 *                 on chip); larger values return PK_ERR_UNSUPPORTED
 *   scale, sliding_window  as for decode
 *
 * With prefix P_b = Lk_b - Lq_b, new query i of sequence b sits at position
 * P_b + i and attends keys j <= P_b + i (and P_b + i - j < W when W > 0).
 * Sequences with Lk_b < Lq_b are invalid; their rows are left unwritten.
 */
pk_status pk_paged_prefill(void* out, const void* q,
                           const void* k_cache, const void* v_cache,
                           int32_t num_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                           int32_t num_q_heads, float scale, int32_t sliding_window,
                           void* stream);

/* A mixed batch (chunked prefill: decode sequences and prefill chunks in one
 * step, the step bounded by a token budget: nano-vllm-rs README, "Run
 * Inference"; "How lunaryes/nano-vllm works", introduction) split by kind:
 * the first num_decode_seqs sequences each have exactly one new token and
 * run on the decode kernel (their K/V stream at decode's rate); the others
 * run on the varlen prefill kernel.  Same result as pk_paged_prefill over the
 * whole batch, within the attention tolerance (a different kernel's fp32
 * summation order for the decode rows).
 *   num_decode_seqs  leading sequences with one new token each (query row
 *                    cu_seqlens_q[b]); a leading sequence with another count
 *                    is left unwritten
 *   max_seqlen_q     upper bound of the prefill sequences' query counts
 *   max_decode_context_len  upper bound of the decode sequences' lengths
 *                    (cu_seqlens_k differences); plans the decode split
 *   workspace        as pk_paged_decode, sized by
 *                    pk_paged_decode_workspace_size(num_decode_seqs, ...,
 *                    max_decode_context_len, sliding_window, 0)
 * One launch on `stream` when the shapes allow it: its workgroups are the
 * prefill's heaviest query tiles, then the decode rows, then the rest of the
 * prefill, so the decode rows stream while the long prefill chains compute.
 * That needs a power-of-two block_size >= 32, one decode partition per
 * sequence, at most 4 query heads per KV head and both kinds present.  Otherwise it makes two launches (decode
 * rows, then the prefill).  Either way each row's result is bit-identical to
 * the separate kernels.  Other arguments and errors as pk_paged_prefill;
 * every argument is checked before any launch. */
pk_status pk_paged_prefill_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  int32_t num_blocks, int32_t block_size,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t num_seqs, int32_t num_decode_seqs, int32_t total_q,
                                  int32_t max_seqlen_q, int32_t max_decode_context_len,
                                  int32_t num_q_heads, float scale, int32_t sliding_window,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Prefill with the new tokens' store fused in: the same result as
 * pk_kv_store of key/value at the slots of positions P_b .. P_b+Lq_b-1 of
 * each sequence (slot_mapping derived from block_tables) followed by
 * pk_paged_prefill, bit for bit, in one launch (the pages name kernel fusion
 * as the lever past graph replay: nano-vllm-sansho README, "Sansho Serving
 * Roofline Anchors").  The new keys are read from key/value directly.
 *   key, value  bf16 [total_q, num_kv_heads, head_dim]: row r is the new
 *               token of query row r (same layout as q's rows)
 *   k_cache, v_cache  read for the prefix, written at the new positions
 * A position whose block-table entry lies outside the table or the cache is
 * not stored (as pk_kv_store skips such a slot).  Queries beyond
 * max_seqlen_q are neither computed nor stored.  key/value must not alias
 * the caches or out.  Other arguments and errors as pk_paged_prefill. */
pk_status pk_paged_prefill_store(void* out, const void* q, const void* key, const void* value,
                                 void* k_cache, void* v_cache,
                                 int32_t num_blocks, int32_t block_size,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                 int32_t num_q_heads, float scale, int32_t sliding_window,
                                 void* stream);

/* ------------------------------------------------------------------------
 * Checked mode.  The attention and store calls trust their index arrays (they
 * bounds-check every access, so a bad index never touches memory outside the
 * caches, but it changes the answer: a key with a bad block contributes
 * nothing, a slot out of range is not stored, duplicate slots race).  This
 * call validates them on the device, for debugging and tests, and writes
 * violation counts to `counts` (device memory, 4 x int32, caller-owned):
 *   counts[0]  slot_mapping entries outside [-1, num_blocks * block_size)
 *   counts[1]  repeated slots (each occurrence of a slot >= 0 after its first)
 *   counts[2]  block-table entries outside [0, num_blocks) in a sequence's
 *              used range (entries past ceil(L / block_size) are not read)
 *   counts[3]  sequences whose length is below 0 or beyond
 *              max_blocks_per_seq * block_size, or (with cu_seqlens) whose
 *              prefix sums decrease or have fewer keys than new queries
 * Any of slot_mapping (num_tokens = 0) and the sequence arrays (num_seqs = 0)
 * may be absent; lengths come from cu_seqlens_k when given, else from
 * context_lens.  workspace: pk_check_indices_workspace_size bytes (a bitmap
 * of the cache slots), cleared by the call itself (no memset).  Enqueued on
 * `stream` like every call; read `counts` after synchronising.  The Python
 * binding raises PK_ERR_INDEX when a count is not zero. */
size_t pk_check_indices_workspace_size(int32_t num_blocks, int32_t block_size);
pk_status pk_check_indices(const int32_t* slot_mapping, int32_t num_tokens,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_seqs, const int32_t* context_lens,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t num_blocks, int32_t block_size, int32_t* counts,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Host-side KV block manager (no GPU work).
 *
 * Hands out the cache blocks that the calls above address through
 * block_tables and slot_mapping, and reuses the full blocks of a prompt whose
 * K/V were computed before (lunaryes/nano-vllm diagram, "Components" and
 * "Connections": the scheduler asks a KV block manager for cached blocks;
 * nano-vllm-sansho README, "Key Features": prefix caching).  The pages fix no
 * policy; this one is:
 *  - a full block is identified by a 64-bit chain hash of the previous
 *    block's hash and its own block_size token ids, and a hit also compares
 *    its token ids, so a block is shared only when its own tokens are equal
 *    and the prefix before it has the same chain hash;
 *  - a new sequence reuses the longest leading run of cached full blocks and
 *    always computes at least one token (a prompt cached in full recomputes
 *    its last block into a new block);
 *  - reference counts track how many sequences hold a block; a block nobody
 *    holds stays cached until its space is handed out again, least recently
 *    freed first;
 *  - only full blocks are shared, so every slot a call writes belongs to one
 *    sequence;
 *  - a block that becomes full (at pk_bm_allocate or pk_bm_append) is pending
 *    until the next pk_bm_commit and is not found by pk_bm_allocate before
 *    then.  Its K/V are written by the step the caller runs next, so no batch
 *    is ever handed a cached prefix block that the same batch writes: every
 *    call, pk_paged_prefill_store and pk_paged_decode_store included, reads
 *    only prefix rows stored by an earlier, already enqueued step.
 * Typical step: allocate / append / free, pk_bm_prepare, enqueue the step's
 * store and attention calls, then pk_bm_commit.
 * A manager is not thread-safe: one thread (the scheduler) owns it.  Errors
 * return a non-OK status, set pk_last_error_message(), and leave the manager
 * unchanged; PK_ERR_WORKSPACE means the free blocks do not suffice.
 * ---------------------------------------------------------------------- */
typedef struct pk_block_manager pk_block_manager;

/* A manager of blocks 0 .. num_blocks-1 of block_size slots each, all free.
 * num_blocks * block_size must fit an int32 slot index.  *out receives the
 * handle (NULL on error); release it with pk_bm_destroy. */
pk_status pk_bm_create(int32_t num_blocks, int32_t block_size, pk_block_manager** out);
void pk_bm_destroy(pk_block_manager* m);

/* Blocks that no sequence holds (cached or empty). */
pk_status pk_bm_num_free_blocks(const pk_block_manager* m, int32_t* out);

/* How many sequences hold `block`, and whether its content is registered
 * (committed, so findable by prefix hash; a pending block reports 0). */
pk_status pk_bm_block_info(const pk_block_manager* m, int32_t block, int32_t* ref_count,
                           int32_t* cached);

/* Admit sequence `seq_id` (unused so far) with its prompt tokens[0..n) (host
 * memory, n >= 1).  *num_cached_tokens receives how many leading tokens reuse
 * committed blocks (a multiple of block_size, < n): only tokens from there on
 * need K/V computed and stored.  The prompt's other full blocks are pending
 * until the next pk_bm_commit. */
pk_status pk_bm_allocate(pk_block_manager* m, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens, int32_t* num_cached_tokens);

/* Append one generated token to `seq_id`; takes a new block when the token
 * opens one, and a block that it fills becomes pending. */
pk_status pk_bm_append(pk_block_manager* m, int64_t seq_id, int32_t token);

/* Make every pending block findable by later pk_bm_allocate calls.  Call it
 * once the step that stores those blocks' K/V has been enqueued (on the stream
 * that later attention calls use).  A pending block whose sequence was freed
 * in the meantime is dropped, not registered.  *num_registered (may be NULL)
 * receives how many blocks became findable. */
pk_status pk_bm_commit(pk_block_manager* m, int32_t* num_registered);

/* Drop `seq_id` and its block references (last block first). */
pk_status pk_bm_free(pk_block_manager* m, int64_t seq_id);

/* Tokens, blocks and cached leading tokens of `seq_id` (NULL outputs skipped). */
pk_status pk_bm_seq_info(const pk_block_manager* m, int64_t seq_id, int32_t* num_tokens,
                         int32_t* num_blocks, int32_t* num_cached_tokens);

/* Fill the host arrays one attention call of the sequences seq_ids[0..B)
 * needs, where the last num_new[b] tokens of sequence b are the new queries
 * (0 <= num_new[b] <= its length):
 *   block_tables  [B, max_blocks_per_seq] block ids, rows padded with -1
 *   cu_seqlens_q  [B + 1] prefix sums of num_new
 *   cu_seqlens_k  [B + 1] prefix sums of the sequence lengths
 *   slot_mapping  [cu_seqlens_q[B]] cache slot of each new token, in order
 *                 (may be NULL when there are no new tokens)
 * A decode step uses num_new = 1 (context length = cu_seqlens_k difference). */
pk_status pk_bm_prepare(const pk_block_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                        const int32_t* num_new, int32_t max_blocks_per_seq,
                        int32_t* block_tables, int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                        int32_t* slot_mapping);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
