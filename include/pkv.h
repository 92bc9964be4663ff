/*
 * pkv.h -- C ABI of the paged KV-cache attention library (libpkv.so).
 *
 * The method: a request's keys and values are logically contiguous but stored
 * in fixed 16-token blocks scattered through one preallocated pool, and a
 * block table maps each logical block to a physical one
 * ["(2) vLLM Internals: From PagedAttention to Removing PagedAttention",
 * section 1.1 "The Analogy"; "My Understanding of vLLM and PagedAttention",
 * sections "1. Logical Blocks", "2. Physical Blocks", "3. Block Table"].
 * The worker keeps the table as a dense int32 tensor
 * [rows, max_blocks_per_row] and the new tokens' destinations as an int64 slot
 * mapping, both indexed by the kernels themselves ["vLLM: what PagedAttention
 * turned into", section "The problem PagedAttention was actually solving"];
 * the attention kernels gather the paged KV inside the kernel ["(2) vLLM
 * Internals ...", section 4.1 "Why It Could Go"].
 *
 * Conventions
 *  - Every function returns an int: PKV_OK (0) or a negative PKV_ERR_* code.
 *    pkv_last_error() then holds a message (per thread).
 *  - Block size is fixed at PKV_BLOCK_SIZE = 16 tokens.
 *  - Pool layout (one tensor for K, one for V, row-major, contiguous):
 *        [num_blocks][num_kv_heads][16][head_dim]
 *    Token position p of a sequence whose logical block p/16 is physical
 *    block b lives at slot b*16 + p%16, i.e. at [b][h][p%16][:] for head h.
 *  - Block 0 is the null block: never handed out, used as table padding.
 *  - Device entry points only enqueue work on the given stream (a hipStream_t,
 *    NULL = the null stream); they never synchronise with the host and
 *    allocate no device memory, so they may be captured in a HIP graph.
 *    Arguments are checked on the host before any launch; a rejected call
 *    enqueues nothing. Device-resident values (slots, block ids, context
 *    lengths) are range-checked inside the kernels: out-of-range entries are
 *    skipped or clamped as documented per call, never dereferenced.
 *  - Ownership: the caller owns every buffer (pools, queries, outputs, tables,
 *    slot mappings, workspaces) and the stream. The library keeps no device
 *    pointer past a call. An allocator handle is host-only, owned by the
 *    caller and not thread-safe (callers serialise access to one handle).
 *  - dtype: PKV_F32 (float32) or PKV_BF16 (bfloat16, raw 16-bit storage);
 *    head_dim 64 or 128; num_q_heads a multiple of num_kv_heads with at most
 *    16 query heads per KV head.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 16

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,   /* a null pointer, a negative size, a bad id  */
  PKV_ERR_UNSUPPORTED = -2,   /* dtype / head_dim / group size not built    */
  PKV_ERR_OUT_OF_BLOCKS = -3, /* the pool cannot satisfy the request        */
  PKV_ERR_NO_SUCH_SEQ = -4,   /* an unknown sequence id                     */
  PKV_ERR_SEQ_EXISTS = -5,    /* a sequence id already in use               */
  PKV_ERR_WORKSPACE = -6,     /* workspace missing or smaller than required */
  PKV_ERR_HIP = -7            /* the HIP runtime reported an error          */
};

enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1 };

/* Message for the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);
/* Fixed description of a status code. */
const char* pkv_strerror(int code);
/* Library version, major*10000 + minor*100 + patch. */
int pkv_version(void);

/* Debug checks (off by default; on when PKV_DEBUG_CHECKS=1 is set in the
 * environment when the library is first used, or after
 * pkv_set_debug_checks(1)). With them on, pkv_reshape_and_cache waits for
 * its stream, reads the slot mapping back and refuses (PKV_ERR_INVALID_ARG,
 * nothing launched) a mapping that pkv_check_slot_mapping rejects. They
 * synchronise with the host: not for graph capture or timed runs.
 * Process-wide. */
int pkv_set_debug_checks(int32_t enabled);
/* Host check of a slot mapping held in host memory, the one the debug mode
 * of pkv_reshape_and_cache applies: every token's new K/V has one slot of its
 * own ["vLLM: what PagedAttention turned into", section "The problem
 * PagedAttention was actually solving"], so PKV_ERR_INVALID_ARG (the message
 * names the entry) for a non-negative slot that an earlier token of the same
 * call also has, a slot in the null block 0 (never a write target, section
 * "The block pool, and the two tricks in it") or one beyond
 * num_blocks*16. Negative slots (padding) pass. */
int pkv_check_slot_mapping(const int64_t* slot_mapping, int64_t num_tokens, int32_t num_blocks);

/* ------------------------------------------------------------------------ */
/* Host allocator: the KV-cache manager that allocates blocks, frees them and
 * maintains block tables ["My Understanding of vLLM and PagedAttention",
 * "vLLM System Architecture", item "2. KV-Cache Manager"]. Host memory only.
 *
 * Policy ["vLLM: what PagedAttention turned into", section "The block pool,
 * and the two tricks in it"]: the free queue starts as 0, 1, ..., NB-1 and
 * its first block, 0, is burned as the null block; allocation takes blocks
 * from the front; a sequence is released tail first and every block whose
 * refcount reaches zero goes back to the front in that order (so the tail is
 * reused first). Sequences share blocks by reference counting; appending to
 * a sequence whose last block is partially filled and shared first moves it
 * to a private copy and reports the (source, destination) pair for
 * pkv_copy_blocks ["(2) vLLM Internals ...", 1.2 "Three Direct Wins"].
 * Every call is all-or-nothing: on failure the allocator is unchanged.
 */
typedef struct pkv_allocator pkv_allocator;

typedef struct pkv_stats {
  int32_t num_seqs;        /* live sequences                                 */
  int32_t used_blocks;     /* blocks with refcount > 0                       */
  int32_t free_blocks;     /* blocks in the free queue                       */
  int32_t shared_blocks;   /* blocks with refcount > 1                       */
  int64_t logical_tokens;  /* sum of sequence lengths (shared tokens counted per sequence) */
  int64_t stored_tokens;   /* distinct token slots holding state             */
  double utilisation;      /* stored_tokens / (16 * used_blocks), 0 if none  */
} pkv_stats;

/* Create an allocator over num_blocks blocks (>= 2: block 0 is the null
 * block). *out receives the handle. */
int pkv_allocator_create(int32_t num_blocks, pkv_allocator** out);
/* Destroy a handle (NULL is accepted). */
int pkv_allocator_destroy(pkv_allocator* a);
/* Replace the free-queue order by order[0..n-1], which must be a permutation
 * of 1..num_blocks-1 (n = num_blocks-1); only while no sequence exists.
 * Used to place blocks at random physical positions. */
int pkv_allocator_set_free_order(pkv_allocator* a, const int32_t* order, int32_t n);
/* Random physical placement from a seed ["My Understanding of vLLM and
 * PagedAttention", section "2. Physical Blocks": a sequence's blocks need not
 * be contiguous]: installs as the free order the ids 1..num_blocks-1,
 * ascending, permuted by a Fisher-Yates shuffle (Durstenfeld's form: for i =
 * n-1 down to 1, swap entries i and r % (i+1)) whose draws r are successive
 * SplitMix64 outputs (Steele, Lea and Flood, OOPSLA 2014: a 64-bit counter
 * starting at seed, advanced by 0x9E3779B97F4A7C15 and mixed). Same
 * conditions and errors as pkv_allocator_set_free_order, which it calls. */
int pkv_allocator_shuffle_free_list(pkv_allocator* a, uint64_t seed);
/* Create an empty sequence. PKV_ERR_SEQ_EXISTS if the id is taken. */
int pkv_seq_add(pkv_allocator* a, int64_t seq_id);
/* Append n_tokens >= 0 tokens to one sequence. out_slots[n_tokens] receives
 * each new token's slot (int64, block*16 + offset). out_cow_pairs receives up
 * to max_pairs (source, destination) block pairs (2 int64 each) that the
 * caller must copy with pkv_copy_blocks before writing the new tokens;
 * *out_n_pairs their number (0 or 1 here). PKV_ERR_OUT_OF_BLOCKS if the pool
 * is too small; PKV_ERR_INVALID_ARG if max_pairs is too small. */
int pkv_seq_append(pkv_allocator* a, int64_t seq_id, int32_t n_tokens, int64_t* out_slots,
                   int64_t* out_cow_pairs, int32_t max_pairs, int32_t* out_n_pairs);
/* Batched append: n_tokens[i] tokens to seq_ids[i] for i < n_seqs (no
 * duplicates), in that order, all or nothing. Slots of all new tokens are
 * written back to back to out_slots (sum of n_tokens entries). */
int pkv_batch_append(pkv_allocator* a, const int64_t* seq_ids, const int32_t* n_tokens,
                     int32_t n_seqs, int64_t* out_slots, int64_t* out_cow_pairs,
                     int32_t max_pairs, int32_t* out_n_pairs);
/* Make child share every block of parent (refcount +1 each); child gets
 * parent's length. Used for shared prefixes and parallel sampling. */
int pkv_seq_fork(pkv_allocator* a, int64_t parent_id, int64_t child_id);
/* Release a sequence (tail first, see above). */
int pkv_seq_free(pkv_allocator* a, int64_t seq_id);
/* ---- Prefix caching (content-addressed blocks) ----
 * ["vLLM: what PagedAttention turned into", sections "The block pool, and the
 * two tricks in it" and "What a block hash actually is"]. A full block whose
 * token ids have been recorded gets a chained content hash (see
 * pkv_hash_block_tokens) and enters a hash -> block map, keyed by the hash
 * followed by the KV-cache group id (4 bytes big endian; one group, 0). If
 * another block already holds that key, the new block stays unhashed. A
 * freed block with a hash keeps it and goes to the back of the free queue
 * (FIFO: least recently freed is evicted first); it leaves the map only when
 * the queue hands it out again (lazy eviction). Freed blocks without a hash
 * go to the front (LIFO). Off by default. */
/* Switch prefix caching on (enabled != 0) or off; only while no sequence
 * exists. Either way the map is emptied. */
int pkv_allocator_enable_prefix_caching(pkv_allocator* a, int32_t enabled);
/* What pkv_seq_add_cached would attach for this prompt, without changing
 * anything: *out_cached_tokens (a multiple of 16) and *out_revived_blocks,
 * how many of those blocks are free now and would leave the free queue.
 * A scheduler uses it to check that a prompt fits before admitting it. */
int pkv_prefix_lookup(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens,
                      uint64_t extra_key, int32_t max_cached_tokens, int32_t* out_cached_tokens,
                      int32_t* out_revived_blocks);
/* Create a sequence for a prompt of n_tokens token ids and attach the
 * longest run of cached full blocks from its start (at most
 * max_cached_tokens tokens; < 0 means no limit), walking block by block and
 * stopping at the first miss (sound because the hashes chain). A cached block
 * that is free is taken back out of the free queue. *out_cached_tokens
 * (may be NULL) receives the number of tokens attached (a multiple of 16);
 * the sequence's length is that number and its first that many token ids are
 * recorded. extra_key is folded into the first block's hash only (a per-tenant
 * salt: different keys never share blocks). With caching off, the sequence
 * starts empty. */
int pkv_seq_add_cached(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                       uint64_t extra_key, int32_t max_cached_tokens, int32_t* out_cached_tokens);
/* Record the ids of the sequence's next n tokens (in order, within its
 * appended length; call once their K/V are written). Every block this
 * fills gets its chained hash and, with caching on, enters the map. */
int pkv_seq_record_tokens(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n);
/* The content hash of a block: out[32] and *has_hash (0: none, out zeroed). */
int pkv_block_hash(pkv_allocator* a, int32_t block, uint8_t* out, int32_t* has_hash);
/* Blocks in the hash map, prefix lookups made, and blocks they attached
 * (any pointer may be NULL). */
int pkv_prefix_cache_stats(pkv_allocator* a, int32_t* cached_blocks, int64_t* lookups,
                           int64_t* hit_blocks);
/* Chained block hash: SHA-256 of parent_hash (32 bytes; NULL for a first
 * block, which uses the fixed seed hash SHA-256("pkv none hash")), the 16
 * token ids as little-endian int32 and extra_key as little-endian uint64;
 * out[32]. */
int pkv_hash_block_tokens(const uint8_t* parent_hash, const int32_t* tokens, uint64_t extra_key,
                          uint8_t* out);
/* SHA-256 (FIPS 180-4) of n bytes into out[32]. */
int pkv_sha256(const void* data, size_t n, uint8_t* out);

/* Length of a sequence in tokens. */
int pkv_seq_len(pkv_allocator* a, int64_t seq_id, int64_t* out);
/* Dense block table for n sequences: table[n][max_blocks] (int32, row-major)
 * with unused entries set to the null block 0, and context_lens[n] (int32,
 * may be NULL). PKV_ERR_INVALID_ARG if a sequence needs more than max_blocks
 * blocks. Host buffers (e.g. pinned, then copied to the device). */
int pkv_fill_block_table(pkv_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* table,
                         int32_t max_blocks, int32_t* context_lens);
/* Refcount of one block (the null block reports 0). */
int pkv_block_refcount(pkv_allocator* a, int32_t block, int32_t* out);
/* Number of blocks in the free queue. */
int pkv_num_free_blocks(pkv_allocator* a, int32_t* out);
/* Pool accounting (see pkv_stats); utilisation is the share of in-use slots
 * that hold token state ["vLLM: what PagedAttention turned into", section
 * "Checking the 96.3%"]. */
int pkv_allocator_stats(pkv_allocator* a, pkv_stats* out);
/* How many blocks (null block included) fit in `bytes` of device memory for
 * K and V pools of the given shape: floor(bytes / (2*num_kv_heads*16*head_dim
 * *elem_size)). The engine sizes its pool once this way at start-up ["vLLM:
 * what PagedAttention turned into", section "Checking the 96.3%"]. */
int pkv_blocks_for_bytes(int64_t bytes, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         int32_t* out);

/* ------------------------------------------------------------------------ */
/* Step scheduler (host, C++) over an allocator.
 * Iteration-level scheduling with one token budget per step and no prefill
 * or decode phase: each request has the tokens it holds (prompt, then
 * generated tokens) and the count whose K/V are computed. A step walks the
 * running requests first, in admission order, giving each
 * min(tokens still to compute, budget left); then the waiting queue, each
 * admitted prompt getting the same share, capped by long_prefill_threshold
 * when it is > 0 (the cap applies to running requests too). A prompt cut by
 * the budget continues next step (chunked prefill); with chunked_prefill ==
 * 0 a prompt that does not fit stops the admission walk and waits
 * ["vLLM: what PagedAttention turned into", "The scheduler, and what it has
 * to balance now"; "(2) vLLM Internals ...", "2. Continuous Batching"].
 * When the pool cannot hold a running request's tokens, the request admitted
 * last is preempted: its blocks are freed, its computed count reset to 0 and
 * it goes to the front of the waiting queue (recompute); a step that
 * preempted admits no one ["vLLM: what PagedAttention turned into",
 * "Preemption, and the path that got deleted"]. At admission the prompt's
 * cached full blocks (prefix caching on the allocator) are attached and count
 * as computed, at most all tokens but one. A step that completes a request's
 * tokens samples one token (passed to pkv_scheduler_update), computed in a
 * later step; a request finishes with max_new_tokens generated tokens and
 * its blocks are freed. max_num_seqs > 0 bounds the running requests.
 * Each request owns the allocator sequence with its id; the caller must not
 * touch those sequences. The scheduler does not own the allocator, which
 * must outlive it. Not thread-safe. */
typedef struct pkv_scheduler pkv_scheduler;
int pkv_scheduler_create(pkv_allocator* alloc, int32_t token_budget, int32_t long_prefill_threshold,
                         int32_t chunked_prefill, int32_t max_num_seqs, pkv_scheduler** out);
int pkv_scheduler_destroy(pkv_scheduler* s);
/* Queue a request (prompt_len >= 1 token ids, copied). PKV_ERR_SEQ_EXISTS
 * if the id was used before; PKV_ERR_OUT_OF_BLOCKS (nothing queued) if its
 * prompt_len + max_new_tokens - 1 tokens need more blocks than the pool
 * holds, so that it could never finish. */
int pkv_scheduler_add_request(pkv_scheduler* s, int64_t req_id, const int32_t* prompt,
                              int32_t prompt_len, int32_t max_new_tokens, uint64_t extra_key);
/* Plan one step: sizes of the plan (outputs may be NULL). The allocator
 * already holds the planned positions' slots when this returns. Must be
 * followed by pkv_scheduler_update before the next call. */
int pkv_scheduler_schedule(pkv_scheduler* s, int32_t* out_num_scheduled, int64_t* out_num_tokens,
                           int32_t* out_num_preempted);
/* Copy the plan out (each pointer may be NULL): per scheduled request, in
 * plan order: id, first position computed this step, number of positions,
 * whether the step samples a token for it (1/0); the slots of all planned
 * positions in plan order (int64, out_num_tokens of them); the ids
 * preempted this step. A request's context after the step is
 * start + num_new tokens (its block table from pkv_fill_block_table). */
int pkv_scheduler_plan(pkv_scheduler* s, int64_t* req_ids, int32_t* start_pos, int32_t* num_new,
                       int32_t* samples, int64_t* slots, int64_t* preempted);
/* The planned step ran (its K/V are in the pool): record the token ids of
 * the computed positions (block hashes), advance the computed counts,
 * append sampled[k] to the k-th sampling request in plan order, and free the
 * requests that are now complete (*out_num_finished of them, ids from
 * pkv_scheduler_finished). */
int pkv_scheduler_update(pkv_scheduler* s, const int32_t* sampled, int32_t n_sampled,
                         int32_t* out_num_finished);
int pkv_scheduler_finished(pkv_scheduler* s, int64_t* req_ids);
/* Drop a request in any state: a waiting one leaves the queue, a running one
 * has its blocks freed (an abort), a finished one has its record (and token
 * ids) released; its id may then be used again. Refused while a plan is
 * pending. Finished requests are kept until removed, so that their tokens
 * can be read. */
int pkv_scheduler_remove_request(pkv_scheduler* s, int64_t req_id);
int pkv_scheduler_counts(pkv_scheduler* s, int32_t* num_waiting, int32_t* num_running);
/* One request: state (0 waiting, 1 running, 2 finished), tokens held,
 * computed count, times preempted, and (if tokens != NULL, max_tokens >=
 * num_tokens) its token ids. Each output may be NULL. */
int pkv_scheduler_request(pkv_scheduler* s, int64_t req_id, int32_t* state, int32_t* num_tokens,
                          int32_t* computed, int32_t* preemptions, int32_t* tokens,
                          int32_t max_tokens);

/* ------------------------------------------------------------------------ */
/* Device kernels (asynchronous on `stream`).
 * Index arrays (slot_mapping, pairs, block_table, context_lens, cu_q_lens)
 * may live in device memory or in pinned, mapped host memory (hipHostMalloc):
 * the kernels read them in place, so the host must leave them unchanged
 * until the call's kernels have finished on the stream. Every other pointer
 * is device memory. */

/* Scatter new tokens into the pools through the slot mapping ["vLLM: what
 * PagedAttention turned into", "The problem PagedAttention was actually
 * solving"; "My Understanding of vLLM and PagedAttention", "Step 3 -- Tokens
 * Generated Sequentially"]:
 *   k_cache[slot/16][h][slot%16][:] = k_new[t][h][:]   (and V alike)
 * for t < num_tokens. k_new/v_new: device [num_tokens][num_kv_heads][head_dim]
 * with a stride of new_token_stride elements between tokens (>= num_kv_heads
 * *head_dim; heads and dims contiguous). slot_mapping: device int64
 * [num_tokens]. A slot < 0 or >= num_blocks*16 is skipped (no write). Two
 * tokens with the same slot in one call race (caller error; refused in the
 * debug mode, see pkv_set_debug_checks). Bit-exact copy. */
int pkv_reshape_and_cache(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          int64_t new_token_stride, const int64_t* slot_mapping,
                          int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, int32_t dtype, void* stream);

/* Copy whole blocks, K and V: for each pair i < n, block pairs[2i+1] becomes a
 * copy of block pairs[2i] (copy-on-write of a shared block ["vLLM: what
 * PagedAttention turned into", section "What a block hash actually is"]).
 * pairs: device int64 [n][2]. Pairs with an id outside [0, num_blocks) are
 * skipped. Destinations must be distinct and must not be sources of other
 * pairs in the same call. */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t n,
                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                    void* stream);

/* Copy the per-step index arrays (slot mapping, context lengths, block table)
 * to the device with a kernel on `stream`: the table is rebuilt by the host
 * every step and mirrored to the device ["vLLM: what PagedAttention turned
 * into", section "The problem PagedAttention was actually solving"], and for
 * copies of this size a kernel starts sooner than the DMA engine. dst: device
 * memory; src: pinned host memory or device memory; both 16-byte aligned, not
 * overlapping; `bytes` may be any size. The host must leave src unchanged
 * until the copy has run. */
int pkv_stage_copy(void* dst, const void* src, size_t bytes, void* stream);
/* Measurement aid, not part of the attention path: a plain streaming read of
 * `bytes` of device memory at src (both multiples of 16) by `workgroups`
 * workgroups of 256 threads, each reading one contiguous slice with 16-byte
 * loads; workgroup b writes one word folded from its data to out[b] (device
 * memory, `workgroups` words), so the reads cannot be dropped. Timing it
 * gives the read bandwidth plain streaming reaches on the device, the
 * practical ceiling of the HBM-bound decode. */
int pkv_stream_read(const void* src, size_t bytes, uint32_t* out, int32_t workgroups, void* stream);

/* Workspace bytes pkv_paged_attention_decode needs for these sizes on the
 * current device (split-KV partial results and bookkeeping). The size does
 * not depend on context lengths. */
int pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, size_t* out);

/* Tuning: the split-KV decode runs a fixed number of single-wave workgroups,
 * per_cu per compute unit (default 3; 0 restores it), and splits the
 * sequences' blocks evenly over them, so this sets how the contexts are
 * partitioned. The result does not depend on it beyond rounding. It changes
 * the workspace size: size workspaces after setting it (a decode given a
 * workspace that is now too small fails with PKV_ERR_WORKSPACE). Process-wide,
 * not thread-safe; per_cu outside [0, 32] gives PKV_ERR_INVALID_ARG. */
int pkv_decode_set_waves_per_cu(int32_t per_cu);

/* Decode attention: one query token per sequence over its paged KV
 * ["My Understanding of vLLM and PagedAttention", "3. PagedAttention CUDA
 * Kernel" and "Step 4 -- Attention Computation"]:
 *   out[s][h] = sum_{t < n_s} softmax_t(scale * q[s][h] . K_s[t]) V_s[t],
 * K_s/V_s = sequence s's tokens in logical order for KV head
 * h / (num_q_heads/num_kv_heads); n_s = context_lens[s] counts every cached
 * token including the current one (write it with pkv_reshape_and_cache first).
 * n_s == 0 gives a zero output. n_s is clamped to [0, max_blocks_per_seq*16];
 * block ids outside [0, num_blocks) read block 0 instead.
 * q, out: device [num_seqs][num_q_heads][head_dim] in `dtype` (fp32
 * accumulation, output rounded to nearest even for bf16). block_table: device
 * int32 [num_seqs][max_blocks_per_seq]. context_lens: device int32 [num_seqs].
 * workspace: device, >= pkv_decode_workspace_size(...) bytes, no
 * initialisation needed; its contents are scratch. Calls that overlap in
 * time must not share a workspace.
 * Long contexts are split across waves (split-KV) and the partial softmax
 * states merged in token order by a second kernel, so the result is
 * deterministic and does not depend on the physical placement of blocks. */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float scale, int32_t dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* The two phases of pkv_paged_attention_decode, for callers that time or
 * interleave them: the split-KV kernel (writes whole sequences' outputs and
 * the partial states of split ones into the workspace), then the merge
 * kernel (folds the partial states in token order, writes the remaining
 * outputs). Called in that order on one stream with identical arguments and
 * workspace, they produce exactly what pkv_paged_attention_decode produces. */
int pkv_paged_attention_decode_split(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_blocks, int32_t max_blocks_per_seq,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float scale, int32_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream);
int pkv_paged_attention_decode_merge(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_blocks, int32_t max_blocks_per_seq,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float scale, int32_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* A decode step with the current token's cache write folded into the
 * split-KV kernel: the token's key and value are appended to each sequence's
 * paged KV and attended in the same pass ["My Understanding of vLLM and
 * PagedAttention", "Step 3 -- Tokens Generated Sequentially" and "Step 4 --
 * Attention Computation"; "(2) vLLM Internals ...", 4.1 "Why It Could Go"].
 * For each sequence s with n_s = context_lens[s] >= 1 (after the clamp of
 * pkv_paged_attention_decode), the key and value rows k_new[s], v_new[s]
 * ([num_kv_heads][head_dim], tokens new_token_stride elements apart, as in
 * pkv_reshape_and_cache) are written to position n_s - 1 of s, i.e. slot
 * block_table[s][(n_s-1)/16]*16 + (n_s-1)%16, and the output is then exactly
 * what pkv_paged_attention_decode gives on the updated cache: the same as
 * pkv_reshape_and_cache with that slot per sequence followed by
 * pkv_paged_attention_decode, bit for bit, with one kernel fewer. A block id
 * outside [1, num_blocks) at that position is not written (the attention
 * then reads block 0, as the decode does for such ids). The block holding
 * position n_s - 1 must be read by no other sequence of the call (a block
 * being appended to is private: pkv_seq_append reports the copy-on-write
 * pairs to run through pkv_copy_blocks first); otherwise the other sequence
 * may see the old or the new row. k_cache and v_cache are written. Same errors as
 * pkv_paged_attention_decode, plus PKV_ERR_INVALID_ARG for NULL or
 * misaligned k_new/v_new or a stride below num_kv_heads*head_dim. */
int pkv_paged_attention_decode_append(void* out, const void* q, const void* k_new,
                                      const void* v_new, int64_t new_token_stride, void* k_cache,
                                      void* v_cache, const int32_t* block_table,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_blocks, int32_t max_blocks_per_seq,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float scale, int32_t dtype, void* workspace,
                                      size_t workspace_bytes, void* stream);
/* Its first phase alone (the split-KV kernel with the append), for callers
 * that time the phases; the second is pkv_paged_attention_decode_merge with
 * the same workspace and shared arguments. */
int pkv_paged_attention_decode_append_split(void* out, const void* q, const void* k_new,
                                            const void* v_new, int64_t new_token_stride,
                                            void* k_cache, void* v_cache,
                                            const int32_t* block_table,
                                            const int32_t* context_lens, int32_t num_seqs,
                                            int32_t num_blocks, int32_t max_blocks_per_seq,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, float scale, int32_t dtype,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/* Size of the scratch array each GPU holds for pkv_paged_attention_decode_noalloc. */
#define PKV_DECODE_SCRATCH_BYTES (16 * 1024 * 1024)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * of pkv_paged_attention_decode, same arguments and same kernels, minus the
 * workspace. Its bookkeeping and partial states live in a file-scope device
 * array of PKV_DECODE_SCRATCH_BYTES (16 MiB) that every GPU the library runs
 * on holds until the process ends; the call allocates nothing (the first call
 * on a device looks the array's device address up once). Sizes whose decode
 * workspace (pkv_decode_workspace_size) exceeds the array are refused with
 * PKV_ERR_WORKSPACE: about 4 MB at 4 query heads per KV head and head_dim 128
 * with the default 3 waves per CU, 13 MB at 16. All calls on one GPU share
 * the array, which keeps the last call's contents (the decode needs no
 * initialisation of it): calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller. */
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_table,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       float scale, int32_t dtype, void* stream);

/* Workspace bytes pkv_paged_attention_decode_shared_prefix needs for these
 * sizes on the current device. */
int pkv_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t prefix_blocks, size_t* out);

/* Decode attention for a batch whose sequences all start with the same
 * prefix_blocks physical blocks (a shared prefix held once, refcounted
 * ["(2) vLLM Internals ...", 1.2 "Three Direct Wins", items 2 and 3;
 * "vLLM: what PagedAttention turned into", "The block pool, and the two
 * tricks in it"]). Same result as pkv_paged_attention_decode (to rounding),
 * computed as: the queries against the shared prefix as dense MFMA tiles
 * whose columns are the query rows of 2 to 32 sequences at once (the prefix
 * is read once per KV head and column block instead of once per sequence),
 * in the same launch as, and beside, the decode over each sequence's own
 * blocks; then a merge that folds the prefix's softmax states with the
 * sequence's own (online-softmax rescaling, prefix first). The prefix block ids are read
 * from row 0 of block_table; every sequence's context_lens must be at least
 * prefix_blocks*16 and its first prefix_blocks table entries equal row 0's
 * (caller contract; otherwise the result is undefined but every access stays
 * inside the pools and the table). fp32 and prefix_blocks == 0 run the
 * ordinary decode. workspace: >= pkv_decode_shared_prefix_workspace_size
 * bytes, device memory, no initialisation. Other arguments as
 * pkv_paged_attention_decode. */
int pkv_paged_attention_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                             const void* v_cache, const int32_t* block_table,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t num_blocks, int32_t max_blocks_per_seq,
                                             int32_t prefix_blocks, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, float scale,
                                             int32_t dtype, void* workspace,
                                             size_t workspace_bytes, void* stream);

/* Workspace bytes pkv_paged_attention_prefill_chunk can use on the current
 * device (0: none for these sizes). A bf16 call whose row blocks (chunks x
 * KV heads x ceil(max_q_len / row tokens)) are fewer than the device's CUs
 * cuts each row block's positions into parts (enough to keep every CU
 * busy, at most 16), one workgroup each,
 * when it is given a workspace of this size: the parts leave softmax states
 * there and a second kernel folds them in part order. total_q and
 * max_context_len do not change the size. */
int pkv_prefill_workspace_size(int32_t num_chunks, int32_t total_q, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t max_q_len,
                               int32_t max_context_len, size_t* out);

/* Chunked-prefill attention: each chunk is a run of consecutive query tokens
 * of one sequence, attending causally to the sequence's cached tokens plus
 * the chunk's own ["(2) vLLM Internals ...", section "2. Continuous
 * Batching"; "vLLM: what PagedAttention turned into", section "The
 * scheduler, and what it has to balance now"]. Chunk c owns query rows
 * cu_q_lens[c] .. cu_q_lens[c+1]-1 of q/out; context_lens[c] is the
 * sequence's total length including the chunk (the chunk's K/V are already
 * in the pool), so query i of the chunk sits at position
 * p = context_lens[c] - q_len_c + i and attends to positions 0..p.
 * q, out: device [total_q][num_q_heads][head_dim] in `dtype`; total_q is
 * normally cu_q_lens[num_chunks] (rows a chunk would place at or beyond
 * total_q are not computed, never read or written).
 * cu_q_lens: device int32 [num_chunks+1], non-decreasing from 0.
 * context_lens: device int32 [num_chunks]. block_table: device int32
 * [num_chunks][max_blocks_per_seq]. max_q_len bounds every chunk's length
 * (rows beyond it are not computed). Chunks with context_lens < q_len are
 * treated as starting at position 0.
 * workspace: NULL, or device memory of at least
 * pkv_prefill_workspace_size(...) bytes, 16-byte aligned, no initialisation
 * needed (smaller gives PKV_ERR_WORKSPACE); with it, a launch with few row
 * blocks splits their positions over more workgroups (the result differs
 * only in rounding). Calls that overlap in time must not share a workspace. */
int pkv_paged_attention_prefill_chunk(void* out, const void* q, const int32_t* cu_q_lens,
                                      const int32_t* context_lens, const int32_t* block_table,
                                      const void* k_cache, const void* v_cache,
                                      int32_t num_chunks, int32_t total_q, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_q_len,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float scale, int32_t dtype,
                                      void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
