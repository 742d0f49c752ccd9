/*
 * pkv.h — C interface of libpkv: decode-step attention over a paged KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * The cache is cut into fixed-size blocks of `block_size` tokens; a sequence
 * owns an ordered list of physical block ids (its block-table row), so its
 * cache is logically contiguous and physically scattered
 * (hnwysp.cn/news/103996 §2.2; icman.com.cn/news/78786 §2.1).  The library has
 * two halves:
 *
 *   - a host block allocator (FIFO free queue + per-block reference counts,
 *     sequence fork / reserve / release with copy-on-write), pure C++, no GPU;
 *   - three device operations: scatter new K/V rows into their slots
 *     (pkv_append), duplicate whole blocks for copy-on-write
 *     (pkv_copy_blocks), and decode attention through the block table
 *     (pkv_attention_decode).
 *
 * Conventions
 *   - Every function returns a status: PKV_OK (0) or a negative PKV_ERR_*.
 *     pkv_last_error() returns a human-readable detail of the calling
 *     thread's most recent failure.  Out-parameters are written only on
 *     success, and a failed allocator call leaves the allocator unchanged.
 *   - Device pointers are caller-owned memory the GPU can access.  Pools, K/V
 *     rows, queries, outputs and workspaces are device memory.  The small
 *     per-step metadata (slot mappings, block tables, lengths, copy pairs)
 *     may also be pinned host memory (hipHostMalloc), which the kernels read
 *     in place: a few host-memory reads per work-group instead of a
 *     host-to-device copy on the queue.  The library keeps no pointer after
 *     a call returns and never allocates, frees or synchronises: device
 *     operations are enqueued on `stream` and return.  The caller keeps every
 *     buffer alive and unchanged until the stream has finished with it.
 *   - Pool layout (both K and V, per layer): [num_blocks][block_size]
 *     [num_heads][head_dim], contiguous, element type `dtype`.  Token
 *     position `pos` of a sequence lives in block table[pos / block_size] at
 *     slot pos % block_size — the [page, slot, head, dim] order of
 *     m.lqnn.cn/news/240480 §3.3.  The flat slot index of a token is
 *     block * block_size + pos % block_size.
 *   - Supported shapes: head_dim 64 or 128; block_size 8, 16 or 32; dtype
 *     f32, f16 or bf16.  Anything else returns PKV_ERR_INVALID.
 *   - Pools, K/V rows, queries, outputs and scale pools are moved 16 bytes
 *     per lane: their base addresses must be 16-byte aligned (any device
 *     allocation is).  Calls check this on the host and return
 *     PKV_ERR_INVALID before enqueueing anything.
 *   - The allocator is not thread-safe; callers serialise access to one
 *     allocator.  Device operations are reentrant.
 *   - Device-side indices are always range-checked, in every build: a block
 *     id outside [0, num_blocks) or a slot outside the pool is never used to
 *     form an address.  Decode calls turn such a sequence's output into NaN
 *     rows; scatter and block copies skip the row or pair.  (The page this
 *     follows checks its indices with asserts in debug builds only,
 *     m.lqnn.cn/news/240480 §5.2 tip 3; here the check is one compare per
 *     64 block ids and stays on, and there is no build that traps.)
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(PKV_BUILDING_LIBRARY)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,   /* bad argument: null pointer, unsupported shape, inconsistent sizes */
  PKV_ERR_NO_BLOCKS = -2, /* pool exhausted: the request took nothing (caller queues or preempts) */
  PKV_ERR_BAD_BLOCK = -3, /* block id outside [0, num_blocks) */
  PKV_ERR_REFCOUNT = -4,  /* reference count would go below zero, or a free block was shared */
  PKV_ERR_HIP = -5        /* a HIP runtime call failed (launch error) */
};

/* Element types.  F32/F16/BF16 are the types of queries, outputs, new K/V
 * rows and 16/32-bit caches; I8 and FP8_E4M3 are 8-bit cache formats only
 * (symmetric int8 codes in [-127, 127]; OCP FP8 E4M3, bias 7, largest 448). */
typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_I8 = 3, PKV_FP8_E4M3 = 4 } pkv_dtype;

/* Short description of a status code (static storage). */
PKV_API const char* pkv_strerror(int status);
/* Detail of the calling thread's last failure ("" if none). */
PKV_API const char* pkv_last_error(void);
/* Library interface version (major * 100 + minor). */
PKV_API int pkv_version(void);

/* Kernel timing of the calling thread's next decode-attention call (any
 * pkv_*attention_decode* entry point): `start` is recorded when that call's
 * first kernel starts and `stop` when its last kernel ends, as timestamps of
 * those kernels themselves (hipExtLaunchKernelGGL), so no extra packet
 * enters the queue — on MI355X an event recorded between two kernels delays
 * the second one's start by about 4 us, which would be counted as the
 * call's time.  Either event may be null.  The caller creates both
 * (hipEventCreate, timing enabled) and reads them with hipEventElapsedTime
 * after the stream has passed the call.  The request is consumed by the next
 * decode call on this thread, whether that call succeeds or not (a call that
 * fails before enqueueing leaves the events unrecorded).  Always PKV_OK. */
PKV_API int pkv_time_next_decode(hipEvent_t start, hipEvent_t stop);

/* ---------------------------------------------------------------------------
 * Host block allocator
 *
 * One object per pool.  Block ids are 0 .. num_blocks-1.  The free list is a
 * queue: allocation takes its head, a block whose count drops to zero goes
 * to its tail (hnwysp.cn/news/103996 §3.4).  Allocation is O(1) — no scan of
 * the pool (m.lqnn.cn/news/240480 §5.2 tip 1).  Host memory owned by the
 * allocator; released by pkv_allocator_destroy.
 * ------------------------------------------------------------------------- */
typedef struct pkv_allocator pkv_allocator;

/* Create a pool of `num_blocks` blocks of `block_size` tokens.
 * `initial_free_order` (may be NULL = 0,1,..,n-1) must be a permutation of the
 * ids: it is the initial queue order, which decides where blocks land
 * physically (hnwysp.cn/news/103996 §3.2 threads every block onto the free
 * list at start-up).  PKV_ERR_INVALID on a bad size or non-permutation. */
PKV_API int pkv_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                                 pkv_allocator** out);
PKV_API void pkv_allocator_destroy(pkv_allocator* a);

/* Pop the head of the free queue (with the prefix cache on and the queue
 * empty: evict the least recently released cached block); its count becomes
 * 1.  PKV_ERR_NO_BLOCKS when nothing is available — the pool is full and the
 * caller queues the request (hnwysp.cn/news/103996 §4.4 alloc_block). */
PKV_API int pkv_block_alloc(pkv_allocator* a, int32_t* block_out);
/* Take n blocks at once, each as pkv_block_alloc would in turn, into
 * blocks_out[0 .. n).  All or nothing: PKV_ERR_NO_BLOCKS takes nothing when
 * fewer than n are available (the page pool's allocate_pages(n), which
 * checks the free count before taking pages from the front,
 * m.lqnn.cn/news/240480 §4.2).  Release them with pkv_seq_release. */
PKV_API int pkv_blocks_alloc(pkv_allocator* a, int32_t n, int32_t* blocks_out);
/* Share a block: count + 1.  PKV_ERR_REFCOUNT if the block is free
 * (hnwysp.cn/news/103996 §3.3: a prefix hit raises the count). */
PKV_API int pkv_block_incref(pkv_allocator* a, int32_t block);
/* Drop one reference; at zero the block joins the tail of the free queue
 * (hnwysp.cn/news/103996 §4.4 free_block; icman.com.cn/news/78786 §3.3), or
 * the prefix cache's evictable list if it holds a key.
 * PKV_ERR_REFCOUNT if the block is already free. */
PKV_API int pkv_block_decref(pkv_allocator* a, int32_t block);
/* Reference count (>= 0) of a block, or PKV_ERR_BAD_BLOCK. */
PKV_API int pkv_block_refcount(const pkv_allocator* a, int32_t block);
/* Blocks in the free queue (evictable cached blocks are not counted). */
PKV_API int32_t pkv_num_free(const pkv_allocator* a);
PKV_API int32_t pkv_num_blocks(const pkv_allocator* a);
PKV_API int32_t pkv_block_size(const pkv_allocator* a);
/* Copy the free queue, head first, into out[0 .. min(capacity, num_free)).
 * Returns the number of ids written. */
PKV_API int pkv_free_list(const pkv_allocator* a, int32_t* out, int32_t capacity);

/* Sequence helpers over caller-owned block-table rows (host int32 arrays).  */

/* Share all `n_blocks` blocks of src_row with a new sequence: each count + 1,
 * ids copied to dst_row (a prefix hit maps the new request's table entries to
 * the same physical blocks, icman.com.cn/news/78786 §3.4).  All or nothing. */
PKV_API int pkv_seq_fork(pkv_allocator* a, const int32_t* src_row, int32_t n_blocks, int32_t* dst_row);

/* Make room for positions cur_len .. cur_len+n_new-1 of one sequence.
 * `row` holds *n_blocks ids (must equal ceil(cur_len / block_size)) and has
 * room for row_capacity.  For each new position in order:
 *   - a position that opens a new block appends a fresh block
 *     (hnwysp.cn/news/103996 §4.2: take a block when the last one is full);
 *   - the first write into an existing block whose count is above one copies
 *     it: a fresh destination block is taken, (source, destination) is
 *     emitted into cow_pairs_out, the source loses one reference and the row
 *     entry is patched (copy-on-write, hnwysp.cn/news/103996 §3.3);
 *   - slots_out[i] = row[pos / block_size] * block_size + pos % block_size.
 * At most one pair is produced (only the partly filled last block can be
 * shared), so cow_pairs_out needs room for 2 int32.  Fresh blocks plus the
 * copy are checked against the free count first: PKV_ERR_NO_BLOCKS takes
 * nothing (m.lqnn.cn/news/240480 §4.2 allocate_pages).  The copy must be
 * enqueued (pkv_copy_blocks) before the append that writes the new rows. */
PKV_API int pkv_seq_reserve(pkv_allocator* a, int32_t* row, int32_t row_capacity, int32_t* n_blocks,
                            int32_t cur_len, int32_t n_new, int64_t* slots_out, int32_t* cow_pairs_out,
                            int32_t* n_cow_out);

/* pkv_seq_reserve over `batch` sequences in ascending order, all or nothing.
 * tables: [batch][row_stride] (row capacity = row_stride); n_blocks[batch] is
 * updated; slots_out receives sum(n_new) slots, sequence-major;
 * cow_pairs_out: [cow_capacity][2] (cow_capacity >= batch suffices). */
PKV_API int pkv_seq_reserve_batch(pkv_allocator* a, int32_t* tables, int32_t row_stride, int32_t* n_blocks,
                                  const int32_t* cur_lens, const int32_t* n_new, int32_t batch,
                                  int64_t* slots_out, int32_t* cow_pairs_out, int32_t cow_capacity,
                                  int32_t* n_cow_out);

/* Release a sequence: one reference dropped from each block, in logical
 * order.  Validated first (ids in range, enough references), so a failure
 * changes nothing.  Finished, cancelled and failed requests all go through
 * this one call (m.lqnn.cn/news/240480 §5.3; icman.com.cn/news/78786 §6.3). */
PKV_API int pkv_seq_release(pkv_allocator* a, const int32_t* row, int32_t n_blocks);

/* ---------------------------------------------------------------------------
 * Block-level prefix cache (host, inside the allocator; off until enabled)
 *
 * Requests that share a token prefix share the blocks holding its K/V
 * (icman.com.cn/news/78786 §3.1-§3.4; hnwysp.cn/news/103996 §4.2, §4.3;
 * m.lqnn.cn/news/240480 §3.2 step 1).  Each full block of a sequence can be
 * recorded under a key naming the token prefix that ends with it:
 *   key_i = SHA-256(key_{i-1} || tokens of block i as little-endian int32),
 *   key_{-1} = 32 zero bytes
 * (a collision-resistant hash over the token sequence itself, extended block
 * by block, icman.com.cn/news/78786 §3.2, §4.4).  A new request's blocks are
 * matched from the first one until the first miss; a hit increments the
 * block's count and joins the request's table with no copy (§3.4).  A cached
 * block whose count falls to zero is not freed: it waits in a
 * least-recently-released list and can still be matched.  Allocation takes
 * the free queue first; only when it is empty is the least recently released
 * cached block evicted (its key dropped) and handed out, so "available"
 * blocks = free + evictable (§3.3; hnwysp.cn/news/103996 §3.5).  Only full
 * blocks are cached, so copy-on-write never meets a cached block.
 * ------------------------------------------------------------------------- */

/* Turn the prefix cache on (idempotent; O(num_blocks) host memory). */
PKV_API int pkv_prefix_cache_enable(pkv_allocator* a);

/* Chained keys of the full blocks of tokens[0 .. n_tokens): writes
 * min(n_tokens / block_size, capacity) keys of 32 bytes to keys_out and
 * returns that count (or a negative status).  Needs no allocator. */
PKV_API int pkv_prefix_block_keys(const int32_t* tokens, int32_t n_tokens, int32_t block_size, uint8_t* keys_out,
                                  int32_t capacity);

/* Longest cached prefix of tokens[0 .. n_tokens), at most row_capacity
 * blocks: the matched block ids go to row_out[0 .. *n_blocks_out) (the
 * start of the request's table row; its first *n_blocks_out * block_size
 * tokens need no prefill) and each matched block's count is incremented.
 * The caller then reserves the rest with pkv_seq_reserve from cur_len =
 * *n_blocks_out * block_size.  PKV_ERR_INVALID if the cache is off. */
PKV_API int pkv_prefix_match(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens, int32_t* row_out,
                             int32_t row_capacity, int32_t* n_blocks_out);

/* Record a sequence's full blocks under their keys once their K/V are
 * written: blocks row[first_block .. min(n_blocks, n_tokens / block_size)).
 * Blocks before first_block are the ones pkv_prefix_match returned for
 * these tokens: the key chain resumes from the key of row[first_block - 1]
 * (which must be cached), so matched blocks are not hashed again.  A key
 * already recorded keeps its first block (this one stays an ordinary block);
 * a block already recorded under the same key is skipped.  Every block
 * recorded must be held (count >= 1), and a block recorded under a different
 * key is PKV_ERR_INVALID; both are checked before anything changes.
 * *n_new_out (may be NULL) = blocks newly recorded. */
PKV_API int pkv_prefix_register(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens, const int32_t* row,
                                int32_t n_blocks, int32_t first_block, int32_t* n_new_out);

/* Blocks currently holding a key (held or evictable). */
PKV_API int32_t pkv_prefix_cached_blocks(const pkv_allocator* a);

/* Evictable cached blocks (count zero), least recently released first: writes
 * up to `capacity` ids, returns how many. */
PKV_API int pkv_prefix_lru(const pkv_allocator* a, int32_t* out, int32_t capacity);

/* ---------------------------------------------------------------------------
 * Device operations
 * ------------------------------------------------------------------------- */

/* Scatter new K/V rows into the pools.
 * k_new, v_new: device [num_tokens][num_heads][head_dim] of `dtype`;
 * slot_mapping: int64 [num_tokens] (device or pinned host); token t goes to flat slot
 * slot_mapping[t] of k_cache / v_cache (device pools, layout above).  A
 * negative slot is skipped (padding); a slot >= num_blocks * block_size is
 * also skipped, never written.  A bit copy: the new step's K/V join the cache
 * before attention reads it (hnwysp.cn/news/103996 §1.1;
 * m.lqnn.cn/news/240480 §3.2 step 3). */
PKV_API int pkv_append(const void* k_new, const void* v_new, int32_t num_tokens, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size, int32_t num_heads,
                       int32_t head_dim, pkv_dtype dtype, hipStream_t stream);

/* Copy whole blocks for copy-on-write (hnwysp.cn/news/103996 §3.3).
 * k_caches, v_caches: HOST arrays of `num_layers` device pool pointers.
 * pairs: int32 [n_pairs][2] (device or pinned host) = (source, destination) block ids.
 * Every layer's K and V block `dst` becomes a bit copy of block `src`
 * (bytes_per_block = block_size * num_heads * head_dim * dtype bytes, a
 * multiple of 16).  Pairs are copied concurrently: destinations must be
 * distinct and no destination may be a source (the allocator never emits
 * such pairs).  A pair with an id outside [0, num_blocks) is skipped. */
PKV_API int pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                            const int32_t* pairs, int32_t n_pairs, int32_t num_blocks, size_t bytes_per_block,
                            hipStream_t stream);

/* Swap whole blocks between two pool sets, for preemption: one side device
 * pools, the other pinned host pools (hipHostMalloc), or both device.  A
 * preempted request's blocks are swapped out to host memory and back in when
 * blocks free up, instead of being recomputed (icman.com.cn/news/78786 §4.2;
 * the host tier of l189.com/news/1438543 §3).  For every pool i < num_pools
 * and pair j: block pairs[j][1] of dst_pools[i] becomes a bit copy of block
 * pairs[j][0] of src_pools[i] (bytes_per_block each, a multiple of 16; pools
 * 16-byte aligned).  dst_pools / src_pools are HOST arrays of num_pools
 * pointers (typically K and V of every layer, plus the scale pools of an
 * 8-bit cache in a second call); pairs: int32 [n_pairs][2] (device or pinned
 * host).  Pair ids outside [0, src_num_blocks) / [0, dst_num_blocks) are
 * skipped; destinations must be distinct (a host-side pkv_allocator for the
 * swap space hands out such ids).  Every pool and the pairs are checked with
 * hipPointerGetAttributes before the launch: pageable host memory is
 * PKV_ERR_INVALID.  One launch per 64 pools; asynchronous on `stream`. */
PKV_API int pkv_swap_blocks(void* const* dst_pools, const void* const* src_pools, int32_t num_pools,
                            const int32_t* pairs, int32_t n_pairs, int32_t src_num_blocks, int32_t dst_num_blocks,
                            size_t bytes_per_block, hipStream_t stream);

/* Chunk streams a decode call runs when called with num_work_groups = 0,
 * for caches of `cache_dtype`: seven eighths of the compute units of the
 * current device for F32/F16/BF16 caches (224 on MI355X, one work-group
 * each), seven eighths of two per compute unit for I8 and FP8_E4M3 caches
 * (448, run two to a work-group where both fit, see
 * pkv_attention_decode_quant).  PKV_ERR_HIP if no device is current,
 * PKV_ERR_INVALID for an unknown type. */
PKV_API int32_t pkv_decode_work_groups(pkv_dtype cache_dtype);

/* Device workspace a decode call needs for `num_work_groups` (0 = the
 * automatic count for that cache type).  `dtype` is the cache element type:
 * F32/F16/BF16 for pkv_attention_decode, I8/FP8_E4M3 for
 * pkv_attention_decode_quant.  It holds a per-sequence plan (2 int32 per sequence and head
 * slice, at most 5460 per launch) and float32 partial softmax states for
 * 2 * num_work_groups pieces of num_heads * (head_dim + 2) floats, each
 * region 256-byte aligned.  It does not depend on sequence lengths.
 * Returns 0 for an invalid shape. */
PKV_API size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype dtype,
                                          int32_t num_work_groups);

/* Decode attention through the block table.
 * For every sequence b < batch and head h < num_heads, with L = seq_lens[b]:
 *   out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) V_t,  t = 0 .. L-1,
 * where K_t, V_t are the rows of logical position t, found at block
 * block_tables[b][t / block_size], slot t % block_size (the attention kernel
 * walks the table block by block, icman.com.cn/news/78786 §2.4; the logical
 * to physical index redirection of m.lqnn.cn/news/240480 §3.3).  L includes
 * the token appended this step.
 *   out, q: device [batch][num_heads][head_dim] of `dtype`; out rounded to
 *     nearest-even from float32 accumulation.
 *   k_cache, v_cache: device pools of num_blocks blocks (layout above).
 *   block_tables: int32 [batch][max_blocks_per_seq] (device or pinned host).
 *   seq_lens: int32 [batch] (device or pinned host).  max_seq_len: host upper bound of every
 *     seq_lens entry (sizes the launch and the workspace).
 *   scale: softmax scale (1/sqrt(head_dim) for plain scaled dot-product).
 *   num_work_groups: 0 = automatic (pkv_decode_work_groups), else the
 *     number of work-groups.  The tokens of all sequences are laid end to
 *     end in chunks of 8 and every work-group takes an equal contiguous
 *     range of chunks, so the work is balanced however ragged the lengths
 *     are.  A sequence split across ranges is computed in pieces whose
 *     partial softmax states (max, sum, weighted values) a second kernel on
 *     the same stream merges.  Cut points depend only on logical positions,
 *     so the result does not depend on where the blocks sit physically.
 *   workspace: device memory of at least pkv_decode_workspace_bytes(...)
 *     (no initialisation needed; calls sharing one must not overlap).
 * L = 0 gives a zero row.  A sequence whose length is negative or exceeds
 * max_seq_len or max_blocks_per_seq * block_size, or whose table holds an id
 * outside [0, num_blocks) in its first ceil(L / block_size) entries, gets
 * NaN rows: the kernel checks every id before using it and never reads
 * outside the pools. */
PKV_API int pkv_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype,
                                 int32_t num_work_groups, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Size of the device scratch array pkv_attention_decode_scratch uses on each
 * device (32 MiB). */
#define PKV_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/* pkv_attention_decode for callers that cannot allocate device memory (code
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a 32 MiB array the library holds on each
 * device, so the call takes no workspace argument and allocates nothing.
 * Every argument and result is that of pkv_attention_decode (same kernels,
 * same work split: bit-identical output for the same num_work_groups).
 * Sizes whose workspace (pkv_decode_workspace_bytes) would exceed
 * PKV_DECODE_SCRATCH_BYTES return PKV_ERR_INVALID and launch nothing (the
 * 7B shape, 32 heads x 128 at the automatic 224 work-groups, needs about 7.5
 * MB).  The array is shared by every call on its device and keeps the last
 * call's contents (nothing in it needs clearing): calls that may overlap on
 * one device must go through one stream, in order.  The first call on a
 * device looks up the array's device address (PKV_ERR_HIP if that fails). */
PKV_API int pkv_attention_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                         int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         float scale, pkv_dtype dtype, int32_t num_work_groups, hipStream_t stream);

/* Scatter and decode attention in one launch: for every sequence b with
 * L = seq_lens[b] >= 1, the new rows k_new[b], v_new[b] (device
 * [batch][num_heads][head_dim] of `dtype`) are stored at logical position
 * L - 1, i.e. at block block_tables[b][(L - 1) / block_size], slot
 * (L - 1) % block_size, and attention then runs over positions 0 .. L - 1
 * exactly as pkv_attention_decode.  The result, in `out` and in the pools,
 * equals pkv_append with slot_mapping[b] = that slot followed by
 * pkv_attention_decode; one launch (one kernel boundary) less per layer.
 * The slot is taken from the table, so the caller's reservation must already
 * have put the block there (and copied it if it was shared).  A sequence
 * whose length is invalid, or whose block for L - 1 is outside
 * [0, num_blocks), writes nothing and gets NaN rows.  Every other argument
 * is that of pkv_attention_decode. */
PKV_API int pkv_append_attention_decode(void* out, const void* q, const void* k_new, const void* v_new,
                                        void* k_cache, void* v_cache, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                        int32_t batch, int32_t num_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, float scale, pkv_dtype dtype, int32_t num_work_groups,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 8-bit caches (int8 or OCP FP8 E4M3)
 *
 * Storing K/V in 8 bits halves the bytes per token against fp16 and changes
 * nothing of the paging: block tables, slots, the allocator and
 * pkv_copy_blocks are the same (hnwysp.cn/news/103996 §5.4;
 * icman.com.cn/news/78786 §1.3; m.lqnn.cn/news/240480 §6.2).
 *
 * Code pools: [num_blocks][block_size][num_heads][head_dim] bytes, the
 * layout above with one-byte elements.  Scale pools: float32
 * [num_blocks][num_heads][block_size], one scale per (token, head) row, for K
 * and for V.  A row x of head_dim values is stored as
 *   scale = max_i |x_i| / QMAX          (QMAX = 127 for I8, 448 for FP8_E4M3)
 *   I8:       code_i = clamp(rint(x_i / scale), -127, 127)
 *   FP8_E4M3: code_i = the E4M3 value nearest clamp(x_i / scale, -448, 448),
 *             ties to the even code (bias 7, subnormals, no infinities)
 * with float32 arithmetic (IEEE division); a row of zeros stores scale 0 and
 * zero codes.  It reads back as code_i * scale.  New rows must be finite.
 * Copy-on-write copies a block of the code pools and of the scale pools:
 * call pkv_copy_blocks once with the code pools (bytes_per_block =
 * block_size * num_heads * head_dim) and once with the scale pools
 * (num_heads * block_size * 4).
 * ------------------------------------------------------------------------- */

/* Quantise and scatter new K/V rows.
 * k_new, v_new: device [num_tokens][num_heads][head_dim] of src_dtype
 * (F32, F16 or BF16); slot_mapping: int64 [num_tokens] (device or pinned
 * host).  Token t's codes go to flat slot slot_mapping[t] of k_cache /
 * v_cache and its per-head scales to k_scales / v_scales at
 * [slot / block_size][h][slot % block_size].  Negative slots and slots >=
 * num_blocks * block_size are skipped.  cache_dtype: I8 or FP8_E4M3.
 * Rows and pools must be 16-byte aligned. */
PKV_API int pkv_append_quant(const void* k_new, const void* v_new, int32_t num_tokens,
                             const int64_t* slot_mapping, void* k_cache, void* v_cache, float* k_scales,
                             float* v_scales, int32_t num_blocks, int32_t block_size, int32_t num_heads,
                             int32_t head_dim, pkv_dtype src_dtype, pkv_dtype cache_dtype, hipStream_t stream);

/* Decode attention over an 8-bit paged cache: pkv_attention_decode's result
 * with every K/V element read as code * scale of its row, dequantised inside
 * the kernel.  q and out are device [batch][num_heads][head_dim] of q_dtype
 * (F32, F16 or BF16); k_scales / v_scales the scale pools above;
 * cache_dtype I8 or FP8_E4M3; every other argument, the workspace
 * (pkv_decode_workspace_bytes with dtype = cache_dtype) and the handling of
 * bad lengths and block ids are those of pkv_attention_decode, except that
 * num_work_groups counts chunk streams: where two sets of the wavefronts
 * that cover the heads fit one work-group of 8 (32 heads of 128, 64 of 64),
 * the call runs ceil(num_work_groups / 2) work-groups whose two streams take
 * alternate chunks of one range (the score variant keeps one stream per
 * work-group).  q, out, pools and scale pools must be 16-byte aligned. */
PKV_API int pkv_attention_decode_quant(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const float* k_scales, const float* v_scales,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                       int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                       int32_t num_work_groups, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* pkv_append_attention_decode for an 8-bit cache: each sequence's new rows
 * (k_new, v_new: device [batch][num_heads][head_dim] of q_dtype, 16-byte
 * aligned) are quantised exactly as pkv_append_quant does, stored with their
 * scales at position L - 1, and attention runs over positions 0 .. L - 1 as
 * pkv_attention_decode_quant. */
PKV_API int pkv_append_attention_decode_quant(void* out, const void* q, const void* k_new, const void* v_new,
                                              void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                              int32_t num_heads, int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                              pkv_dtype cache_dtype, int32_t num_work_groups, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Cumulative attention score per cached token
 *
 * A cached token's importance is the attention past queries paid to it:
 * after each step every key position adds the weight it received, and the
 * running total decays exponentially once per step (zskr.cn/news/1363082.html
 * §3.1 cumulative attention score, §4.1 decay factor).  For every sequence b
 * and logical position t < L = seq_lens[b]:
 *   scores[b][t] = decay * scores[b][t] + (1/H) sum_h p_{b,h}(t)
 * where p_{b,h} is this step's softmax distribution of head h (the weights
 * the decode output is averaged with).  Positions >= L and sequences with an
 * invalid length are untouched; a row starts from zero when its sequence
 * starts (the caller zeroes it).  The decode launch stores each position's
 * scaled logit, and each head's final softmax (max, sum) for sequences it
 * attends in one piece, in `scores_workspace`; the second launch on the
 * stream merges split sequences and folds the logits into `scores` (for a
 * split sequence it forms each head's (max, sum) from the pieces).
 * ------------------------------------------------------------------------- */

/* Bytes of the score workspace: float32 logits [batch][num_heads][S] with S =
 * max_seq_len rounded up to a multiple of 32 (so that 32 positions of a head
 * fill one 128-byte line), and float2 [batch][num_heads], each region
 * 256-byte aligned; 0 for an invalid shape. */
PKV_API size_t pkv_decode_scores_workspace_bytes(int32_t batch, int32_t num_heads, int32_t max_seq_len);

/* pkv_attention_decode plus the score update above.  scores: device float32
 * [batch][score_stride], score_stride >= max_seq_len, updated in place;
 * decay: finite (e.g. 0.995); scores_workspace: device memory of at least
 * pkv_decode_scores_workspace_bytes(batch, num_heads, max_seq_len).  `out`
 * is pkv_attention_decode's result (a separate kernel instantiation: it may
 * differ from it in the last place). */
PKV_API int pkv_attention_decode_scores(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                        int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        float scale, pkv_dtype dtype, int32_t num_work_groups, void* workspace,
                                        size_t workspace_bytes, float* scores, int32_t score_stride, float decay,
                                        void* scores_workspace, size_t scores_workspace_bytes, hipStream_t stream);

/* The same for an 8-bit cache (pkv_attention_decode_quant plus scores). */
PKV_API int pkv_attention_decode_quant_scores(void* out, const void* q, const void* k_cache, const void* v_cache,
                                              const float* k_scales, const float* v_scales,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                              int32_t num_heads, int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                              pkv_dtype cache_dtype, int32_t num_work_groups, void* workspace,
                                              size_t workspace_bytes, float* scores, int32_t score_stride,
                                              float decay, void* scores_workspace, size_t scores_workspace_bytes,
                                              hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Grouped decode: shared prefixes read once per group.
 *
 * Sequences forked from one prompt, or matched in the prefix cache, begin
 * with the same physical blocks (hnwysp.cn/news/103996 §3.3;
 * icman.com.cn/news/78786 §3.1).  Plain decode reads such a prefix once per
 * sequence.  The grouped call reads it once per tile of up to 16 sequences
 * and head, with the tile's queries against the prefix as two small matrix
 * products on the matrix cores (scores = K Q^T, weighted values = V^T P^T,
 * with P split into two 16-bit parts so that the weights keep float32
 * precision); each sequence's own positions are attended by the decode
 * kernel, and the merge kernel combines the prefix's partial (max, sum,
 * weighted values) with those of the sequence's own positions.  The result
 * equals pkv_attention_decode.
 * ------------------------------------------------------------------------- */

#define PKV_PREFIX_TILE_SEQS 16    /* sequences per prefix tile */
#define PKV_PREFIX_TILE_INTS 18    /* int32 per tile: prefix blocks, member count, 16 sequence indices */
#define PKV_PREFIX_MAX_BLOCKS 1024 /* longest prefix a tile may cover, in blocks */

/* Host helper: groups the batch's sequences by shared leading blocks.
 * tables: host int32 [batch][max_blocks_per_seq]; seq_lens: host int32
 * [batch] (this step's lengths).  Sequences with the same first block id
 * form a group when there are at least max(2, min_sharers) of them; the
 * group's prefix is the longest run of leading ids all its members share,
 * capped for every member at the whole blocks before its last position
 * ((L - 1) / block_size), so each member keeps at least one position of
 * its own, and at PKV_PREFIX_MAX_BLOCKS (positions past it are read per
 * sequence).  A group with a prefix of at least one block is cut into tiles
 * of at most PKV_PREFIX_TILE_SEQS members in ascending sequence order.
 * Out: seq_prefix_blocks[b] = the prefix of b's group in blocks, or 0;
 * tiles: int32 [max_tiles][PKV_PREFIX_TILE_INTS], each
 * {prefix blocks, member count, member indices..., -1 padding}, the first
 * member's table row being the one the tile reads; *num_tiles.  At most
 * (batch + 1) / 2 tiles are ever needed.  PKV_ERR_INVALID if more than
 * max_tiles are needed (nothing written). */
PKV_API int pkv_prefix_tiles(const int32_t* tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             int32_t batch, int32_t block_size, int32_t min_sharers, int32_t* seq_prefix_blocks,
                             int32_t* tiles, int32_t max_tiles, int32_t* num_tiles);

/* Workspace bytes of pkv_attention_decode_grouped (dtype F16/BF16) and
 * pkv_attention_decode_grouped_quant (dtype = the cache's, I8/FP8_E4M3): the
 * plain decode workspace with room for one more partial state per sequence
 * and head slice (a sequence with a shared prefix always leaves one), plus
 * float32 prefix states [16][batch][num_heads][head_dim + 4] (up to 16
 * work-groups share one tile and head, each writing its part). */
PKV_API size_t pkv_decode_grouped_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim,
                                                  pkv_dtype dtype, int32_t num_work_groups);

/* pkv_attention_decode with shared prefixes read once per tile.
 * seq_prefix_blocks: int32 [batch] (device or pinned host), tiles: int32
 * [num_tiles][PKV_PREFIX_TILE_INTS] (device or pinned host), as written by
 * pkv_prefix_tiles from the same tables and lengths; num_tiles on the host,
 * 0 to 4,194,304 (2^22; more returns PKV_ERR_INVALID).
 * dtype f16 or bf16 (a cache of another type returns PKV_ERR_INVALID).  The
 * caller guarantees that the members of a tile share their first
 * seq_prefix_blocks blocks and that every sequence with seq_prefix_blocks
 * > 0 is a member of exactly one tile with that prefix; the prefix is read
 * from the first member's row; a tile's prefix is at most
 * PKV_PREFIX_MAX_BLOCKS blocks (a longer tile's members get NaN rows).  A
 * member whose length is refused, or not
 * longer than its prefix, is attended as an ungrouped sequence (with the
 * plain call's handling of refused lengths); out-of-range sequence indices
 * in a tile are skipped.  A prefix block id outside [0, num_blocks) makes
 * the tile's members NaN.  With num_tiles = 0 the call runs
 * pkv_attention_decode's kernels (seq_prefix_blocks is not read).  When the
 * decode work-groups are fewer than the device's compute units (the
 * automatic count is), hold 4 or 8 wavefronts (32 heads
 * of 128, for instance) and batch is at most 1024 per head slice, the prefix
 * work runs in the decode launch, in work-groups placed after the decode
 * ones; otherwise it has a launch of its own before the decode launch.  The
 * two ways split the prefix differently (results agree within rounding;
 * each is deterministic for given arguments and device).  Every other
 * argument is that of pkv_attention_decode; workspace:
 * pkv_decode_grouped_workspace_bytes. */
PKV_API int pkv_attention_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                         int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         float scale, pkv_dtype dtype, const int32_t* seq_prefix_blocks,
                                         const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* pkv_attention_decode_grouped for an 8-bit cache (int8 or OCP FP8 E4M3
 * codes with per-(token, head) scales, the format of
 * pkv_attention_decode_quant): the result equals pkv_attention_decode_quant.
 * Shared prefixes are quantised caches too: their codes enter the matrix
 * cores as the query's type (every E4M3 value, and every int8 value in
 * [-127, 127], is exact in f16 and in bf16), each position's K scale
 * multiplies its scores and its V scale its softmax weight
 * (icman.com.cn/news/78786 §1.3 and §3.4: quantised caches and shared
 * prefixes together).  q_dtype F16 or BF16 (else PKV_ERR_INVALID);
 * cache_dtype I8 or FP8_E4M3; k_scales, v_scales as for
 * pkv_attention_decode_quant; seq_prefix_blocks, tiles, num_tiles as for
 * pkv_attention_decode_grouped; workspace:
 * pkv_decode_grouped_workspace_bytes with dtype = cache_dtype.  The prefix
 * work runs in the decode launch under pkv_attention_decode_grouped's rule,
 * counting the decode work-groups (two chunk streams each where they fit,
 * as in pkv_attention_decode_quant).  Every other argument is that of
 * pkv_attention_decode_quant. */
PKV_API int pkv_attention_decode_grouped_quant(void* out, const void* q, const void* k_cache, const void* v_cache,
                                               const float* k_scales, const float* v_scales,
                                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                                               const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                               int32_t num_heads, int32_t head_dim, int32_t block_size,
                                               int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                               pkv_dtype cache_dtype, const int32_t* seq_prefix_blocks,
                                               const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Grouped decode with the step's new rows stored in the same launch: for
 * every sequence b with L = seq_lens[b] >= 1, k_new[b] and v_new[b] (device
 * [batch][num_heads][head_dim] of `dtype`) are stored at logical position
 * L - 1 as pkv_append_attention_decode stores them, then attention runs as
 * pkv_attention_decode_grouped.  A tile's prefix ends before each member's
 * last block (pkv_prefix_tiles), so the rows stored never lie in a prefix
 * the prefix kernel reads; the result, in `out` and in the pools, equals
 * pkv_append followed by pkv_attention_decode_grouped.  A sequence whose
 * length is invalid, or whose block for L - 1 is outside [0, num_blocks),
 * writes nothing and gets NaN rows.  Every other argument is that of
 * pkv_attention_decode_grouped. */
PKV_API int pkv_append_attention_decode_grouped(void* out, const void* q, const void* k_new, const void* v_new,
                                                void* k_cache, void* v_cache, const int32_t* block_tables,
                                                int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                int32_t max_seq_len, int32_t batch, int32_t num_heads,
                                                int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                                pkv_dtype dtype, const int32_t* seq_prefix_blocks,
                                                const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* pkv_append_attention_decode_grouped for an 8-bit cache: the new rows
 * (k_new, v_new of q_dtype, 16-byte aligned) are quantised and stored with
 * their scales as pkv_append_attention_decode_quant stores them, then
 * attention runs as pkv_attention_decode_grouped_quant. */
PKV_API int pkv_append_attention_decode_grouped_quant(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, float* k_scales,
    float* v_scales, const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, const int32_t* seq_prefix_blocks, const int32_t* tiles,
    int32_t num_tiles, int32_t num_work_groups, void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
