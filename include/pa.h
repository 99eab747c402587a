/*
 * pa.h -- C ABI of the paged KV-cache attention library (libpa.so, gfx950).
 *
 * The KV cache is cut into fixed 16-token blocks that live in one global
 * pool; every sequence owns a block table mapping its logical blocks to
 * physical blocks ("vLLM-Ascend 原理", §2.1 "PagedAttention 分页 KV 缓存").
 * The attention calls read K/V through that table, block by block, with no
 * gather into contiguous memory ("vLLM 在 CANN 上的推理优化", section
 * "CANN 上的 PagedAttention 算子" and the note after it on passing block ids
 * and the table straight to attention).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer to contiguous row-major
 * memory in the layout stated on the call; 16-bit tensors and the workspace
 * must be 16-byte aligned (the kernels move 16-byte vectors).  The caller allocates and owns
 * every buffer, including the decode workspace; the library allocates
 * nothing, keeps no pointer after a call returns, and holds no state, so
 * every call is re-entrant and may be issued from any host thread.
 *
 * Element types.  q, out, key, value and both caches share one 16-bit type,
 * pa_dtype (the *_fp8 calls at the end keep the caches as 8-bit codes with
 * float32 scales instead).  Accumulation is float32; outputs are rounded to
 * nearest even.
 *
 * KV cache layout.  k_cache and v_cache are two separate tensors, each
 * [num_blocks][block_size][num_kv_heads][head_dim].  Token slot
 * s = physical_block * block_size + offset addresses row s of the
 * [num_blocks * block_size][num_kv_heads][head_dim] view.  block_size is 16
 * or 32, the two usual block sizes ("vLLM 在 CANN 上的推理优化", section
 * "vLLM 的 PagedAttention 数据结构", the PagedKVCache sketch); the FP8 calls
 * take 16 only.  head_dim is 64 or 128.  The attention calls take pools of at
 * most 2^31 blocks (2^30 with 32-token blocks), the range an int32 table entry
 * can name in 16-token units; a larger num_blocks gives PA_ERR_SHAPE, and so
 * does an empty pool (num_blocks < 1), also in a call with nothing to do.
 *
 * Streams.  Work is enqueued on `stream` (0 = the null stream).  No call
 * synchronises, reads device memory from the host or allocates, so every call
 * may be captured in a HIP graph.  A return of PA_OK means "enqueued";
 * faults inside kernels surface at the caller's next synchronisation.
 *
 * Errors.  Arguments, and the launch grids they imply, are validated on the
 * host before anything is enqueued ("Hardware abstraction and portability",
 * §九: unsupported configurations fail early, at the boundary): after
 * PA_ERR_NULL_PTR, PA_ERR_UNSUPPORTED, PA_ERR_SHAPE, PA_ERR_WORKSPACE or
 * PA_ERR_ALIGNMENT nothing was launched.  PA_ERR_HIP means the HIP runtime
 * refused a launch; it is that launch's own status, so an error an earlier,
 * unrelated HIP call left on the thread is neither reported as PA_ERR_HIP nor
 * cleared.  The calls that enqueue several kernels (pa_decode, pa_decode_multi
 * and pa_decode_fp8 when they split or take sequence groups,
 * pa_copy_blocks_fp8) may have enqueued the first before the runtime refused a
 * later one.  No C++ exception crosses this
 * interface.  Device-resident indices are not validated on the host (that
 * would need a read-back): a block-table entry outside [0, num_blocks) or a
 * slot outside [0, num_blocks * block_size) is never dereferenced -- the
 * kernels skip it -- but results involving it are unspecified.  A debug build
 * of the library reports such indices (pa_debug_bounds, at the end).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's opaque stream handle (the same typedef as hip_runtime_api.h). */
typedef struct ihipStream_t* hipStream_t;

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
    PA_ERR_UNSUPPORTED = -2, /* head_dim, block_size or dtype outside what is built */
    PA_ERR_SHAPE = -3,       /* inconsistent or out-of-range sizes */
    PA_ERR_WORKSPACE = -4,   /* decode workspace missing or too small */
    PA_ERR_HIP = -5,         /* the HIP runtime refused a launch */
    PA_ERR_ALIGNMENT = -6,   /* a tensor or the workspace is not 16-byte aligned */
    PA_ERR_SCRATCH = -7,     /* pa_decode_noalloc: partials exceed PA_NOALLOC_SCRATCH_BYTES */
    PA_STATUS_RANGE_MAX_ = 0x7fffffff   /* not a status: see below */
} pa_status;

typedef enum pa_dtype {
    PA_F16 = 0,  /* IEEE binary16 */
    PA_BF16 = 1, /* bfloat16 */
    PA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,   /* not types: see below */
    PA_DTYPE_RANGE_MAX_ = 0x7fffffff
} pa_dtype;
/* The *_RANGE_* enumerators are never returned or accepted as values.  They
 * make every 32-bit integer a value of the enum type (in C++ an enum holds only
 * the values of the smallest bit-field that spans its enumerators), so a
 * caller's unknown dtype or status is refused or named "unknown" instead of
 * being undefined behaviour inside the library. */

#define PA_BLOCK_SIZE 16

/*
 * Decode flags.
 * PA_DECODE_STREAM_KV -- the caller guarantees that no physical block is read
 * twice within the call (no block shared by two sequences of the batch, as a
 * block manager knows from its reference counts -- "vLLM学习整理", §三 on
 * prefix caching).  K/V are then loaded with a non-temporal hint, which streams
 * them faster from HBM on gfx950.  Without the flag the loads stay cacheable,
 * which lets shared-prefix blocks be served from cache.  Results are
 * bit-identical either way; a wrong promise costs speed, not correctness.
 */
#define PA_DECODE_STREAM_KV 1u
/*
 * PA_DECODE_SHARED_PREFIX -- the caller (a block manager with prefix caching,
 * "vLLM学习整理", §三; "vLLM-Ascend 原理", §2.1) says that consecutive sequences
 * of the batch may point at the same physical blocks, typically their common
 * prefix.  Honoured by pa_decode and pa_decode_noalloc on the 16-bit matrix-core
 * decode (head_dim 128, 3 to 8 q heads per kv head) with partition_tokens 0 or
 * PA_PARTITION_BALANCED, where the balanced split fits (at most 512
 * sequences): one wave then carries the heads of S = 16 / group consecutive
 * sequences (S = 5, 4, 3, 2, 2, 2 for groups 3 to 8) through their leading
 * blocks, as long as two or more of them are still in play and all of those
 * name the same block, reading each such block once for all of them; the
 * balanced split takes the rest.  Sharing pays where runs of sequences with a
 * common prefix are aligned to S.  Everywhere else the flag is accepted and
 * has no effect.  Results agree with the unflagged call to the decode
 * tolerance, not bit for bit (the partial sums fall in other places).  Block
 * rows inside any sequence's context must be finite for the other sequences of
 * its wave to be exact (a zero weight times an infinite value is NaN).
 */
#define PA_DECODE_SHARED_PREFIX 2u

/*
 * Split-KV work split of the decode calls (their partition_tokens argument).
 *   > 0  fixed partitions of that many tokens (a multiple of 16): one wave per
 *        (sequence, kv head, q-head chunk, partition), states merged by length.
 *   0    library default: the balanced split when fixed partitions of the
 *        default length would need more than one round of resident waves (a
 *        mix of lengths then leaves the last round to a few long sequences),
 *        else those fixed partitions.
 *   PA_PARTITION_BALANCED  the balanced split: the blocks of all sequences,
 *        one after another, are cut into equal stretches, each read by one
 *        wave per kv head (and q-head chunk), so every wave gets the same
 *        work whatever the mix of lengths.  At most 512 sequences; several
 *        queries per sequence (pa_decode_multi) only on the matrix-core path
 *        (head_dim 128, q_per_seq x group >= 3); otherwise PA_ERR_SHAPE.
 * The split changes float32 rounding only: the online-softmax merge of
 * partial states is exact ("vLLM-Ascend 原理", §四 "ATB 算子").
 */
#define PA_PARTITION_BALANCED (-1)

/*
 * pa_kv_bytes_per_token -- K+V bytes one token occupies over all layers:
 * 2 * layers * kv_heads * head_dim * dtype_bytes ("vLLM-Ascend 原理", §2.1,
 * the KV size formula).  Pure host arithmetic; returns 0 if any argument is
 * not positive.
 */
uint64_t pa_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                               int32_t dtype_bytes);

/* pa_status_string -- static, never-NULL description of a status code
 * ("unknown status" for a value outside pa_status). */
const char* pa_status_string(pa_status status);

/*
 * pa_reshape_and_cache -- the cache write: store each new token's k and v in
 * its slot ("vLLM-Ascend 原理", §2.3 step 3 and §2.4 step 3: new k, v go into
 * the physical blocks named by the block table, 16 tokens per block).
 *
 *   key, value    [num_tokens][num_kv_heads][head_dim]            (read)
 *   k_cache,
 *   v_cache       [num_blocks][block_size][num_kv_heads][head_dim] (written)
 *   slot_mapping  int64 [num_tokens]; slot s -> block s / block_size,
 *                 offset s % block_size.  s < 0 marks a padding row and is
 *                 skipped; s >= num_blocks * block_size is skipped too.
 *
 * A bit copy: no conversion.  Slots must be distinct (two tokens writing one
 * slot leave either value).  num_tokens == 0 is a no-op returning PA_OK.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache,
                               void* v_cache, const int64_t* slot_mapping,
                               int64_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               pa_dtype dtype, hipStream_t stream);

/*
 * pa_copy_blocks -- copy whole physical blocks: block dst becomes a copy of
 * block src, K and V, every kv head.  This is the block copy behind a
 * copy-on-write fork of a shared prefix ("vLLM-Ascend 原理", §2.1: sequences
 * with the same prefix point at the same physical blocks and fork by
 * copy-on-write) and behind swapping ("vLLM学习整理", §三 "Preemption").
 *
 *   k_cache, v_cache  [num_blocks][block_size][num_kv_heads][head_dim] (read/written)
 *   block_pairs       int64 [num_pairs][2] = (src, dst), device memory.  A pair
 *                     with a negative or out-of-range entry, or src == dst, is
 *                     skipped.
 *
 * Destinations must be distinct and no destination may be the source of
 * another pair; otherwise the result depends on scheduling.  num_pairs == 0
 * is a no-op returning PA_OK.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                         int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                         hipStream_t stream);

/*
 * pa_decode_default_partition -- the split-KV partition length, in tokens, that
 * pa_decode uses when given partition_tokens == 0 and the default is fixed
 * partitions rather than the balanced split (a power of two >= 256).  It
 * depends only on host-known sizes: about max_blocks_per_seq * block_size / 8,
 * capped at 2048 tokens where decode runs on matrix cores (head_dim 128 and 3
 * or more q heads per kv head) and at 512 otherwise; 256 for invalid
 * arguments.  A partition covering max_blocks_per_seq * block_size tokens or
 * more means a single pass with no merge.  The online-softmax merge of partitions is exact
 * ("vLLM-Ascend 原理", §四 "ATB 算子": softmax statistics kept online), so the
 * choice changes only float32 rounding.
 */
int32_t pa_decode_default_partition(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_blocks_per_seq);

/*
 * pa_decode_split -- the split a single-query decode call (pa_decode,
 * pa_decode_fp8, pa_decode_noalloc) of this shape makes for partition_tokens:
 * its partition length in tokens, or PA_PARTITION_BALANCED for the balanced
 * split; 0 for invalid arguments.  Host arithmetic only.
 */
int32_t pa_decode_split(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int32_t partition_tokens);

/*
 * pa_decode_workspace_size -- bytes of float32 partial results the decode calls
 * (16-bit and FP8) need for this shape and split (partition_tokens as for
 * pa_decode), enough for either split that partition_tokens 0 may choose and,
 * where PA_DECODE_SHARED_PREFIX can take effect, for its sequence groups (their
 * shared runs' states and per-group block counts).  0 when every sequence fits
 * one partition.  Layout (internal to the library): per partial state a
 * running max, a running sum and head_dim accumulators.  Also 0 for a
 * block_size other than 16 or 32 or other invalid sizes.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t partition_tokens);

/*
 * pa_decode -- paged decode attention ("vLLM-Ascend 原理", §2.4 step 3: the
 * new position's q attends to the whole prefix, whose K/V are read block by
 * block through the block table; under GQA only the kv heads are read).
 *
 *   out           [num_seqs][num_q_heads][head_dim]                (written)
 *   q             [num_seqs][num_q_heads][head_dim]
 *   k_cache,
 *   v_cache       [num_blocks][block_size][num_kv_heads][head_dim]
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(seq_lens[b] / block_size) are never read.
 *   seq_lens      int32 [num_seqs]: cached tokens INCLUDING the current one
 *                 (its k/v already written by pa_reshape_and_cache).  0 gives
 *                 an all-zero output row; values above
 *                 max_blocks_per_seq * block_size are clamped to it.
 *   scale         softmax scale applied to q.k (natural-base softmax); must be
 *                 positive and finite.
 *   partition_tokens  split-KV work split: a partition length (multiple of
 *                 16), 0 for the library default or PA_PARTITION_BALANCED.
 *   flags         0, PA_DECODE_STREAM_KV, PA_DECODE_SHARED_PREFIX or both; other
 *                 bits give PA_ERR_UNSUPPORTED.
 *   workspace     device buffer of at least pa_decode_workspace_size() bytes
 *                 (may be NULL when that size is 0), 16-byte aligned.
 *
 * q head h reads kv head h / (num_q_heads / num_kv_heads); num_q_heads must be
 * a multiple of num_kv_heads, with at most 128 q heads per kv head (a wave
 * carries up to 16 of them; more run as several chunks, each reading the kv
 * head's K/V).  Slots past
 * seq_lens[b] inside the last block may hold any bits, NaN included; they
 * never reach the output.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                    float scale, pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_step -- one decode step: the cache write of each sequence's newest
 * token and pa_decode over the caches it leaves ("vLLM-Ascend 原理", §2.4 step 3:
 * the step stores the new k/v, then the new position's q attends to the whole
 * prefix).  The same as pa_reshape_and_cache with slot_mapping[b] = the slot of
 * position seq_lens[b] - 1 through block_tables, followed by pa_decode with the
 * same arguments, except that the decode kernels perform the write themselves:
 * the wave that reads a sequence's last block takes the newest row from
 * key / value rather than from the pool, scores it in one more step, and stores
 * it to its slot -- one kernel fewer per step (16-bit caches).
 *
 *   key, value    [num_seqs][num_kv_heads][head_dim], the dtype of q: the k and
 *                 v of each sequence's newest token (position seq_lens[b] - 1);
 *                 rows of sequences with seq_lens[b] = 0 are not read.
 *   the rest      as pa_decode; k_cache / v_cache are written.
 *
 * The pools afterwards equal those of the separate write bit for bit; a slot
 * whose table entry lies outside the pool is not written (as the cache write
 * skips it).  Outputs agree with the separate calls to the decode tolerance,
 * not bit for bit (the newest key joins the softmax in its own step).  With
 * PA_DECODE_SHARED_PREFIX taking effect, the write runs first as its own
 * kernel and the grouped decode follows (outputs then equal the separate calls
 * bit for bit).  Two sequences whose newest tokens name the same slot, or a
 * slot inside another sequence's context, are a caller error, as with the
 * separate write.  Errors: as pa_decode; PA_ERR_NULL_PTR for a missing
 * key / value, PA_ERR_ALIGNMENT for one not 16-byte aligned.
 */
pa_status pa_decode_step(void* out, const void* q, const void* key, const void* value, void* k_cache,
                         void* v_cache, const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks, float scale, pa_dtype dtype,
                         int32_t partition_tokens, uint32_t flags, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments minus the workspace, the same kernels
 * and the same results bit for bit.  The split-KV partial states go to a
 * static scratch array inside the library, PA_NOALLOC_SCRATCH_BYTES (64 MiB)
 * per GPU, held by every GPU the library runs on until the process ends.  The
 * call itself allocates nothing; on its first call on a device it looks up
 * that device's copy of the array (the device current on the calling
 * thread, which must be the stream's device).
 *
 * A shape whose partials need more than PA_NOALLOC_SCRATCH_BYTES
 * (pa_decode_workspace_size) gives PA_ERR_SCRATCH before anything is
 * enqueued; PA_ERR_HIP if the device or the array's address cannot be
 * queried.  All calls on one GPU share its scratch: calls that overlap in
 * time on one GPU (different streams, or host threads, without ordering
 * between them) race and give undefined results.  Calls ordered on a stream
 * are safe; nothing needs clearing between them.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                            float scale, pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                            hipStream_t stream);

/*
 * pa_decode_multi -- paged decode with several new queries per sequence, as
 * speculative decoding verifies its draft tokens: the target model scores the
 * k proposed tokens (and the last accepted one) in one pass, like a small
 * prefill ("vLLM-Ascend 原理", §四, the speculative-decoding paragraphs).  Each
 * K/V tile is read once for all q_per_seq queries of its sequence.
 *
 *   out, q        [num_seqs][q_per_seq][num_q_heads][head_dim]; query j of
 *                 sequence b sits at position seq_lens[b] - q_per_seq + j and
 *                 sees keys 0 .. seq_lens[b] - q_per_seq + j (causal among the
 *                 new tokens, whose k/v are already in the cache).  A query
 *                 whose position is negative gives an all-zero row.
 *   q_per_seq     1 .. PA_MAX_QUERIES_PER_SEQ (1 is exactly pa_decode).
 *   workspace     pa_decode_workspace_size(num_seqs * q_per_seq, ...) bytes.
 *   partition_tokens  0 picks a default: with q_per_seq > 1 on the matrix-core
 *                 kernel (head_dim 128, q_per_seq x group >= 3) the balanced
 *                 split, whose units carry the (query, head) columns of a kv
 *                 head, where its partial states fit the workspace size above;
 *                 else the single-query default partition, doubled (at most
 *                 2048 tokens) on the matrix-core kernel.  The workspace size
 *                 above, taken with partition_tokens 0, always suffices for it.
 *
 * Rejecting drafts needs no work here: the next step simply passes the
 * shorter seq_lens.  Every other argument and rule as for pa_decode.
 */
#define PA_MAX_QUERIES_PER_SEQ 16
pa_status pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t q_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int64_t num_blocks, float scale, pa_dtype dtype, int32_t partition_tokens,
                          uint32_t flags, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * pa_decode_partitions / pa_decode_merge -- the two phases of pa_decode, for
 * callers that schedule or time them separately.  Same arguments and
 * contract as pa_decode; the arguments the two calls share must be identical.
 * pa_decode_partitions writes the final output of every sequence one
 * partition (or one stretch of the balanced split) covers whole, and partial
 * states for the others; pa_decode_merge combines the partial states and, in
 * the balanced split, writes the zero rows of empty sequences (a no-op when
 * nothing was split).
 */
pa_status pa_decode_partitions(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, float scale, pa_dtype dtype,
                               int32_t partition_tokens, uint32_t flags, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
pa_status pa_decode_merge(void* out, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, pa_dtype dtype,
                          int32_t partition_tokens, const void* workspace,
                          size_t workspace_bytes, hipStream_t stream);
/*
 * pa_decode_partitions_step -- the first phase of pa_decode_step: the decode
 * partitions with the step's cache write inside them (key / value as for
 * pa_decode_step), followed by pa_decode_merge.  PA_DECODE_SHARED_PREFIX has
 * no effect here, as for pa_decode_partitions.
 */
pa_status pa_decode_partitions_step(void* out, const void* q, const void* key, const void* value,
                                    void* k_cache, void* v_cache, const int32_t* block_tables,
                                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                    pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_prefill_paged -- causal chunked prefill over the paged cache
 * ("vLLM-Ascend 原理", §2.3 step 3: position i's q dots keys 0..i under a
 * triangular mask, GQA heads sharing k/v; §2.4 on chunked prefill: a later
 * chunk reads the KV earlier chunks wrote).
 *
 *   out              [num_tokens][num_q_heads][head_dim]           (written)
 *   q                [num_tokens][num_q_heads][head_dim]; rows of sequence
 *                    b are query_start_loc[b] .. query_start_loc[b+1]-1.
 *   k_cache, v_cache as for pa_decode; the new tokens' k/v must already be
 *                    in the cache (pa_reshape_and_cache first).
 *   block_tables     int32 [num_seqs][max_blocks_per_seq]
 *   ctx_lens         int32 [num_seqs]: tokens cached BEFORE this chunk.  Row i
 *                    of sequence b sits at position ctx_lens[b] + i and sees
 *                    keys 0 .. ctx_lens[b] + i.
 *   query_start_loc  int32 [num_seqs + 1], non-decreasing, first entry 0,
 *                    last entry <= num_tokens.
 *   max_q_len        host-known upper bound of any sequence's row count
 *                    (sizes the grid; rows past it are not computed).
 *   scale            softmax scale, positive and finite.
 *
 * Rows owned by no sequence are left untouched.  head_dim must be 64 or 128;
 * the q-head group (num_q_heads / num_kv_heads) at most 128.
 */
pa_status pa_prefill_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* ctx_lens,
                           const int32_t* query_start_loc, int32_t num_seqs,
                           int64_t num_tokens, int32_t max_q_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                           pa_dtype dtype, hipStream_t stream);

/*
 * ------------------------------------------------------------------------
 * FP8 KV cache.  Each layer's per-head k and v are stored in 8 bits, which
 * halves the cache; they are quantised when written and dequantised inside
 * the attention kernels after the block-table lookup ("vLLM-Ascend 原理",
 * §四, the paragraph on KV-cache quantisation).
 *
 * Format: OCP 8-bit floating point E4M3 (bias 7, no infinities, S.1111.111 =
 * NaN, largest finite magnitude 448).  One float32 scale per (token, kv head)
 * row of head_dim elements:
 *     s = amax / 448   (amax = largest |x| of the row; s = 1 if amax == 0)
 *     code = e4m3(clamp(x / s, -448, 448)),  x / s rounded once in float32,
 *            the conversion rounding to nearest, ties to even
 *     value = decode(code) * s
 * Pools:
 *     k_cache, v_cache    uint8   [num_blocks][block_size][num_kv_heads][head_dim]
 *     k_scales, v_scales  float32 [num_blocks][num_kv_heads][block_size]
 * (the scales of one block and head are 64 contiguous bytes).  q, out, key and
 * value keep the 16-bit type `dtype`.  Inputs must be finite and, for the
 * attention calls, every scale of a live token a normal float32 (amax of
 * each row at least 448 * 2^-126); slots past a sequence's end may hold any
 * bits.  All pointers 16-byte aligned.
 * ------------------------------------------------------------------------
 */

/*
 * pa_reshape_and_cache_fp8 -- the cache write into an FP8 cache: quantise
 * each new token's k and v per kv head and store codes and scales in its slot
 * (codes at row s of the [num_blocks * block_size] view, scales at
 * [s / block_size][head][s % block_size]).  Slot conventions as for
 * pa_reshape_and_cache; key and value are [num_tokens][num_kv_heads][head_dim]
 * of `dtype`.  num_tokens == 0 is a no-op returning PA_OK; num_tokens *
 * num_kv_heads above 2^31 - 1 gives PA_ERR_SHAPE.
 */
pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                   void* v_cache, float* k_scales, float* v_scales,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, pa_dtype dtype, hipStream_t stream);

/*
 * pa_copy_blocks_fp8 -- pa_copy_blocks for an FP8 cache: block dst of the code
 * pools and of the scale pools becomes a copy of block src.  Same pair rules.
 */
pa_status pa_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                             const int64_t* block_pairs, int64_t num_pairs, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             hipStream_t stream);

/*
 * pa_decode_fp8 / pa_decode_partitions_fp8 -- pa_decode and its first phase
 * over an FP8 cache: k_cache / v_cache hold codes and k_scales / v_scales
 * their scales; every other argument, the workspace (pa_decode_workspace_size)
 * and the default partition are those of pa_decode.  The second phase of
 * pa_decode_partitions_fp8 is pa_decode_merge, unchanged.  Output: attention
 * over the dequantised K/V, accumulated in float32, rounded to `dtype`.
 */
pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scales, const float* v_scales, const int32_t* block_tables,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                        pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
pa_status pa_decode_partitions_fp8(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const float* k_scales,
                                   const float* v_scales, const int32_t* block_tables,
                                   const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, float scale, pa_dtype dtype,
                                   int32_t partition_tokens, uint32_t flags, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * pa_prefill_paged_fp8 -- pa_prefill_paged over an FP8 cache: k_cache /
 * v_cache hold codes and k_scales / v_scales their scales (the new tokens
 * written by pa_reshape_and_cache_fp8 first); every other argument and rule
 * as for pa_prefill_paged.  Output: causal attention over the dequantised K/V,
 * accumulated in float32, rounded to `dtype`.
 */
pa_status pa_prefill_paged_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scales, const float* v_scales,
                               const int32_t* block_tables, const int32_t* ctx_lens,
                               const int32_t* query_start_loc, int32_t num_seqs, int64_t num_tokens,
                               int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, float scale, pa_dtype dtype, hipStream_t stream);

/*
 * pa_debug_bounds -- the index checks of a debug build.  Device-resident
 * indices are not validated by the normal library (see "Errors" above).  A
 * library built with PA_DEBUG_BOUNDS defined (libpa_debug.so) launches, ahead
 * of each call's own kernels, a check of the indices that call is about to
 * use, which sets bits of a device word ("Hardware abstraction and
 * portability", §六: asynchronous errors surface at synchronisation points):
 *
 *   PA_DEBUG_BLOCK_ID     a block-table entry of a block some sequence uses
 *                         (its first ceil(seq_len / 16) blocks, or ctx + chunk
 *                         in prefill) is outside [0, num_blocks), or a copy
 *                         pair names a block >= num_blocks;
 *   PA_DEBUG_SEQ_LEN      a seq_len (or ctx_len + chunk length) is negative or
 *                         larger than the table row can name;
 *   PA_DEBUG_SLOT         a cache-write slot is >= num_blocks * block_size;
 *   PA_DEBUG_QUERY_RANGE  query_start_loc is not non-decreasing within
 *                         [0, num_tokens], or a chunk is longer than max_q_len.
 *
 * Negative slots and copy pairs stay legal padding.  pa_debug_bounds waits for
 * `stream`, stores the bits set since the last clear in *word and, if `clear`
 * is non-zero, clears them.  It synchronises, so it is the one call that
 * cannot be captured in a graph.  In the normal library it returns
 * PA_ERR_UNSUPPORTED and does nothing.  The word is per device and shared by
 * every caller of the library on it.
 */
#define PA_DEBUG_BLOCK_ID 1u
#define PA_DEBUG_SEQ_LEN 2u
#define PA_DEBUG_SLOT 4u
#define PA_DEBUG_QUERY_RANGE 8u
pa_status pa_debug_bounds(uint32_t* word, int32_t clear, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
