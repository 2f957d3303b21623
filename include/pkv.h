/*
 * pkv — paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Every pointer argument is device memory owned by the
 * caller unless a comment says "host"; the library allocates no device
 * memory, and the only handles it keeps between calls are, per device, the
 * side stream and two events that pkv_paged_mixed creates on first use
 * (default priority, kept until the process ends).  Every call validates its
 * scalar arguments on the host, returns a status code (nothing is thrown
 * across the ABI), and on PKV_OK has queued its kernels asynchronously on
 * `stream`.  On any other status nothing was launched and pkv_last_error()
 * describes the problem.
 *
 * Pages cited (titles as published):
 *   [T] "'안녕하세요 반갑습니다'로 배우는 vLLM — KV Cache와 PagedAttention 완전 해부"
 *       (hrletsgo.me)
 *   [W] "[vLLM] PagedAttention: OS 페이징 기법으로 KV 캐시를 관리하는 방법"
 *       (blog.secrett2633.cloud)
 *   [R] "vLLM: LLM 서빙 메모리 최적화의 교과서" (velog.io/@doogunwo)
 *   [S] "Sparse Computation and Memory Management for Efficient LLM Inference"
 *       (pyy0715.github.io)
 *
 * ----------------------------------------------------------------------------
 * The block pool ([T] step 5; [R] section "02. Idea: PagedAttention"; [S]
 * section "PagedAttention: Borrowing from Operating Systems"): device memory
 * cut into fixed-size blocks of `block_size` token slots.  A request's block
 * table maps its logical block i to any physical block; a token's slot is
 *
 *     slot = physical_block * block_size + offset_in_block.
 *
 * Layout in HBM (this library's choice; the pages fix only "blocks of B
 * tokens"):
 *
 *   k_pool  [num_blocks][num_kv_heads][head_dim/X][block_size][X],
 *           X = 64 bytes / element size (32 fp16/bf16 values, 16 fp32
 *           values): each key row is cut into 64-byte pieces and a block's
 *           pieces of one dimension range sit together, so 16 tokens x 64
 *           bytes of a (block, head) key tile are one contiguous KiB; element
 *           (block, head, offset, e) is at
 *           (((block*H + head)*(d/X) + e/X)*B + offset)*X + e%X;
 *   v_pool  [num_blocks][num_kv_heads][head_dim][block_size]
 *           a (block, head) value tile is d x B, dimension-major, contiguous,
 *           so the B tokens of one value dimension are adjacent: the operand
 *           shape that the P.V matrix-core products read directly.
 *
 * A (block, head) tile of either pool is B*d contiguous elements.
 * q, out, key and value rows are [tokens][heads][head_dim], contiguous.
 * Query/output and cache share one dtype, except over an 8-bit (E4M3)
 * cache, whose queries, outputs and key/value rows are f16 or bf16.
 * Supported: dtype f32/f16/bf16/fp8-e4m3, head_dim 64 or 128, block_size 8,
 * 16 or 32.  Base pointers must be 16-byte aligned.
 *
 * Device-side contract (not checked on the device; pkv_validate_host checks
 * it on host copies): block ids in the first ceil(L/B) table entries of a
 * sequence lie in [0, num_blocks); 1 <= L <= max_blocks_per_seq * block_size;
 * L <= max_context_len; no two tokens of one scatter share a slot.  The
 * kernels never touch memory outside the pool for a block id out of range
 * (that block is skipped, or with block_size 8 read as block 0 by decode)
 * and clamp lengths to the table, so a broken contract gives wrong numbers,
 * not a fault.
 * ----------------------------------------------------------------------------
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* PKV_FP8_E4M3 is a cache storage type only (OCP FP8 E4M3: 4 exponent bits,
 * bias 7, 3 mantissa bits, S.1111.111 = NaN, no infinities, |x| <= 448). */
typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = 1,     /* null pointer, bad size, misalignment, Hq % Hkv != 0, ... */
  PKV_ERR_UNSUPPORTED = 2, /* a valid request the library has no kernel for */
  PKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  PKV_ERR_HIP = 4          /* a HIP launch error (message from the runtime) */
} pkv_status;

/*
 * Describes caller-owned device memory of one layer's cache.
 *
 * An 8-bit cache ([W] section "PagedAttention 커널: 비연속 메모리 접근":
 * write_to_paged_cache passes kv_cache_dtype, k_scale and v_scale to
 * reshape_and_cache): dtype PKV_FP8_E4M3, model_dtype PKV_F16 or PKV_BF16.
 * A key element x is stored as the E4M3 code of the fp32 quotient x /
 * k_scale (nearest, ties to even; magnitudes >= 448 saturate to 448; NaN
 * stays NaN) and read back as code * k_scale; values likewise with v_scale.
 * Otherwise model_dtype equals dtype and the scales are ignored.
 */
typedef struct {
  void *k_pool;          /* [num_blocks][num_kv_heads][head_dim/X][block_size][X] */
  void *v_pool;          /* [num_blocks][num_kv_heads][head_dim][block_size] */
  int64_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;    /* 8, 16 or 32 */
  int32_t head_dim;      /* 64 or 128 */
  int32_t dtype;         /* pkv_dtype of the pools */
  int32_t model_dtype;   /* pkv_dtype of key/value inputs, queries and outputs */
  float k_scale;         /* 8-bit cache only: positive, finite */
  float v_scale;
} pkv_cache;

/*
 * Slot scatter, "reshape_and_cache".  [W] section "PagedAttention 커널:
 * 비연속 메모리 접근": write_to_paged_cache passes the new tokens' key and
 * value and their slot_mapping to reshape_and_cache, which stores each token
 * in the slot named for it; [T] step 6: decode stores the new token's K/V in
 * the next free slot of the request's last block.
 *
 *   key, value     [num_tokens][num_kv_heads][head_dim], model_dtype
 *   slot_mapping   int64 [num_tokens]; a negative slot skips that token
 *                  (padding); slots >= num_blocks * block_size are skipped too
 *
 * Bit-exact copy into a 16/32-bit cache; into an 8-bit cache each element
 * is quantised as described at pkv_cache.  Duplicate non-negative slots are
 * a caller error with no defined winner.  num_tokens == 0 is a no-op.
 */
pkv_status pkv_reshape_and_cache(const pkv_cache *cache, const void *key, const void *value,
                                 const int64_t *slot_mapping, int64_t num_tokens,
                                 hipStream_t stream);

/*
 * Whole-block copy for copy-on-write.  [S] section "Copy-on-Write": before a
 * sequence writes into a block whose reference count is above one, the block
 * is copied to a new physical block (fused_block_copy) and the sequence's
 * table is repointed; [T] step 9 (shared prompt blocks).  The decision and
 * the table update are the caller's; this call copies the K and V tiles of
 * every head for each pair.
 *
 *   src_dst  int32 [num_pairs][2] = (src, dst); every dst distinct and not a
 *            src of any pair (copies are unordered).  Pairs with an id out of
 *            range are skipped.  num_pairs == 0 is a no-op.
 */
pkv_status pkv_copy_blocks(const pkv_cache *cache, const int32_t *src_dst, int64_t num_pairs,
                           hipStream_t stream);

/* partition_size value: let the library split the work (see pkv_paged_decode). */
#define PKV_PARTITION_AUTO (-1)

/*
 * Workspace bytes pkv_paged_decode needs for a call with these arguments (0
 * when it needs none: partition_size 0, or every sequence fits one
 * partition).  With PKV_PARTITION_AUTO the size depends on how many
 * workgroups the current device keeps resident, so query it on the device
 * the call will run on.  Returns 0 for invalid arguments (the decode call
 * then reports them).
 */
size_t pkv_decode_workspace_bytes(const pkv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition_size);

/*
 * Paged decode attention: one new query per sequence over its whole cache.
 * [R] section "01. Problem Definition": o_i = sum_{j<=i} softmax_j(q_i.k_j /
 * sqrt(d)) v_j; eq. (4) of the same section 02 and [S] section "Block-level
 * Attention Formulation": the same result computed block by block; [T]
 * "부록": walk the blocks through the block table, load the keys, compute
 * partial scores, update a running softmax normaliser, accumulate the
 * weighted values.  Query head hq reads KV head hq / (Hq / Hkv) (grouped
 * heads, [S] section "The Hidden Waste of KV Cache").
 *
 *   out, q            [num_seqs][num_q_heads][head_dim]; q in model_dtype
 *   out_dtype         model_dtype (out rounded once, to nearest even, from
 *                     the fp32 result) or PKV_F32 (the fp32 result itself)
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]
 *   context_lens      int32 [num_seqs]; L_s counts every cached token,
 *                     including the new one (scatter it first); L_s >= 1
 *   max_context_len   host bound on every L_s (sizes the launch)
 *   scale             the softmax scale, normally 1/sqrt(head_dim) in fp32;
 *                     must be positive and finite
 *   partition_size    0: one workgroup pass over each whole sequence;
 *                     a positive multiple of block_size: each sequence is
 *                     split into partitions of that many tokens starting at
 *                     position 0, each partition writes (running max,
 *                     denominator, weighted sum) to the workspace and a
 *                     reduce kernel combines them (block-wise aggregation of
 *                     partial results, [R] section 02 "Aggregation");
 *                     PKV_PARTITION_AUTO: the blocks of all (sequence, head)
 *                     pairs are dealt out in equal contiguous shares, one
 *                     per resident workgroup, and pairs cut between shares
 *                     are combined the same way (up to 8192 sequences; more
 *                     run as partition_size 0)
 *   workspace         device scratch of >= pkv_decode_workspace_bytes(...)
 *                     bytes, 16-byte aligned; may be NULL when that is 0
 *
 * Grouped heads (num_q_heads > num_kv_heads) over an f16/bf16/8-bit cache
 * run on the matrix cores with the group's queries stacked into one tile
 * (group size <= 16; 8-bit key codes are widened to the model dtype and
 * value codes to fp16 as they arrive, both exactly); fp32 caches and single
 * heads run the wavefront dot-product kernel, over an fp32 cache with each
 * score and weight exponent formed in fp64.
 */
pkv_status pkv_paged_decode(const pkv_cache *cache, void *out, int32_t out_dtype, const void *q,
                            int32_t num_q_heads,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, int32_t num_seqs,
                            int32_t max_context_len, float scale, int32_t partition_size,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_paged_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The call allocates nothing; the split
 * partials go to a static device array of 64 MiB that the library holds on
 * every GPU it runs on until the process ends.  A call that would need more
 * (pkv_decode_workspace_bytes above 64 MiB) returns PKV_ERR_WORKSPACE and
 * launches nothing.  Every call on one GPU shares that GPU's array; nothing
 * in it has to start at zero (each call writes every partial it later
 * reads), but calls that may run at the same time on one GPU (other streams
 * or threads) race on it and must be serialised by the caller.  Arguments
 * and result as for pkv_paged_decode.
 */
pkv_status pkv_paged_decode_noalloc(const pkv_cache *cache, void *out, int32_t out_dtype,
                                    const void *q, int32_t num_q_heads,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t num_seqs,
                                    int32_t max_context_len, float scale, int32_t partition_size,
                                    hipStream_t stream);

/*
 * Sliding-window decode.  [W] section "블록 할당: allocate_slots" (under
 * "KVCacheManager: 블록 단위 할당의 중심"): before a step's allocation the
 * cache manager releases the blocks that fell out of the sliding window, as
 * an OS pages out frames, then allocates new ones.  Reading
 * taken: the query at position L-1 attends to positions max(0, L - W) .. L-1
 * (the W most recent tokens, itself included); a block holding only earlier
 * positions may have been released, so its table entry may name any block
 * or none, and is never read.  Everything else as for pkv_paged_decode,
 * which is this call with sliding_window 0 (no window); the same workspace
 * size applies.
 *
 *   sliding_window    W in tokens, >= 0 (0: the whole context)
 */
pkv_status pkv_paged_decode_window(const pkv_cache *cache, void *out, int32_t out_dtype,
                                   const void *q, int32_t num_q_heads,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, int32_t num_seqs,
                                   int32_t max_context_len, int32_t sliding_window, float scale,
                                   int32_t partition_size, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Append and attend in one call: for every sequence, the new token's key and
 * value rows are written into the cache at the slot its block table gives
 * for position L-1 (physical block table[s][(L-1)/B], offset (L-1) mod B),
 * and the decode of pkv_paged_decode_window runs over the cache with that
 * token in place.  The result, cache and output, is bit for bit that of
 * pkv_reshape_and_cache with those slots followed by
 * pkv_paged_decode_window: [T] step 6 (decode stores the new token's K/V,
 * then attends).  The decode kernel takes the new token from the input rows
 * instead of the cache, and the short kernel that follows it (the split
 * reduce, launched for this call also when nothing is split) stores the
 * rows, which saves the scatter's launch and keeps stores out of the decode
 * kernel's read stream.
 *
 *   key, value        [num_seqs][num_kv_heads][head_dim], model dtype
 *                     (8-bit cache: quantised with k_scale / v_scale as the
 *                     scatter does)
 *   other arguments   as for pkv_paged_decode_window (same workspace size)
 * The block holding position L-1 must belong to sequence s alone (copy on
 * write done), as for any append.  A table entry for position L-1 that is
 * out of range receives nothing.
 */
pkv_status pkv_paged_decode_append(const pkv_cache *cache, const void *key, const void *value,
                                   void *out, int32_t out_dtype, const void *q,
                                   int32_t num_q_heads, const int32_t *block_tables,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   int32_t num_seqs, int32_t max_context_len,
                                   int32_t sliding_window, float scale, int32_t partition_size,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Causal chunked prefill over the paged cache.  [S] section "Prefill-Decode
 * Disaggregation": a long prompt is processed in chunks over several steps;
 * [T] step 6 and [R] section 01: prefill processes all prompt tokens at once
 * as a matrix-matrix product.  Sequence s owns query rows
 * query_start_loc[s] .. query_start_loc[s+1]-1, the last qlen_s of its
 * context_lens[s] cached tokens (scatter the chunk's K/V first): row i sits
 * at position context_lens[s] - qlen_s + i and attends to positions 0..that
 * position.  Blocks may be shared between sequences (prefix sharing).
 *
 *   out, q            [total_rows][num_q_heads][head_dim] in the model dtype:
 *                     an f16 or bf16 cache's own, or an 8-bit cache's
 *                     model_dtype ([W] section "PagedAttention 커널: 비연속
 *                     메모리 접근": the cache write's kv_cache_dtype, k_scale
 *                     and v_scale serve every later read; an element's value
 *                     is code * scale).  out_dtype as for pkv_paged_decode
 *                     (fp32 cache: PKV_ERR_UNSUPPORTED)
 *   query_start_loc   int32 [num_seqs + 1], non-decreasing, starts at 0
 *   context_lens      int32 [num_seqs], >= qlen_s, >= 1
 *   max_query_len     host bound on every qlen_s
 *   max_context_len   host bound on every context_lens[s]
 */
pkv_status pkv_paged_prefill(const pkv_cache *cache, void *out, int32_t out_dtype, const void *q,
                             int32_t num_q_heads, const int32_t *query_start_loc,
                             const int32_t *context_lens, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, int32_t num_seqs, int32_t max_query_len,
                             int32_t max_context_len, float scale, hipStream_t stream);

/*
 * One step's attention over a batch that mixes decode rows and prefill-chunk
 * rows.  [S] section "Prefill-Decode Disaggregation": on a single GPU a long
 * prompt is cut into chunks, and every step batches one chunk together with
 * the decode tokens of the other requests.  The result is exactly that of
 * pkv_paged_prefill over all num_seqs sequences (a decode row is a chunk of
 * one row at position context_lens[s] - 1), computed by two kernels that run
 * at once: the decode kernel of pkv_paged_decode over the decode sequences
 * and the prefill kernel over the chunk sequences.  The decode kernel is
 * enqueued on a stream the library owns, forked from and joined back into
 * `stream` with two events; the reduce of its split rows then runs on
 * `stream`, so work enqueued on `stream` after this call sees both parts
 * finished.  The library keeps that stream and its events (default
 * priority) for each (device, caller stream) pair it has served, until the
 * process ends: the one call of this interface that holds handles, so that
 * the two parts can run at once on one caller stream.
 *
 *   sequences 0 .. num_decode_seqs-1   decode: one query row each, row s
 *                     (query_start_loc[s] == s for s <= num_decode_seqs; the
 *                     decode part does not read query_start_loc)
 *   sequences num_decode_seqs .. num_seqs-1   chunks, as for pkv_paged_prefill
 *                     (query_start_loc holds absolute row numbers)
 *   out, q            [total_rows][num_q_heads][head_dim], model dtype; out
 *                     also PKV_F32.  A cache with chunk sequences must be f16,
 *                     bf16 or 8-bit (fp32: PKV_ERR_UNSUPPORTED); decode-only
 *                     calls take every cache pkv_paged_decode takes
 *   partition_size, workspace   as for pkv_paged_decode over the decode
 *                     sequences: pkv_decode_workspace_bytes(cache,
 *                     num_decode_seqs, num_q_heads, max_context_len,
 *                     partition_size) bytes
 *   max_query_len     host bound on the chunk lengths; max_context_len a host
 *                     bound on every context length
 * Host-side locking serialises concurrent calls on one caller stream while
 * they enqueue; a graph capture on `stream` takes in its side stream only.
 */
pkv_status pkv_paged_mixed(const pkv_cache *cache, void *out, int32_t out_dtype, const void *q,
                           int32_t num_q_heads, const int32_t *query_start_loc,
                           const int32_t *context_lens, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_decode_seqs,
                           int32_t max_query_len, int32_t max_context_len, float scale,
                           int32_t partition_size, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Gather with the kernels' own address arithmetic: the contiguous K and V of
 * every sequence, back to back, token-major.  [T] step 5: the block table
 * maps a request's logical blocks, in order, to physical blocks, so logical
 * position j of sequence s is slot table[s][j / B] * B + j mod B; this call
 * writes those slots out in logical order, the contiguous cache a
 * non-paged system would hold.  Positions past context_lens[s] are not
 * written; a table entry out of range leaves its rows unwritten.
 *
 *   k_out, v_out      [sum_s L_s][num_kv_heads][head_dim], cache dtype (the
 *                     stored codes for an 8-bit cache)
 *   cu_context_lens   int32 [num_seqs + 1], prefix sums of context_lens
 */
pkv_status pkv_gather_kv(const pkv_cache *cache, void *k_out, void *v_out,
                         const int32_t *block_tables, int32_t max_blocks_per_seq,
                         const int32_t *context_lens, const int32_t *cu_context_lens,
                         int32_t num_seqs, int32_t max_context_len, hipStream_t stream);

/*
 * Host-side check of the device-side contract, on HOST copies of the
 * integer inputs (any pointer may be NULL with its count 0 to skip that
 * part): slots in range and unique, every L in [1, max_blocks*B] and, when
 * max_context_len > 0, L <= max_context_len, every table entry a sequence
 * uses in [0, num_blocks).  The slot rule is the one the scatter passage
 * defines ([W] section "PagedAttention 커널: 비연속 메모리 접근": each
 * token's slot_mapping entry names one slot); the table rule is [T] step 5
 * (a block table entry names a physical block of the pool).  Returns PKV_OK
 * or PKV_ERR_INVALID with pkv_last_error() naming the first violation.
 * Reads only the host arrays; launches nothing.
 */
pkv_status pkv_validate_host(const int64_t *slot_mapping, int64_t num_tokens,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t num_seqs, int64_t num_blocks,
                             int32_t block_size, int32_t max_context_len);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *pkv_last_error(void);

/* Library version string. */
const char *pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
