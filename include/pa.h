/*
 * pa.h -- paged-KV decode attention for MI355X (gfx950): the C ABI of libpa.so.
 *
 * What is computed (by page title and section):
 *   "19.2 KV Cache 系统化管理" §19.2.2 and §19.2.3: the keys and values of all
 *   requests live in two pools of fixed-size physical blocks, each shaped
 *   [num_blocks, block_size, num_kv_heads, head_dim]; a request's block
 *   table maps its logical block i (tokens i*block_size ...) to a physical
 *   block; attention of a query walks the request's blocks in order and
 *   folds them into a running maximum, running sum and running weighted sum
 *   (online softmax), then divides -- which equals ordinary softmax
 *   attention over the request's tokens.
 *   "LLM 推理引擎的内存管理与调度" §3: the kernel finds a token through the
 *   block table (logical block -> physical block) plus its in-block offset.
 *   §4 of that page and §19.2.2 above: blocks are shared between requests
 *   with reference counts and copied on the first diverging write.
 *   §8 of that page: a long prompt is processed in chunks whose query tokens
 *   attend to the cached context and, causally, to each other.
 *
 * Conventions shared by every call.
 *   - Device pointers name caller-owned device memory (hipMalloc or a torch
 *     tensor); arrays are dense and row-major with the shapes given below.
 *     The library never allocates or frees device memory, never
 *     synchronizes and never reads device memory on the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls are asynchronous and ordered on that stream.
 *   - Every call returns a pa_status; on anything but PA_OK,
 *     pa_last_error() returns a message for the calling thread and no
 *     kernel was launched (PA_ERR_HIP: the launch itself failed).
 *   - Host-side arguments (sizes, null pointers, supported shapes) are
 *     validated.  Device-side contents are the caller's contract: block-table
 *     entries of the logical blocks a sequence uses must lie in
 *     [0, num_blocks) and seq_lens in [0, max_blocks_per_seq*block_size].
 *     Violations give unspecified results, but the kernels clamp every index
 *     they derive from device data, so no access leaves the arrays passed.
 *   - Supported shapes: dtype PA_F32, PA_BF16 or PA_FP8; head_dim 32, 64,
 *     128 or 256 (PA_FP8: 64, 128 or 256); block_size a power of two from 1
 *     to 256; num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 *   - Softmax scores are scale * dot(q, k) with a finite scale > 0; every
 *     workload passes 1/sqrt(head_dim), the value the pages use.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,    /* null pointer, bad size, inconsistent shapes */
  PA_ERR_UNSUPPORTED = 2,    /* valid but not built: dtype/head_dim/GQA ratio */
  PA_ERR_NO_FREE_BLOCKS = 3, /* the pool's free list cannot cover the request */
  PA_ERR_HIP = 4,            /* a HIP runtime call or kernel launch failed */
  PA_ERR_NOT_FOUND = 5       /* unknown sequence handle */
} pa_status;

/* Pool element types.  PA_FP8: e4m3 codes (1 byte: sign, 4 exponent bits of
 * bias 7, 3 mantissa bits; largest finite 448; 0x7F/0xFF are NaN) with one
 * float32 scale per (token, KV head) in separate scale pools
 * [num_blocks, num_kv_heads, block_size] (the rows of one head contiguous);
 * the stored value is code * scale.
 * Queries and outputs of fp8 pools are bfloat16. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8 = 2 } pa_dtype;

/* Shape of the two KV pools (K and V share it): [num_blocks, block_size,
 * num_kv_heads, head_dim] elements of `dtype`.  "19.2 KV Cache 系统化管理"
 * §19.2.3 gives this layout for its PhysicalBlockPool. */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pa_dtype */
} pa_kv_layout;

/* Message describing the last non-OK status returned on this thread. */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

/* ------------------------------------------------------------------------ */
/* Device calls                                                              */
/* ------------------------------------------------------------------------ */

/* Cache write ("19.2 KV Cache 系统化管理" §19.2.3, write_slot/append_token):
 * for every token t with slot s = slot_mapping[t] >= 0,
 *   k_pool[s / block_size, s % block_size, :, :] = k_new[t, :, :]   (and V).
 *   k_new, v_new : [num_tokens, num_kv_heads, head_dim], pool dtype
 *   slot_mapping : device int32 [num_tokens]; s = physical*block_size+offset;
 *                  negative = skip (padding); s >= num_blocks*block_size is
 *                  skipped as well.
 * Two tokens with the same slot in one call: which one lands is unspecified.
 * num_tokens == 0 is a no-op. */
pa_status pa_kv_write(const pa_kv_layout* layout, void* k_pool, void* v_pool,
                      const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/* Whole-block copies, the copy step of copy-on-write ("19.2 KV Cache
 * 系统化管理" §19.2.2): for every pair i, pool[dst_i] = pool[src_i] for K and V.
 *   pairs : device int32 [num_pairs, 2] as (src, dst).
 * Destinations must be distinct and must not be sources in the same call
 * (the block pool never produces such pairs); out-of-range ids are skipped. */
pa_status pa_copy_blocks(const pa_kv_layout* layout, void* k_pool, void* v_pool,
                         const int32_t* pairs, int32_t num_pairs, void* stream);

/* Paged decode ("19.2 KV Cache 系统化管理" §19.2.3, paged_attention): one
 * query token per sequence, at position seq_len-1, attending to keys
 * 0 .. seq_len-1 of its own table; returns the final output in one call.
 *   q, out       : [num_seqs, num_q_heads, head_dim], pool dtype; query head h
 *                  reads KV head h / (num_q_heads/num_kv_heads)
 *   block_tables : device int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens     : device int32 [num_seqs] (tokens in the cache, including
 *                  this step's token); seq_len 0 gives a zero row
 *   workspace    : NULL, or caller-owned device memory of workspace_bytes >=
 *                  pa_decode_workspace_size(...), 256-byte aligned.  With a
 *                  workspace the batch's work is split into equal slices,
 *                  one per workgroup the device holds at once (balanced over
 *                  uneven lengths; queries cut by a slice boundary are merged
 *                  by a second kernel in the same call).  Without one, each
 *                  (sequence, KV-head group) is one workgroup.  Calls sharing
 *                  a workspace must be ordered on one stream.
 * Accumulation is fp32; bf16 outputs are rounded to nearest even. */
pa_status pa_decode(const pa_kv_layout* layout, void* out, const void* q,
                    const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                    float scale, void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, and the same balanced decode, whose
 * workspace is a library-owned device array of 8 MiB per device (held until
 * the process ends).  The call itself allocates nothing.  The batch is cut
 * into as many slices as the device holds workgroups at once, or as many as
 * fit in the 8 MiB when fewer do (the same result, less parallel); sizes of
 * which even one slice does not fit (num_q_heads * head_dim beyond about
 * 8 Mi elements / 8) return PA_ERR_UNSUPPORTED; batches the balanced path
 * does not take (more than 4096 sequences) run the single-pass kernels,
 * which need no scratch.  Every call on one device
 * shares that device's array: calls that overlap in time on one device (on
 * different streams, or from different threads) race and must not be
 * issued. */
pa_status pa_decode_noalloc(const pa_kv_layout* layout, void* out, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            float scale, void* stream);

/* Bytes of workspace pa_decode uses for these sizes on the current device
 * (0: the balanced path does not apply, e.g. more than 4096 sequences, and
 * the workspace is ignored). */
pa_status pa_decode_workspace_size(const pa_kv_layout* layout, int32_t num_seqs,
                                   int32_t num_q_heads, size_t* bytes);

/* FP8 KV cache ("19.2 KV Cache 系统化管理" §19.2.4, KV Cache 量化压缩: every
 * token's K and V vectors are scaled and quantized on their own, and
 * dequantized by multiplying the scale back; the page's formula is lost, the
 * reading here is symmetric absmax).  layout->dtype must be PA_FP8; k_pool
 * and v_pool hold e4m3 codes [num_blocks, block_size, num_kv_heads,
 * head_dim], k_scale and v_scale float32 [num_blocks, num_kv_heads,
 * block_size] (the scale of row r of block b for head h at (b, h, r)), all
 * caller-owned device memory.
 *
 * Quantizing cache write: for every token t with slot s = slot_mapping[t]
 * in [0, num_blocks*block_size) and every KV head, the row x (head_dim
 * values of k_new / v_new, bfloat16 [num_tokens, num_kv_heads, head_dim])
 * gets scale = max|x| / 448 and codes e4m3(x / scale) (float32 division,
 * clamped to +-448, nearest even; scale 0 and zero codes for a zero row),
 * stored at row s of the pools.  Other slots are skipped. */
pa_status pa_kv_write_fp8(const pa_kv_layout* layout, void* k_pool, void* v_pool,
                          float* k_scale, float* v_scale, const void* k_new, const void* v_new,
                          const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/* Paged decode over fp8 pools: as pa_decode, with key and value rows read as
 * code * scale.  q and out are bfloat16 [num_seqs, num_q_heads, head_dim];
 * the workspace is sized by pa_decode_workspace_size with the same layout. */
pa_status pa_decode_fp8(const pa_kv_layout* layout, void* out, const void* q,
                        const void* k_pool, const void* v_pool, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_q_heads, float scale, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Block swap between two pools ("LLM 推理引擎的内存管理与调度" §9 and
 * "19.2 KV Cache 系统化管理" §19.2.6: a preempted request's KV blocks move to
 * CPU memory and come back when HBM has room).  For every pair i,
 * dst_pool[dst_i] = src_pool[src_i], K and V, whole blocks.
 *   dst_layout : shape and dtype of the destination pools; the source pools
 *                have the same block shape and dtype and src_num_blocks
 *                blocks
 *   dst_k/dst_v, src_k/src_v : device memory or pinned host memory (e.g.
 *                hipHostMalloc), which the GPU accesses through the same
 *                pointers: swap-out has host destinations, swap-in host
 *                sources; the copy runs on the GPU and is bound by the host
 *                link
 *   pairs      : int32 [num_pairs, 2] as (src, dst), device or pinned host
 *                memory; pairs with an id out of range are skipped
 * Destinations must be distinct.  For fp8 pools swap the scale pools too,
 * with the same pairs and a layout of head_dim 1 and dtype PA_F32. */
pa_status pa_swap_blocks(const pa_kv_layout* dst_layout, void* dst_k, void* dst_v,
                         const void* src_k, const void* src_v, int32_t src_num_blocks,
                         const int32_t* pairs, int32_t num_pairs, void* stream);

/* Copy-on-write of fp8 pools: as pa_copy_blocks, for the codes and the
 * scales of every (src, dst) pair. */
pa_status pa_copy_blocks_fp8(const pa_kv_layout* layout, void* k_pool, void* v_pool,
                             float* k_scale, float* v_scale, const int32_t* pairs,
                             int32_t num_pairs, void* stream);

/* Split-sequence paged attention.  The first pass summarises the keys of
 * every query by partitions; the second (pa_reduce) merges the summaries.
 * Both share one caller-owned device workspace, sized and laid out by
 * pa_split_workspace_layout:
 *   part_o   at part_o_offset   fp32 [num_q_tokens, num_q_heads, max_partitions, head_dim]
 *   part_lse at part_lse_offset fp32 [num_q_tokens, num_q_heads, max_partitions]
 *   control  at control_offset  256 bytes of work-queue counters
 * Entry (j, h, p) of a partition that exists for query j is
 *   part_o   = softmax-weighted mean of the partition's values
 *   part_lse = log(sum over its keys of exp(scale*q.k))   (natural log)
 * -- the running max / running sum state of the pages' online softmax
 * ("19.2 KV Cache 系统化管理" §19.2.3) with one partition as the unit.  The
 * control block must hold zeros before the first pa_decode_split on a
 * workspace (allocate it zeroed, e.g. hipMemset once); every call leaves it
 * zeroed again.  Calls sharing a workspace must be ordered on one stream. */
typedef struct {
  size_t part_o_offset;
  size_t part_lse_offset;
  size_t control_offset;
  size_t total_bytes; /* workspace bytes; offsets are 256-byte aligned */
} pa_split_layout;

pa_status pa_split_workspace_layout(int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_partitions, pa_split_layout* layout);
/* total_bytes of the same layout, or 0 if a size is out of range. */
size_t pa_split_workspace_bytes(int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_partitions);

/* First pass.  A sequence with one query token (a decode step) has its keys
 * 0 .. seq_len-1 cut into partitions of `partition_size` tokens (partition p
 * = keys [p*P, min((p+1)*P, seq_len)), ceil(seq_len/P) of them).  A
 * sequence with several query tokens holds a chunk of a prefill ("LLM 推理引擎
 * 的内存管理与调度" §8): its query tokens are its last q_len tokens, query i
 * sits at position seq_len - q_len + i and sees keys 0 .. position (causal).
 * Each of its queries has two partitions, keys [0, h) and [h, position],
 * split at h = 32 * floor(ceil(ctx / 32) / 2) with ctx = seq_len - q_len
 * (half the context cached before the chunk, in whole 32-key tiles), or
 * one partition with all its keys when h is 0.  Only existing partitions are
 * written.
 *   workspace    : device memory of workspace_bytes >= total_bytes of
 *                  pa_split_workspace_layout(num_q_tokens, num_q_heads,
 *                  head_dim, max_partitions), 256-byte aligned
 *   q            : [num_q_tokens, num_q_heads, head_dim], pool dtype
 *   cu_q_lens    : device int32 [num_seqs+1] prefix sums of query tokens per
 *                  sequence, or NULL when each sequence has exactly one (then
 *                  num_q_tokens == num_seqs)
 * One launch runs a work list that mixes decode partitions (vector units) and
 * prefill tiles (bf16 pools, head_dim <= 128: 128 (token, head) rows x one
 * partition per tile on the matrix cores with v_mfma_f32_32x32x16_bf16,
 * probabilities rounded to bf16 for the P V product; other pools: vector
 * units), drained by persistent workgroups through the work-queue counters
 * of the workspace's control block.
 * Requires partition_size % block_size == 0, partition_size % 16 == 0,
 * max_partitions*partition_size >= max_blocks_per_seq*block_size,
 * max_partitions >= 2 when cu_q_lens is given, and num_seqs <= 8192. */
pa_status pa_decode_split(const pa_kv_layout* layout, void* workspace, size_t workspace_bytes,
                          int32_t max_partitions, int32_t partition_size,
                          const void* q, const int32_t* cu_q_lens, int32_t num_q_tokens,
                          const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                          float scale, void* stream);

/* The same over fp8 pools (codes and scales as in pa_decode_fp8; bf16 q),
 * with the same partitions; prefill queries run on the vector units. */
pa_status pa_decode_split_fp8(const pa_kv_layout* layout, void* workspace,
                              size_t workspace_bytes, int32_t max_partitions,
                              int32_t partition_size, const void* q, const int32_t* cu_q_lens,
                              int32_t num_q_tokens, const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              float scale, void* stream);

/* Second pass: log-sum-exp merge of the partitions pa_decode_split wrote into
 * `workspace` (same sizes and partition rule).  With L = log sum_p
 * exp(lse_p):  out[j, h, :] = sum_p exp(lse_p - L) * o_p,  lse_out[j, h] = L.
 *   out     : [num_q_tokens, num_q_heads, head_dim] of out_dtype
 *   lse_out : fp32 [num_q_tokens, num_q_heads] or NULL
 * A query with no key gets a zero row and lse -inf. */
pa_status pa_reduce(void* out, int32_t out_dtype, float* lse_out, const void* workspace,
                    size_t workspace_bytes, int32_t max_partitions, int32_t partition_size,
                    const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim,
                    void* stream);

/* ------------------------------------------------------------------------ */
/* Host block pool ("19.2 KV Cache 系统化管理" §19.2.2-§19.2.3)               */
/* ------------------------------------------------------------------------ */
/* A library-owned host object: a LIFO free list of physical block ids,
 * one reference count per block, and per-sequence block tables.  Not
 * thread-safe (one scheduler thread drives it).  Calls are all-or-nothing:
 * on any error the pool is unchanged. */
typedef struct pa_pool pa_pool;

/* initial_free: host int32 [num_blocks], a permutation of 0..num_blocks-1
 * popped from its END (NULL = ascending order, so block num_blocks-1 is
 * handed out first, as in the pages' example). */
pa_status pa_pool_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* initial_free, pa_pool** out);
void pa_pool_destroy(pa_pool* pool);
int32_t pa_pool_num_free(const pa_pool* pool);               /* -1 if pool is NULL */
int32_t pa_pool_refcount(const pa_pool* pool, int32_t block); /* -1 if out of range */
/* Copy the free list (bottom to top) into host `out` (capacity `cap`). */
pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* New empty sequence; its handle is written to *seq. */
pa_status pa_seq_new(pa_pool* pool, int32_t* seq);
/* New sequence sharing every block of `parent` (reference count + 1 each). */
pa_status pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* child);
/* Blocks pa_seq_append(seq, n_tokens) would take from the free list. */
pa_status pa_seq_blocks_needed(const pa_pool* pool, int32_t seq, int32_t n_tokens,
                               int32_t* needed);
/* Reserve slots for n_tokens new tokens of `seq`.  Writes one flat slot
 * (physical*block_size + offset) per token to host slot_mapping_out
 * [n_tokens].  When the first token lands in a partly filled block shared
 * with another sequence, that block is copied first: a new block is taken,
 * the table remapped, the old count lowered, and the pair (old, new) written
 * to host cow_pairs_out [cow_cap, 2]; *n_cow gets the count (0 or 1).  The
 * caller copies those blocks (pa_copy_blocks) before writing the tokens.
 * PA_ERR_NO_FREE_BLOCKS if the free list is short (nothing changes). */
pa_status pa_seq_append(pa_pool* pool, int32_t seq, int32_t n_tokens,
                        int32_t* slot_mapping_out, int32_t* cow_pairs_out,
                        int32_t cow_cap, int32_t* n_cow);
/* Release every block of `seq` in logical order (counts - 1; a block whose
 * count reaches 0 is appended to the free list) and forget the sequence. */
pa_status pa_seq_release(pa_pool* pool, int32_t seq);
pa_status pa_seq_len(const pa_pool* pool, int32_t seq, int32_t* len);

/* Prefix cache over the pool ("LLM 推理引擎的内存管理与调度" §5.1-5.2, "19.2 KV
 * Cache 系统化管理" §19.2.5).  A full block is keyed by a chained hash of its
 * parent's key and its own tokens; a request whose prompt starts with
 * published blocks reuses them (one more reference each) and skips their
 * prefill.  Published blocks outlive their requests: at reference count 0
 * they are evictable rather than free, and an allocation that finds the free
 * list empty reclaims the least recently released one (blocks released by
 * one call in logical order).  pa_pool_num_free counts free plus evictable
 * blocks; pa_pool_free_list lists the free ones only.
 *
 * Key of one block: 64-bit FNV-1a (offset basis 0xCBF29CE484222325, prime
 * 0x100000001B3) over `parent` (8 bytes little endian; 0 for a request's
 * first block), `salt` (8 bytes little endian: model, adapter or other
 * context that changes the KV) and the n token ids (4 bytes little endian
 * each). */
uint64_t pa_prefix_hash(uint64_t parent, const int32_t* tokens, int32_t n, uint64_t salt);
/* For an empty sequence: map the cached blocks of keys[0], keys[1], ... in
 * order until the first key that is not cached; *n_hit blocks are mapped and
 * the sequence then holds n_hit * block_size tokens. */
pa_status pa_seq_match_prefix(pa_pool* pool, int32_t seq, const uint64_t* keys, int32_t n,
                              int32_t* n_hit);
/* Publish the sequence's first n blocks (all full) under keys[0..n-1].  A key
 * that another block already holds keeps that block; a block already
 * published under a different key is an error (nothing changes). */
pa_status pa_seq_register_prefix(pa_pool* pool, int32_t seq, const uint64_t* keys, int32_t n);
/* Host int32 out[n, max_blocks]: row i = table of seqs[i], padded with fill. */
pa_status pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n,
                          int32_t max_blocks, int32_t fill, int32_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
