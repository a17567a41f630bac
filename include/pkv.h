/*
 * pkv.h -- C ABI of libpkv.so: paged KV cache decode kernels for AMD MI355X (gfx950).
 *
 * The KV cache is one pre-allocated pool per tensor, split into num_blocks
 * fixed-size physical blocks of block_size token slots; each sequence owns a
 * block table mapping its logical blocks to physical block ids (pages
 * "nano-vLLM . Ch04 . PagedAttention", section 4 "The Three Mechanisms", and
 * "PagedAttention" (PidokuInfra, topic 10), section 5 "The kernel side").
 *
 * Layouts (row-major, element type given by pkv_dtype):
 *   k_cache, v_cache : [num_blocks, block_size, num_kv_heads, head_dim]
 *   q, out           : [num_seqs, num_heads, head_dim]
 *   k_new, v_new     : [num_tokens, num_kv_heads, head_dim]
 *   block_tables     : int32 [num_seqs, max_blocks_per_seq]
 *   context_lens     : int32 [num_seqs]
 *   slot_mapping     : int64 [num_tokens], slot = block_id * block_size + offset
 *   block_mapping    : int64 [num_pairs, 2], rows (src_block, dst_block)
 *
 * Ownership and threading: every array argument is a DEVICE pointer owned by the
 * caller.  The library allocates nothing, keeps no state between calls and never
 * synchronises: each call only enqueues kernels on `stream` (a hipStream_t; NULL
 * is the default stream) and returns.  Calls are thread-safe.  The one exception is
 * paged_attention_decode_noalloc, whose scratch is a static device array of the library
 * (described with it).
 *
 * Errors: host-visible argument checks return a status before anything is
 * enqueued (the pages' allocator reports failure by return value rather than by
 * crashing; PidokuInfra section 4 ErrNoBlocks, nano-vLLM section 7).  A launch
 * failure returns PKV_ERR_HIP.  Device-resident values cannot be checked on the
 * host; how each kernel treats out-of-range device values is stated per call.
 *
 * Supported shapes: head_dim in {64, 128}; block_size in {4, 8, 16, 32, 64, 128};
 * num_heads % num_kv_heads == 0; dtype fp32 or bf16.  bf16 attention with head_dim
 * 128 and g = num_heads / num_kv_heads <= 16 runs on the tile path, at every block
 * size (matrix cores for g >= 2, fp32 vector dot products for g = 1); everything else
 * runs on the vector path, which needs block_size <= 32 and g <= 8.
 * pkv_attention_path reports which.
 * All data pointers must be 16-byte aligned, index arrays 4- or 8-byte aligned.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, workspace too small */
  PKV_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim, block_size, group size, dtype */
  PKV_ERR_HIP = 3,           /* the HIP runtime rejected a launch */
  PKV_ERR_SCRATCH_LIMIT = 4  /* paged_attention_decode_noalloc: the call needs more than the static scratch */
} pkv_status;

typedef enum { PKV_DTYPE_F32 = 0, PKV_DTYPE_BF16 = 1 } pkv_dtype;

/*
 * Kernel families of paged_attention_decode:
 *   PKV_PATH_VECTOR    -- fp32, or head_dim 64: one token row per lane group, q.k by DPP sums;
 *   PKV_PATH_MFMA      -- bf16, head_dim 128, 2..16 query heads per KV head: 16-token tiles
 *                         on MFMA, the query-head group as the B operand;
 *   PKV_PATH_TILE_VALU -- bf16, head_dim 128, one query head per KV head: the same 16-token
 *                         tile stream with q.k and P.V as fp32 FMAs (q.k summed by DPP).
 */
typedef enum { PKV_PATH_NONE = 0, PKV_PATH_VECTOR = 1, PKV_PATH_MFMA = 2, PKV_PATH_TILE_VALU = 3 } pkv_path;

/*
 * paged_kv_write -- write the K/V rows of new tokens into the pool through a slot
 * mapping computed on the host (nano-vLLM Ch04 section 4, Mechanism 3: slot =
 * physical_block_id * block_size + offset_within_block; the kernel does no address
 * translation of its own).  For token i with slot s, the bytes of k_new[i, :, :]
 * land in k_cache[s / block_size, s % block_size, :, :], and likewise for V.  A bit
 * copy: NaN payloads, -0 and subnormals are preserved; no other byte changes.
 *
 * Device values: slots outside [0, num_blocks * block_size) -- including the
 * conventional -1 "no slot" -- are skipped (nothing is written for that token).
 * Slots must be distinct within one call; with duplicates the result is undefined.
 * num_tokens == 0 is a valid no-op.  A row (num_kv_heads * head_dim elements) above
 * 256 MiB returns PKV_ERR_UNSUPPORTED.
 */
pkv_status paged_kv_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                          const int64_t *slot_mapping, int64_t num_tokens, int32_t num_blocks,
                          int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                          void *stream);

/*
 * pkv_attention_workspace_size -- bytes of device scratch that paged_attention_decode
 * needs: a 256-byte work-queue header, followed, when a sequence can span more than one
 * partition, by the fp32 partial states of the split (given the host-side maximum context
 * length): one record per (sequence, partition, KV head) holding the group's unnormalised
 * partial rows and a 128-byte line of (max, sum) pairs, for which
 * num_seqs * num_heads * partitions * (head_dim + 32) floats always suffice.  Always at least
 * 256.
 */
size_t pkv_attention_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t partition_size);

/*
 * pkv_attention_path -- which kernel family paged_attention_decode would run for these
 * shapes (PKV_PATH_NONE if unsupported).
 */
pkv_path pkv_attention_path(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            pkv_dtype dtype);

/*
 * paged_attention_decode -- one decode query per sequence:
 *   out[s, h, :] = softmax(scale * q[s, h, :] . K_s^T) V_s
 * where K_s, V_s are the rows of positions 0 .. context_lens[s]-1, position t living
 * in physical block block_tables[s, t / block_size] at offset t % block_size
 * (PidokuInfra section 5 "The kernel side": the walk over ceil(ctx / block_size)
 * blocks through the table, with an online-softmax accumulation; tokentrails step 3:
 * the same attention as on contiguous K/V).  Query head h reads KV head
 * h / (num_heads / num_kv_heads).  Only positions < context_lens[s] are read: slots
 * past it in the last block and table entries past ceil(ctx / block_size) are never
 * touched.  Accumulation is fp32; out has the dtype of q.
 *
 * partition_size == 0: each (sequence, KV head) is one unit of work.  Otherwise
 * (a multiple of block_size; a multiple of 16 on the MFMA path) the context is cut
 * into partitions of that many tokens, partial softmax states go to the workspace and
 * a second kernel merges them by log-sum-exp in a fixed order, so results are
 * deterministic.
 *
 * workspace: caller-owned device memory of at least pkv_attention_workspace_size bytes,
 * 16-byte aligned, always required.  Its first 256 bytes are the work-queue counters of
 * the persistent kernels: they must be zero before the first call that uses the
 * workspace (clear them once when it is allocated) and every call leaves them zero.
 * Calls that share a workspace must not overlap (issue them on one stream).
 * max_context_len must bound every context_lens[s] and fit the table
 * (max_context_len <= max_blocks_per_seq * block_size); a sequence may span at most
 * 8192 partitions, max_context_len at most 2^30 and max_blocks_per_seq at most 2^29
 * (PKV_ERR_UNSUPPORTED beyond).
 *
 * Device values: context_lens[s] <= 0 gives out[s] = 0; context_lens[s] >
 * max_context_len, or a table entry read that lies outside [0, num_blocks), gives
 * NaN for the affected outputs.  Neither faults.
 *
 * Work items: on the bf16 / head_dim 128 paths with blocks of 16 slots or more, a large
 * launch whose sequences' blocks lie far apart in the pool hands out the bulk of its work as
 * items of 2 or 4 KV heads (the library decides per launch; see attention.hip).  The item
 * width changes no bit of any output.  The environment variable PKV_WIDE_ITEMS=1, 2 or 4
 * caps the width and applies it to every item of the launch (1: one KV head per item), for
 * tests and tuning.
 */
pkv_status paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, int32_t partition_size, void *workspace,
                                  size_t workspace_bytes, pkv_dtype dtype, void *stream);

/*
 * copy_blocks -- the copy of copy-on-write (nano-vLLM Ch04 section 6: before a write
 * into a block whose refcount is above one, copy the block first, then write;
 * tokentrails Code box, copy_block).  For each row (src, dst) of block_mapping,
 * the whole of physical block src -- all block_size slots -- is copied bit for bit
 * into block dst, in k_cache and in v_cache.
 *
 * Device values: pairs with src or dst outside [0, num_blocks) are skipped.
 * Destinations must be distinct and no destination may also be a source within
 * one call; otherwise the result is undefined.  num_pairs == 0 is a valid no-op.
 */
pkv_status copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping, int64_t num_pairs,
                       int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                       pkv_dtype dtype, void *stream);

/*
 * paged_attention_decode_write -- a decode step's write and attention in one launch: the
 * same as paged_kv_write of k_new[s], v_new[s] ([num_seqs, num_kv_heads, head_dim]) to the
 * slot of position context_lens[s] - 1 of each sequence (the slot its table gives:
 * block_tables[s, (ctx - 1) / block_size] * block_size + (ctx - 1) % block_size), followed by
 * paged_attention_decode over contexts that include that token (tokentrails steps 2-3: write
 * the new token's K/V, then attend; nano-vLLM section 4 "Mechanism 3": the slot from the
 * table).  Outputs and caches are bit-identical to those two calls.  On the tile paths
 * (PKV_PATH_MFMA, PKV_PATH_TILE_VALU) the row of each sequence's new token is written by the
 * work item that attends to it and used from registers, in the one launch; where the MFMA
 * tiles split into partitions of at most 256 tokens, and on the vector path, the write is a
 * launch of its own just before the attention's.
 *
 * Arguments as for paged_attention_decode, plus k_new and v_new (device, 16-byte aligned;
 * null gives PKV_ERR_INVALID_ARG); k_cache and v_cache are written.  The row layout only
 * (PKV_ERR_UNSUPPORTED for shapes paged_attention_decode does not take).  A sequence with
 * context_lens[s] <= 0 or > max_context_len, or whose new token's table entry lies outside
 * [0, num_blocks), writes nothing (and gets the outputs paged_attention_decode gives it).
 * The slots written must be distinct and must not be shared with another sequence (after a
 * fork, copy_blocks first), as for paged_kv_write.
 */
pkv_status paged_attention_decode_write(void *out, const void *q, const void *k_new, const void *v_new,
                                        void *k_cache, void *v_cache, const int32_t *block_tables,
                                        int32_t max_blocks_per_seq, const int32_t *context_lens,
                                        int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, float scale, int32_t partition_size, void *workspace,
                                        size_t workspace_bytes, pkv_dtype dtype, void *stream);

/*
 * The head-major cache layout (PidokuInfra page, section 5 "The layout, more precisely"):
 *   k_cache : [num_blocks, num_kv_heads, head_dim / x, block_size, x],  x = 16 / elem_bytes
 *   v_cache : [num_blocks, num_kv_heads, head_dim, block_size]
 * The same values as the row layout, placed so that one (block, KV head) is contiguous:
 * K[b, o, h, d] of the row layout is k_cache[b, h, d / x, o, d % x] here and V[b, o, h, d]
 * is v_cache[b, h, d, o].  A block is still num_kv_heads * head_dim * block_size elements,
 * so copy_blocks serves both layouts unchanged.
 *
 * paged_kv_write_head_major -- paged_kv_write into this layout: token i with slot
 * s = b * block_size + o fills k_cache[b, :, :, o, :] and v_cache[b, :, :, o] from
 * k_new[i], v_new[i] ([T, num_kv_heads, head_dim]); arguments, checks and device-value
 * handling as for paged_kv_write.
 */
pkv_status paged_kv_write_head_major(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                     const int64_t *slot_mapping, int64_t num_tokens, int32_t num_blocks,
                                     int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                                     void *stream);

/*
 * paged_attention_decode_head_major -- paged_attention_decode on head-major caches: the same
 * arguments, workspace, checks and results (the same attention; outputs may differ from the
 * row layout's only in rounding).  Built for bf16, head_dim 128, block_size in
 * {16, 32, 64, 128}, num_heads / num_kv_heads <= 16 (PKV_ERR_UNSUPPORTED otherwise;
 * pkv_attention_path_head_major reports it).
 */
pkv_status paged_attention_decode_head_major(void *out, const void *q, const void *k_cache, const void *v_cache,
                                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                                             const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_blocks, float scale,
                                             int32_t partition_size, void *workspace, size_t workspace_bytes,
                                             pkv_dtype dtype, void *stream);

pkv_path pkv_attention_path_head_major(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, pkv_dtype dtype);

/*
 * pkv_stream_read_probe -- measurement only, not part of the decode path: one plain streaming
 * read of `bytes` of device memory at `buf` (16-byte aligned; a whole number of 16-byte words
 * is read, the rest ignored) with non-temporal 16-byte loads, to time the rate this device's
 * HBM delivers to a read-only kernel without indirection.  `sink` is a caller-owned device word
 * that the kernel may write (it folds what it reads so that no load is dead); its value means
 * nothing.  PKV_ERR_INVALID_ARG for null or misaligned pointers or bytes < 16; asynchronous on
 * `stream`, like every call here.
 */
pkv_status pkv_stream_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/*
 * paged_attention_decode_noalloc -- for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): paged_attention_decode
 * with the same arguments but no workspace.  The work-queue header and the split's partial states
 * live in a static device array of the library, pkv_static_scratch_bytes() = 64 MiB, which every
 * device the library runs on holds from the first call until the process ends.  Nothing is
 * allocated or freed by the call; results are those of paged_attention_decode (the same kernels).
 *
 * The first call on a device (the current device) looks up that device's array and clears its
 * work-queue header with a small kernel on `stream`; every call leaves the header at zero again.
 * All calls on one device share its array: calls that may overlap on one device (two streams,
 * two threads, or a graph replay beside an eager call) race and must not be issued.  A call
 * whose workspace need (pkv_attention_workspace_size) exceeds the array returns
 * PKV_ERR_SCRATCH_LIMIT before anything is enqueued; other checks and device-value handling as
 * for paged_attention_decode.
 */
pkv_status paged_attention_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                                          const int32_t *block_tables, int32_t max_blocks_per_seq,
                                          const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t num_blocks, float scale,
                                          int32_t partition_size, pkv_dtype dtype, void *stream);

/* Bytes of the static scratch array behind paged_attention_decode_noalloc (per device). */
size_t pkv_static_scratch_bytes(void);

/* Static, human-readable name of a status code. */
const char *pkv_status_string(pkv_status status);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
