// kv_copy.hip -- the two data-movement kernels of the paged KV cache:
//   paged_kv_write: new tokens' K/V rows into the pool through a host-built slot mapping
//                   (nano-vLLM Ch04, section 4 "The Three Mechanisms", Mechanism 3);
//   copy_blocks:    whole-block copies for copy-on-write (nano-vLLM Ch04, section 6).
// Both are pure 16-byte integer moves, so every bit pattern (NaN payloads, -0,
// subnormals) survives.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// Calls that write at least this many bytes load and store with the non-temporal hint: their
// destination is larger than what the next launch could find in cache, and with the hint on both
// sides the bulk write ran 2-3% faster (level with the runtime's own contiguous device copy).
// Smaller calls -- every decode step's write and copy-on-write copies -- keep the cached forms,
// since the attention launch right after them reads what they wrote (with the hint the fused fork
// step took 0.8 us longer).
constexpr int64_t kStreamingMoveBytes = int64_t(32) << 20;

template <bool NT>
__device__ __forceinline__ u32x4 mv_load(const u32x4 *p) {
  if constexpr (NT) return ld16_stream(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void mv_store(u32x4 *p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// One workgroup per (token, 4 KiB chunk of its row), grid-stride over tokens beyond the
// grid.  A slot names one [Hkv, D] row of the pool; consecutive slots are consecutive rows,
// so the row of slot s = b * B + o starts s * row_vecs 16-byte vectors into the pool.  The
// row loads do not depend on the slot, so they are in flight together with the slot load:
// one load round trip, then the stores.
constexpr int kWriteThreads = 128;
constexpr int kWriteVecs = 2;                               // 16-byte vectors per thread and tensor
constexpr int kWriteChunk = kWriteThreads * kWriteVecs;     // vectors of a row per workgroup
template <bool NT>
__global__ __launch_bounds__(kWriteThreads) void kv_write_kernel(const u32x4 *__restrict__ k_new,
                                                                 const u32x4 *__restrict__ v_new,
                                                                 u32x4 *__restrict__ k_cache,
                                                                 u32x4 *__restrict__ v_cache,
                                                                 const int64_t *__restrict__ slots,
                                                                 int64_t num_tokens, int row_vecs, int64_t num_slots) {
  const int c0 = (int)blockIdx.y * kWriteChunk + (int)threadIdx.x;
  for (int64_t tok = blockIdx.x; tok < num_tokens; tok += gridDim.x) {
    const int64_t slot = slots[tok];
    const u32x4 *ks = k_new + tok * row_vecs;
    const u32x4 *vs = v_new + tok * row_vecs;
    u32x4 kv[kWriteVecs], vv[kWriteVecs];
#pragma unroll
    for (int i = 0; i < kWriteVecs; ++i) {
      const int c = c0 + i * kWriteThreads;
      if (c < row_vecs) {
        kv[i] = mv_load<NT>(ks + c);
        vv[i] = mv_load<NT>(vs + c);
      }
    }
    if (slot < 0 || slot >= num_slots) continue;  // -1 / out of range: no write
    u32x4 *kd = k_cache + slot * row_vecs;
    u32x4 *vd = v_cache + slot * row_vecs;
#pragma unroll
    for (int i = 0; i < kWriteVecs; ++i) {
      const int c = c0 + i * kWriteThreads;
      if (c < row_vecs) {
        mv_store<NT>(kd + c, kv[i]);
        mv_store<NT>(vd + c, vv[i]);
      }
    }
  }
}

// The same write into the head-major layout (page "PagedAttention", PidokuInfra topic 10,
// section 5 "The layout, more precisely"): K [N, Hkv, D/x, B, x] with x = 16 / elem_bytes,
// V [N, Hkv, D, B].  Slot s = b * B + o: K vector j (x head dims) of head h goes to 16-byte
// vector ((b * Hkv + h) * (D/x) + j) * B + o; V element (h, d) to element
// ((b * Hkv + h) * D + d) * B + o.  One workgroup per token.
template <typename E>
__global__ __launch_bounds__(256) void kv_write_head_major_kernel(const u32x4 *__restrict__ k_new,
                                                                  const E *__restrict__ v_new,
                                                                  u32x4 *__restrict__ k_cache, E *__restrict__ v_cache,
                                                                  const int64_t *__restrict__ slots, int64_t num_tokens,
                                                                  int num_kv_heads, int head_dim, int block_size,
                                                                  int64_t num_slots) {
  const int kvec = head_dim * (int)sizeof(E) / 16;   // K vectors per head
  const int row_k = num_kv_heads * kvec, row_v = num_kv_heads * head_dim;
  for (int64_t tok = blockIdx.x; tok < num_tokens; tok += gridDim.x) {
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;  // -1 / out of range: no write
    const int64_t b = slot / block_size, o = slot % block_size;
    for (int c = threadIdx.x; c < row_k; c += blockDim.x) {
      const int64_t hj = b * row_k + c;   // (b * Hkv + h) * kvec + j
      k_cache[hj * block_size + o] = k_new[tok * row_k + c];
    }
    for (int c = threadIdx.x; c < row_v; c += blockDim.x) {
      const int64_t hd = b * row_v + c;   // (b * Hkv + h) * D + d
      v_cache[hd * block_size + o] = v_new[tok * row_v + c];
    }
  }
}

// grid = (pairs, chunks of one block, 2 tensors).  Each workgroup copies up to
// 256 threads x 4 vectors = 16 KiB of one block of one tensor.
constexpr int kCopyVecsPerThread = 4;
constexpr int kCopyThreads = 256;
constexpr int kCopyChunk = kCopyThreads * kCopyVecsPerThread;

template <bool NT>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(u32x4 *__restrict__ k_cache,
                                                                   u32x4 *__restrict__ v_cache,
                                                                   const int64_t *__restrict__ pairs,
                                                                   int64_t block_vecs, int32_t num_blocks) {
  const int64_t pair = blockIdx.x;
  const int64_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;  // skipped pair
  u32x4 *pool = blockIdx.z == 0 ? k_cache : v_cache;
  const u32x4 *s = pool + src * block_vecs;
  u32x4 *d = pool + dst * block_vecs;
  const int64_t c0 = (int64_t)blockIdx.y * kCopyChunk + threadIdx.x;
  u32x4 buf[kCopyVecsPerThread];
#pragma unroll
  for (int i = 0; i < kCopyVecsPerThread; ++i) {
    const int64_t c = c0 + (int64_t)i * kCopyThreads;
    if (c < block_vecs) buf[i] = mv_load<NT>(s + c);
  }
#pragma unroll
  for (int i = 0; i < kCopyVecsPerThread; ++i) {
    const int64_t c = c0 + (int64_t)i * kCopyThreads;
    if (c < block_vecs) mv_store<NT>(d + c, buf[i]);
  }
}

// The new token of each decode step: k_new[s], v_new[s] to the slot of position ctx[s] - 1,
// the slot taken from the sequence's table (the write paged_attention_decode_write makes when
// its attention runs as a launch of its own).  Nothing is written for a context outside
// [1, max_ctx] or a table entry outside the pool.
__global__ __launch_bounds__(kWriteThreads) void kv_write_last_kernel(
    const u32x4 *__restrict__ k_new, const u32x4 *__restrict__ v_new, u32x4 *__restrict__ k_cache,
    u32x4 *__restrict__ v_cache, const int32_t *__restrict__ tables, int max_blocks, const int32_t *__restrict__ ctx,
    int max_ctx, int num_blocks, int block_size, int row_vecs) {
  const int s = blockIdx.x;
  const int c = ctx[s];
  if (c < 1 || c > max_ctx) return;
  const int blk = tables[(int64_t)s * max_blocks + (c - 1) / block_size];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t slot = (int64_t)blk * block_size + (c - 1) % block_size;
  const int c0 = (int)blockIdx.y * kWriteChunk + (int)threadIdx.x;
#pragma unroll
  for (int i = 0; i < kWriteVecs; ++i) {
    const int v = c0 + i * kWriteThreads;
    if (v < row_vecs) {
      k_cache[slot * row_vecs + v] = k_new[(int64_t)s * row_vecs + v];
      v_cache[slot * row_vecs + v] = v_new[(int64_t)s * row_vecs + v];
    }
  }
}

pkv_status launch_kv_write_last(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                const int32_t *tables, int max_blocks, const int32_t *ctx, int max_ctx, int num_seqs,
                                int num_blocks, int block_size, int num_kv_heads, int head_dim, int elem_bytes,
                                void *stream) {
  const int64_t row_vecs = (int64_t)num_kv_heads * head_dim * elem_bytes / 16;
  const int64_t chunks = (row_vecs + kWriteChunk - 1) / kWriteChunk;
  if (chunks > 65535 || num_seqs > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kv_write_last_kernel, dim3((unsigned)num_seqs, (unsigned)chunks), dim3(kWriteThreads), 0,
                     (hipStream_t)stream, (const u32x4 *)k_new, (const u32x4 *)v_new, (u32x4 *)k_cache,
                     (u32x4 *)v_cache, tables, max_blocks, ctx, max_ctx, num_blocks, block_size, (int)row_vecs);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

static bool shape_ok(int32_t block_size, int32_t num_kv_heads, int32_t head_dim) {
  return (head_dim == 64 || head_dim == 128) &&
         (block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64 ||
          block_size == 128) &&
         num_kv_heads >= 1;
}

static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status paged_kv_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                     const int64_t *slot_mapping, int64_t num_tokens, int32_t num_blocks,
                                     int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                                     void *stream) {
  if (dtype != PKV_DTYPE_F32 && dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1)
    return PKV_ERR_INVALID_ARG;
  if (!shape_ok(block_size, num_kv_heads, head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_INVALID_ARG;
  const int64_t elem = dtype == PKV_DTYPE_F32 ? 4 : 2;
  const int64_t row_vecs64 = (int64_t)num_kv_heads * head_dim * elem / 16;
  const int64_t chunks = (row_vecs64 + kWriteChunk - 1) / kWriteChunk;
  if (chunks > 65535) return PKV_ERR_UNSUPPORTED;
  const int row_vecs = (int)row_vecs64;
  const unsigned grid = (unsigned)(num_tokens < (1 << 20) ? num_tokens : (1 << 20));
  const bool nt = 2 * num_tokens * row_vecs64 * 16 >= kStreamingMoveBytes;
  hipLaunchKernelGGL(nt ? kv_write_kernel<true> : kv_write_kernel<false>, dim3(grid, (unsigned)chunks),
                     dim3(kWriteThreads), 0, (hipStream_t)stream, (const u32x4 *)k_new, (const u32x4 *)v_new,
                     (u32x4 *)k_cache, (u32x4 *)v_cache, slot_mapping, num_tokens, row_vecs,
                     (int64_t)num_blocks * block_size);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" pkv_status paged_kv_write_head_major(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                                const int64_t *slot_mapping, int64_t num_tokens, int32_t num_blocks,
                                                int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                                pkv_dtype dtype, void *stream) {
  if (dtype != PKV_DTYPE_F32 && dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1)
    return PKV_ERR_INVALID_ARG;
  if (!shape_ok(block_size, num_kv_heads, head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_INVALID_ARG;
  const int64_t grid = num_tokens < 65535 ? num_tokens : 65535;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == PKV_DTYPE_BF16)
    hipLaunchKernelGGL(kv_write_head_major_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, st,
                       (const u32x4 *)k_new, (const uint16_t *)v_new, (u32x4 *)k_cache, (uint16_t *)v_cache,
                       slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_slots);
  else
    hipLaunchKernelGGL(kv_write_head_major_kernel<uint32_t>, dim3((unsigned)grid), dim3(256), 0, st,
                       (const u32x4 *)k_new, (const uint32_t *)v_new, (u32x4 *)k_cache, (uint32_t *)v_cache,
                       slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_slots);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" pkv_status copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping, int64_t num_pairs,
                                  int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                  pkv_dtype dtype, void *stream) {
  if (dtype != PKV_DTYPE_F32 && dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1)
    return PKV_ERR_INVALID_ARG;
  if (!shape_ok(block_size, num_kv_heads, head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (num_pairs > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  if (!k_cache || !v_cache || !block_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_mapping, 8)) return PKV_ERR_INVALID_ARG;
  const int64_t elem = dtype == PKV_DTYPE_F32 ? 4 : 2;
  const int64_t block_vecs = (int64_t)block_size * num_kv_heads * head_dim * elem / 16;
  const int64_t chunks = (block_vecs + kCopyChunk - 1) / kCopyChunk;
  if (chunks > 65535) return PKV_ERR_UNSUPPORTED;
  const bool nt = 2 * num_pairs * block_vecs * 16 >= kStreamingMoveBytes;
  hipLaunchKernelGGL(nt ? copy_blocks_kernel<true> : copy_blocks_kernel<false>,
                     dim3((unsigned)num_pairs, (unsigned)chunks, 2), dim3(kCopyThreads), 0, (hipStream_t)stream,
                     (u32x4 *)k_cache, (u32x4 *)v_cache, block_mapping, block_vecs, num_blocks);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" const char *pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_HIP: return "HIP launch failure";
    case PKV_ERR_SCRATCH_LIMIT: return "needs more scratch than the library's static scratch array holds";
  }
  return "unknown status";
}
