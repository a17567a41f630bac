// pkv_internal.h -- host functions shared between the library's sources (not exported).
#pragma once

#include <stdint.h>

#include "pkv.h"

namespace pkv {

// kv_copy.hip: k_new[s], v_new[s] to the slot of position context_lens[s] - 1 of each
// sequence, the slot taken from its block table (nothing for a context outside
// [1, max_ctx] or an entry outside the pool).  Host checks are the caller's.
pkv_status launch_kv_write_last(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                const int32_t *tables, int max_blocks, const int32_t *ctx, int max_ctx, int num_seqs,
                                int num_blocks, int block_size, int num_kv_heads, int head_dim, int elem_bytes,
                                void *stream);

}  // namespace pkv
