// Host-side pieces of the C ABI shared between its source files.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Argument checks, path choice and launch of paged decode: the body of every decode entry point
// (bf16 or fp8 caches, with or without a sliding window). ppw_override > 0 sets how many
// consecutive split partitions one wave streams (0: the library's choice). Returns a pkv_status;
// on error nothing was enqueued.
int decode_checked(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* seq_lens, void* out, float* lse,
                   int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                   int32_t max_seq_len, float scale, int32_t partition_tokens, void* workspace,
                   size_t workspace_bytes, int kv_fp8, float k_scale, float v_scale, int window,
                   int ppw_override, void* stream);

}  // namespace pkv
