// Internal launchers, one per kernel family. Each validates nothing: the C ABI layer in api.cpp
// checks arguments first and only then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks,
                                    hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  int batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq;
  int max_seq_len;
  float scale;
  int partition_tokens;  // 0 = direct, > 0 = split
  int kv_fp8;            // caches hold fp8 (e4m3) codes dequantised by k_scale / v_scale
  float k_scale, v_scale;
  int window;            // > 0: keys [L - window, L) only
  int ppw_override;      // split: consecutive partitions per wave (0 = the library's choice)
  // split workspace (null for direct)
  float* o_part;
  float* m_part;
  float* l_part;
  int max_partitions;
};

hipError_t launch_stream_state_begin(float* o, float* m, float* l, int rows, int head_dim,
                                     hipStream_t stream);
hipError_t launch_stream_state_finalize(const float* o, const float* m, const float* l, void* out,
                                        float* lse, int rows, int head_dim, hipStream_t stream);

// Split-KV workspace layout for a given shape: o [B, P, Hq, D] f32, m and l [B, P, Hq] f32, each
// region 256-byte aligned.
struct DecodeWorkspaceLayout {
  size_t o_off, m_off, l_off, total;
  int max_partitions;
};
DecodeWorkspaceLayout decode_workspace_layout(int batch, int num_q_heads, int head_dim,
                                              int max_seq_len, int partition_tokens);
// Partition slots per sequence of a windowed split call: its partials are indexed from the
// partition holding the window's first key, so the slots cover the window, not max_seq_len.
int decode_window_partitions(int max_seq_len, int window, int partition_tokens);
DecodeWorkspaceLayout decode_workspace_layout_p(int batch, int num_q_heads, int head_dim, int partitions);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Most consecutive split partitions one wave can stream (its finished partials wait in LDS).
int decode_max_ppw(int num_q_heads, int num_kv_heads, int head_dim);

struct PrefillArgs {
  const void* q;
  const void* k;        // contiguous [Tkv, Hkv, D] (ragged) or k_cache (paged)
  const void* v;
  void* out;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;     // ragged only
  const int32_t* kv_lens;       // paged only
  const int32_t* block_tables;  // paged only
  int batch, num_q_heads, num_kv_heads, head_dim;
  int block_size, num_blocks, max_blocks_per_seq;  // paged only
  int causal;
  float scale;
  const int32_t* qo_indptr_h;   // host copies (order the work-groups; may be null)
  const int32_t* kv_indptr_h;   // ragged only
  const int32_t* kv_lens_h;     // paged only
  int max_qo_len;   // host-side maximum of the q lengths
  int total_q;      // rows of q / out
  int64_t total_kv; // rows of k / v (ragged only)
  int tile_rows;    // q rows of one work item (prefill_tile_rows(head_dim, group))
  int64_t tiles;    // (request, q tile) work items, from the host copies
  void* workspace;  // >= prefill_workspace_bytes(tiles) bytes (the device-built schedule)
};

// q rows of one prefill work item for a head dim; the (request, q tile) work items of a launch;
// and the workspace its schedule needs (0 when the schedule travels with the launch).
int prefill_tile_rows(int head_dim, int group);
int64_t prefill_tile_count(int batch, const int32_t* qo_indptr_h, int tile_rows);
size_t prefill_workspace_bytes(int64_t tiles);

hipError_t launch_ragged_prefill(const PrefillArgs& a, hipStream_t stream);

hipError_t launch_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                        const int64_t* slot_mapping, int num_tokens,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, float k_scale, float v_scale,
                                        hipStream_t stream);

hipError_t launch_copy_blocks(const uint64_t* k_ptrs, const uint64_t* v_ptrs, int num_layers,
                              const int64_t* mapping, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream);
hipError_t swap_blocks(const void* src, void* dst, const int64_t* mapping_h, int num_pairs,
                       int64_t block_bytes, hipStream_t stream);
hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pkv
