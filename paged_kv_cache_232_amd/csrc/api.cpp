// C ABI of the paged-KV attention library: argument checks, path choice, launches.
// Every check runs before anything is enqueued, so an error status means nothing was launched.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/pkv.h"
#include "api_internal.h"
#include "kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

bool block_size_ok(int bs) { return bs >= 16 && bs <= 256 && (bs & (bs - 1)) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_E_HIP; }

// Prefill: the most (request, q tile) work items one launch takes (one grid row each)
constexpr int64_t kMaxPrefillGridRows = 65528;

// Auto choice of the decode path. A direct launch gives one work-group per (sequence, kv head,
// q-head group); when that is too few to fill 256 CUs several times over and sequences are
// longer than one partition, split-KV. Its partition starts at 512 tokens (the vLLM page's
// _PARTITION_SIZE) and doubles while the longest sequence still yields 1024 single-wave
// partitions (four per CU): one wave then streams a long run of keys with nothing parked in LDS.
// On 4 x 131072 tokens (64 / 8 heads) that is 4096-token partitions: bf16 335 us against 348 us
// at 512, an fp8 cache 175 us against 209 us (same box). When 512-token partitions give fewer
// than 384 waves (a short window over few sequences) the partition halves instead, down to 128
// tokens, until they reach that: window 2048 over 4 sequences (64 / 8 heads) runs 24.1 us at 128
// against 32.1 us at 512 (same box), while 4-16-sequence batches of 3000-7000 tokens, with 448 or
// more waves at 512, ran the same or 2 % slower at 256.
constexpr int kDefaultPartition = 512;
constexpr int kMaxAutoPartition = 8192;
constexpr int kMinAutoPartition = 128;
constexpr int kDirectMinGroups = 512;  // two (sequence, kv head) work-groups per CU
constexpr long kSplitMinWaves = 1024;
constexpr long kSplitFewWaves = 384;

int resolve_partition(int batch, int num_q_heads, int num_kv_heads, int max_seq_len,
                      int partition_tokens) {
  if (partition_tokens >= 0) return partition_tokens;
  const int G = num_q_heads / num_kv_heads;
  const long groups = (long)batch * num_kv_heads * ((G + 15) / 16);
  if (max_seq_len <= kDefaultPartition || groups >= kDirectMinGroups) return 0;
  int pt = kDefaultPartition;
  while (pt < kMaxAutoPartition &&
         groups * (((long)max_seq_len + 2 * pt - 1) / (2 * pt)) >= kSplitMinWaves)
    pt *= 2;
  while (pt > kMinAutoPartition && groups * (((long)max_seq_len + pt - 1) / pt) < kSplitFewWaves)
    pt /= 2;
  return pt;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_E_INVALID_ARGUMENT: return "invalid argument";
    case PKV_E_UNSUPPORTED: return "unsupported configuration";
    case PKV_E_BAD_TABLE: return "bad block table";
    case PKV_E_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PKV_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_E_INVALID_ARGUMENT;
  if (head_dim <= 0 || head_dim % 8 != 0 || block_size <= 0) return PKV_E_INVALID_ARGUMENT;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_E_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_E_INVALID_ARGUMENT;
  return hip_status(pkv::launch_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                                  num_kv_heads, head_dim, block_size, num_blocks,
                                                  (hipStream_t)stream));
}

int pkv_decode_plan(const int32_t* seq_lens_h, int32_t batch, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t partition_tokens,
                    int32_t* max_seq_len_out, int32_t* partition_tokens_out,
                    size_t* workspace_bytes_out) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || partition_tokens < -1)
    return PKV_E_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return PKV_E_INVALID_ARGUMENT;
  if (!head_dim_ok(head_dim)) return PKV_E_UNSUPPORTED;
  if (partition_tokens > 0 && partition_tokens % 32 != 0) return PKV_E_UNSUPPORTED;
  if (!max_seq_len_out || !partition_tokens_out || !workspace_bytes_out) return PKV_E_INVALID_ARGUMENT;
  if (batch > 0 && !seq_lens_h) return PKV_E_INVALID_ARGUMENT;
  int32_t mx = 0;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens_h[b] < 0) return PKV_E_INVALID_ARGUMENT;
    if (seq_lens_h[b] > mx) mx = seq_lens_h[b];
  }
  const int pt = batch > 0 ? resolve_partition(batch, num_q_heads, num_kv_heads, mx, partition_tokens) : 0;
  *max_seq_len_out = mx;
  *partition_tokens_out = pt;
  *workspace_bytes_out = batch > 0 ? pkv::decode_workspace_layout(batch, num_q_heads, head_dim, mx, pt).total : 0;
  return PKV_OK;
}

size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int32_t partition_tokens) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0)
    return 0;
  if (num_q_heads % num_kv_heads != 0) return 0;
  const int pt = resolve_partition(batch, num_q_heads, num_kv_heads, max_seq_len, partition_tokens);
  return pkv::decode_workspace_layout(batch, num_q_heads, head_dim, max_seq_len, pt).total;
}

size_t pkv_decode_window_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len, int32_t window,
                                         int32_t partition_tokens) {
  if (window <= 0)
    return pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                      partition_tokens);
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0)
    return 0;
  if (num_q_heads % num_kv_heads != 0) return 0;
  const int pt = resolve_partition(batch, num_q_heads, num_kv_heads,
                                   std::min(max_seq_len, window), partition_tokens);
  if (pt <= 0) return 0;
  return pkv::decode_workspace_layout_p(batch, num_q_heads, head_dim,
                                        pkv::decode_window_partitions(max_seq_len, window, pt))
      .total;
}

}  // extern "C"

int pkv::decode_checked(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens, void* out, float* lse,
                        int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                        int32_t max_seq_len, float scale, int32_t partition_tokens, void* workspace,
                        size_t workspace_bytes, int kv_fp8, float k_scale, float v_scale,
                        int window, int ppw_override, void* stream) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_seq_len < 0 || partition_tokens < -1)
    return PKV_E_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return PKV_E_INVALID_ARGUMENT;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PKV_E_UNSUPPORTED;
  if (partition_tokens > 0 && partition_tokens % 32 != 0) return PKV_E_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return PKV_E_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PKV_E_INVALID_ARGUMENT;
  const int G = num_q_heads / num_kv_heads;
  const long ygrid = (long)num_kv_heads * ((G + 15) / 16);
  if (batch > 65535 || ygrid > 65535) return PKV_E_UNSUPPORTED;

  pkv::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.scale = scale;
  a.kv_fp8 = kv_fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.window = window;
  a.ppw_override = ppw_override;
  // a windowed call is planned on the keys it can see, and its partials cover only the window
  a.partition_tokens = resolve_partition(batch, num_q_heads, num_kv_heads,
                                         window > 0 ? std::min(max_seq_len, window) : max_seq_len,
                                         partition_tokens);
  if (a.partition_tokens > 0) {
    const pkv::DecodeWorkspaceLayout wl =
        window > 0 ? pkv::decode_workspace_layout_p(
                         batch, num_q_heads, head_dim,
                         pkv::decode_window_partitions(max_seq_len, window, a.partition_tokens))
                   : pkv::decode_workspace_layout(batch, num_q_heads, head_dim, max_seq_len,
                                                  a.partition_tokens);
    if (wl.max_partitions > 65535) return PKV_E_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < wl.total) return PKV_E_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return PKV_E_INVALID_ARGUMENT;
    char* ws = static_cast<char*>(workspace);
    a.o_part = reinterpret_cast<float*>(ws + wl.o_off);
    a.m_part = reinterpret_cast<float*>(ws + wl.m_off);
    a.l_part = reinterpret_cast<float*>(ws + wl.l_off);
    a.max_partitions = wl.max_partitions;
  }
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream));
}

static bool scale_ok(float s) { return s > 0.f && s <= 3.4028235e38f; }

extern "C" {

int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, void* out, float* lse,
                          int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_seq_len, float scale, int32_t partition_tokens, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return pkv::decode_checked(q, k_cache, v_cache, block_tables, seq_lens, out, lse, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_seq_len, scale, partition_tokens, workspace, workspace_bytes, 0, 1.f, 1.f,
                     0, 0, stream);
}

int pkv_paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens, void* out,
                              float* lse, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                              float k_scale, float v_scale, int32_t partition_tokens,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PKV_E_INVALID_ARGUMENT;
  return pkv::decode_checked(q, k_cache, v_cache, block_tables, seq_lens, out, lse, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_seq_len, scale, partition_tokens, workspace, workspace_bytes, 1, k_scale,
                     v_scale, 0, 0, stream);
}

int pkv_paged_attn_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* seq_lens, void* out,
                                 float* lse, int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t max_blocks_per_seq,
                                 int32_t max_seq_len, float scale, int32_t window,
                                 int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (window < 0) return PKV_E_INVALID_ARGUMENT;
  return pkv::decode_checked(q, k_cache, v_cache, block_tables, seq_lens, out, lse, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_seq_len, scale, partition_tokens, workspace, workspace_bytes, 0, 1.f, 1.f,
                     window, 0, stream);
}

static pkv::DecodeWorkspaceLayout stream_state_layout(int batch, int num_q_heads, int head_dim) {
  // one partition per (sequence, q head): o [B, 1, Hq, D], m and l [B, 1, Hq]
  return pkv::decode_workspace_layout(batch, num_q_heads, head_dim, 1, 1);
}

size_t pkv_stream_attn_state_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim) {
  if (batch <= 0 || num_q_heads <= 0 || !head_dim_ok(head_dim)) return 0;
  return stream_state_layout(batch, num_q_heads, head_dim).total;
}

int pkv_stream_attn_begin(void* state, size_t state_bytes, int32_t batch, int32_t num_q_heads,
                          int32_t head_dim, void* stream) {
  if (batch < 0 || num_q_heads <= 0) return PKV_E_INVALID_ARGUMENT;
  if (!head_dim_ok(head_dim)) return PKV_E_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  const pkv::DecodeWorkspaceLayout l = stream_state_layout(batch, num_q_heads, head_dim);
  if (!state || !aligned16(state)) return PKV_E_INVALID_ARGUMENT;
  if (state_bytes < l.total) return PKV_E_WORKSPACE_TOO_SMALL;
  char* st = static_cast<char*>(state);
  return hip_status(pkv::launch_stream_state_begin(
      reinterpret_cast<float*>(st + l.o_off), reinterpret_cast<float*>(st + l.m_off),
      reinterpret_cast<float*>(st + l.l_off), batch * num_q_heads, head_dim, (hipStream_t)stream));
}

int pkv_stream_attn_step(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* tile_tables, const int32_t* tile_lens, void* state,
                         size_t state_bytes, int32_t batch, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t tile_capacity, float scale, void* stream) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || tile_capacity <= 0)
    return PKV_E_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return PKV_E_INVALID_ARGUMENT;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PKV_E_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !tile_tables || !tile_lens || !state) return PKV_E_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(state))
    return PKV_E_INVALID_ARGUMENT;
  const int G = num_q_heads / num_kv_heads;
  if (batch > 65535 || (long)num_kv_heads * ((G + 15) / 16) > 65535) return PKV_E_UNSUPPORTED;
  const pkv::DecodeWorkspaceLayout l = stream_state_layout(batch, num_q_heads, head_dim);
  if (state_bytes < l.total) return PKV_E_WORKSPACE_TOO_SMALL;
  char* st = static_cast<char*>(state);
  pkv::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = tile_tables;
  a.seq_lens = tile_lens;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = tile_capacity;
  a.max_seq_len = tile_capacity * block_size;
  a.scale = scale;
  a.k_scale = a.v_scale = 1.f;
  a.partition_tokens = 0;  // one direct pass over the tile, folded into the state
  a.o_part = reinterpret_cast<float*>(st + l.o_off);
  a.m_part = reinterpret_cast<float*>(st + l.m_off);
  a.l_part = reinterpret_cast<float*>(st + l.l_off);
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream));
}

int pkv_stream_attn_finalize(const void* state, size_t state_bytes, void* out, float* lse,
                             int32_t batch, int32_t num_q_heads, int32_t head_dim, void* stream) {
  if (batch < 0 || num_q_heads <= 0) return PKV_E_INVALID_ARGUMENT;
  if (!head_dim_ok(head_dim)) return PKV_E_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (!state || !out || !aligned16(state) || !aligned16(out)) return PKV_E_INVALID_ARGUMENT;
  const pkv::DecodeWorkspaceLayout l = stream_state_layout(batch, num_q_heads, head_dim);
  if (state_bytes < l.total) return PKV_E_WORKSPACE_TOO_SMALL;
  const char* st = static_cast<const char*>(state);
  return hip_status(pkv::launch_stream_state_finalize(
      reinterpret_cast<const float*>(st + l.o_off), reinterpret_cast<const float*>(st + l.m_off),
      reinterpret_cast<const float*>(st + l.l_off), out, lse, batch * num_q_heads, head_dim,
      (hipStream_t)stream));
}

int pkv_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, float k_scale,
                              float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_E_INVALID_ARGUMENT;
  if (head_dim <= 0 || head_dim % 16 != 0 || block_size <= 0) return PKV_E_INVALID_ARGUMENT;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PKV_E_INVALID_ARGUMENT;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_E_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_E_INVALID_ARGUMENT;
  return hip_status(pkv::launch_reshape_and_cache_fp8(k, v, k_cache, v_cache, slot_mapping,
                                                      num_tokens, num_kv_heads, head_dim,
                                                      block_size, num_blocks, k_scale, v_scale,
                                                      (hipStream_t)stream));
}

// Checks shared by both prefill forms, on the host copies of the q offsets: sizes, supported
// shapes, and the schedule's limits (request and q-tile indices travel in 16 bits each, one grid
// row per q tile).
static int check_prefill_common(const void* q, const void* out, const int32_t* qo_indptr,
                                const int32_t* qo_indptr_h, int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int* max_qo, int* total_q,
                                int64_t* tiles, int* tile_rows) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0) return PKV_E_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return PKV_E_INVALID_ARGUMENT;
  if (!head_dim_ok(head_dim)) return PKV_E_UNSUPPORTED;
  // the kernels form a tile's per-lane K/V offsets with 24-bit multiplies of the row stride
  if ((int64_t)num_kv_heads * head_dim >= (1 << 23)) return PKV_E_UNSUPPORTED;
  *max_qo = 0;
  *total_q = 0;
  *tiles = 0;
  *tile_rows = pkv::prefill_tile_rows(head_dim, num_q_heads / num_kv_heads);
  if (batch == 0) return PKV_OK;
  if (!qo_indptr_h || !qo_indptr) return PKV_E_INVALID_ARGUMENT;
  if (qo_indptr_h[0] != 0) return PKV_E_INVALID_ARGUMENT;
  int mx = 0;
  for (int b = 0; b < batch; ++b) {
    const int n = qo_indptr_h[b + 1] - qo_indptr_h[b];
    if (n < 0) return PKV_E_INVALID_ARGUMENT;
    if (n > mx) mx = n;
  }
  *max_qo = mx;
  *total_q = qo_indptr_h[batch];
  if (*total_q > 0 && (!q || !out)) return PKV_E_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(out)) return PKV_E_INVALID_ARGUMENT;
  if (batch > 65535 || (int64_t)mx > 0xffffll * *tile_rows) return PKV_E_UNSUPPORTED;
  *tiles = pkv::prefill_tile_count(batch, qo_indptr_h, *tile_rows);
  if (*tiles > kMaxPrefillGridRows) return PKV_E_UNSUPPORTED;
  return PKV_OK;
}

static int check_prefill_workspace(int64_t tiles, const void* workspace, size_t workspace_bytes) {
  const size_t need = pkv::prefill_workspace_bytes(tiles);
  if (need == 0) return PKV_OK;
  if (workspace == nullptr || workspace_bytes < need) return PKV_E_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return PKV_E_INVALID_ARGUMENT;
  return PKV_OK;
}

size_t pkv_prefill_workspace_bytes(int32_t batch, const int32_t* qo_indptr_h, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim) {
  int max_qo = 0, total_q = 0, tile_rows = 0;
  int64_t tiles = 0;
  // q / out are not needed to size the schedule: pass any aligned non-null stand-in
  static const int32_t stand_in[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  if (check_prefill_common(stand_in, stand_in, stand_in, qo_indptr_h, batch, num_q_heads,
                           num_kv_heads, head_dim, &max_qo, &total_q, &tiles, &tile_rows) != PKV_OK)
    return 0;
  return pkv::prefill_workspace_bytes(tiles);
}

int pkv_ragged_prefill(const void* q, const void* k, const void* v, void* out,
                       const int32_t* qo_indptr, const int32_t* kv_indptr,
                       const int32_t* qo_indptr_h, const int32_t* kv_indptr_h, int32_t batch,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t causal,
                       float scale, void* workspace, size_t workspace_bytes, void* stream) {
  int max_qo = 0, total_q = 0, tile_rows = 0;
  int64_t tiles = 0;
  int st = check_prefill_common(q, out, qo_indptr, qo_indptr_h, batch, num_q_heads, num_kv_heads,
                                head_dim, &max_qo, &total_q, &tiles, &tile_rows);
  if (st != PKV_OK || batch == 0) return st;
  if (!kv_indptr_h || !kv_indptr) return PKV_E_INVALID_ARGUMENT;
  if (kv_indptr_h[0] != 0) return PKV_E_INVALID_ARGUMENT;
  for (int b = 0; b < batch; ++b)
    if (kv_indptr_h[b + 1] < kv_indptr_h[b]) return PKV_E_INVALID_ARGUMENT;
  const int64_t total_kv = kv_indptr_h[batch];
  if (total_kv > 0 && (!k || !v || !aligned16(k) || !aligned16(v))) return PKV_E_INVALID_ARGUMENT;
  if (total_q == 0) return PKV_OK;
  st = check_prefill_workspace(tiles, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  pkv::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.causal = causal != 0;
  a.scale = scale;
  a.qo_indptr_h = qo_indptr_h;
  a.kv_indptr_h = kv_indptr_h;
  a.max_qo_len = max_qo;
  a.total_q = total_q;
  a.total_kv = total_kv;
  a.tile_rows = tile_rows;
  a.tiles = tiles;
  a.workspace = workspace;
  const hipError_t e = pkv::launch_ragged_prefill(a, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return PKV_E_UNSUPPORTED;
  return hip_status(e);
}

int pkv_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* qo_indptr, const int32_t* kv_lens,
                      const int32_t* qo_indptr_h, const int32_t* kv_lens_h, void* out, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t causal, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int max_qo = 0, total_q = 0, tile_rows = 0;
  int64_t tiles = 0;
  int st = check_prefill_common(q, out, qo_indptr, qo_indptr_h, batch, num_q_heads, num_kv_heads,
                                head_dim, &max_qo, &total_q, &tiles, &tile_rows);
  if (st != PKV_OK || batch == 0) return st;
  if (!block_size_ok(block_size)) return PKV_E_UNSUPPORTED;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0) return PKV_E_INVALID_ARGUMENT;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PKV_E_UNSUPPORTED;
  if (!kv_lens_h || !kv_lens || !block_tables || !k_cache || !v_cache) return PKV_E_INVALID_ARGUMENT;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_E_INVALID_ARGUMENT;
  for (int b = 0; b < batch; ++b) {
    if (kv_lens_h[b] < 0) return PKV_E_INVALID_ARGUMENT;
    if ((int64_t)kv_lens_h[b] > (int64_t)max_blocks_per_seq * block_size) return PKV_E_BAD_TABLE;
  }
  if (total_q == 0) return PKV_OK;
  st = check_prefill_workspace(tiles, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  pkv::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.qo_indptr = qo_indptr;
  a.kv_lens = kv_lens;
  a.block_tables = block_tables;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.causal = causal != 0;
  a.scale = scale;
  a.qo_indptr_h = qo_indptr_h;
  a.kv_lens_h = kv_lens_h;
  a.max_qo_len = max_qo;
  a.total_q = total_q;
  a.tile_rows = tile_rows;
  a.tiles = tiles;
  a.workspace = workspace;
  const hipError_t e = pkv::launch_paged_prefill(a, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return PKV_E_UNSUPPORTED;
  return hip_status(e);
}

int pkv_validate_block_tables_h(const int32_t* block_tables_h, const int32_t* seq_lens_h,
                                int32_t batch, int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t num_blocks) {
  if (batch < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_blocks < 0)
    return PKV_E_INVALID_ARGUMENT;
  if (batch > 0 && (!seq_lens_h || (max_blocks_per_seq > 0 && !block_tables_h)))
    return PKV_E_INVALID_ARGUMENT;
  for (int b = 0; b < batch; ++b)
    if (seq_lens_h[b] < 0) return PKV_E_INVALID_ARGUMENT;
  for (int b = 0; b < batch; ++b) {
    const int64_t need = ((int64_t)seq_lens_h[b] + block_size - 1) / block_size;
    if (need > max_blocks_per_seq) return PKV_E_BAD_TABLE;
    const int32_t* row = block_tables_h + (size_t)b * max_blocks_per_seq;
    for (int64_t j = 0; j < need; ++j)
      if (row[j] < 0 || row[j] >= num_blocks) return PKV_E_BAD_TABLE;
  }
  return PKV_OK;
}

// Decode autotuning: every candidate configuration is launched on the caller's buffers and timed
// with HIP events on the caller's stream; the fastest one is kept in the caller's plan.
static const int32_t kTunePartitions[] = {256, 512, 1024, 2048, 4096, 8192};
static const int32_t kTunePpw[] = {1, 2, 4, 8, 16};

int pkv_decode_tune(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, void* out,
                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                    int32_t repeats, void* stream, pkv_decode_tuned_plan* plan) {
  if (!plan || repeats < 1 || repeats > 1000) return PKV_E_INVALID_ARGUMENT;
  // the library's own choice: also validates every argument before anything is timed
  auto run = [&](int32_t pt, int32_t ppw) {
    return pkv::decode_checked(q, k_cache, v_cache, block_tables, seq_lens, out, nullptr, batch,
                               num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                               max_blocks_per_seq, max_seq_len, scale, pt, workspace,
                               workspace_bytes, 0, 1.f, 1.f, 0, ppw, stream);
  };
  int st = run(-1, 0);
  if (st != PKV_OK) return st;
  if (batch == 0) {
    memset(plan, 0, sizeof(*plan));
    plan->max_seq_len = max_seq_len;
    return PKV_OK;
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return PKV_E_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return PKV_E_HIP;
  }
  const hipStream_t s = (hipStream_t)stream;
  std::vector<float> ts;
  // median over `repeats` timed launches after one untimed launch; < 0 on a failed launch
  auto time_us = [&](int32_t pt, int32_t ppw) -> float {
    if (run(pt, ppw) != PKV_OK) return -1.f;
    ts.clear();
    for (int r = 0; r < repeats; ++r) {
      if (hipEventRecord(e0, s) != hipSuccess) return -1.f;
      if (run(pt, ppw) != PKV_OK) return -1.f;
      float ms = 0.f;
      if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
          hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
        return -1.f;
      ts.push_back(ms * 1000.f);
    }
    std::sort(ts.begin(), ts.end());
    return ts[ts.size() / 2];
  };
  const int32_t def_pt = resolve_partition(batch, num_q_heads, num_kv_heads, max_seq_len, -1);
  float best = time_us(-1, 0);
  int32_t best_pt = def_pt, best_ppw = 0, n = 1;
  const float def_us = best;
  if (best >= 0.f) {
    auto consider = [&](int32_t pt, int32_t ppw) {
      const float us = time_us(pt, ppw);
      ++n;
      if (us >= 0.f && us < best) {
        best = us;
        best_pt = pt;
        best_ppw = ppw;
      }
    };
    consider(0, 0);
    const int cap = pkv::decode_max_ppw(num_q_heads, num_kv_heads, head_dim);
    for (int32_t pt : kTunePartitions) {
      if (pt >= max_seq_len) continue;  // one partition: the direct path does the same work
      const size_t need = pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                     max_seq_len, pt);
      if (workspace == nullptr || need > workspace_bytes) continue;
      const int32_t parts = (max_seq_len + pt - 1) / pt;
      for (int32_t ppw : kTunePpw)
        if (ppw <= cap && ppw <= parts) consider(pt, ppw);
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (best < 0.f) return PKV_E_HIP;
  plan->partition_tokens = best_pt;
  plan->partitions_per_wave = best_pt > 0 ? best_ppw : 0;
  plan->max_seq_len = max_seq_len;
  plan->candidates = n;
  plan->workspace_bytes = pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                     max_seq_len, best_pt);
  plan->measured_us = best;
  plan->default_us = def_us;
  return PKV_OK;
}

int pkv_paged_attn_decode_tuned(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens, void* out,
                                float* lse, int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, float scale,
                                const pkv_decode_tuned_plan* plan, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!plan || plan->partition_tokens < 0 || plan->partitions_per_wave < 0 ||
      plan->partitions_per_wave > 16)
    return PKV_E_INVALID_ARGUMENT;
  return pkv::decode_checked(q, k_cache, v_cache, block_tables, seq_lens, out, lse, batch,
                             num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_seq_len, scale, plan->partition_tokens,
                             workspace, workspace_bytes, 0, 1.f, 1.f, 0,
                             plan->partition_tokens > 0 ? plan->partitions_per_wave : 0, stream);
}

int pkv_copy_blocks(const uint64_t* k_cache_ptrs, const uint64_t* v_cache_ptrs, int32_t num_layers,
                    const int64_t* block_mapping, int32_t num_pairs, int64_t block_bytes,
                    int32_t num_blocks, void* stream) {
  if (num_layers < 0 || num_pairs < 0 || num_blocks < 0 || block_bytes <= 0 || block_bytes % 16 != 0)
    return PKV_E_INVALID_ARGUMENT;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!k_cache_ptrs || !v_cache_ptrs || !block_mapping) return PKV_E_INVALID_ARGUMENT;
  if (num_layers > 65535) return PKV_E_INVALID_ARGUMENT;  // grid y limit
  return hip_status(pkv::launch_copy_blocks(k_cache_ptrs, v_cache_ptrs, num_layers, block_mapping,
                                            num_pairs, block_bytes, num_blocks,
                                            (hipStream_t)stream));
}

int pkv_swap_blocks(const void* src, void* dst, const int64_t* block_mapping_h, int32_t num_pairs,
                    int64_t block_bytes, int32_t src_num_blocks, int32_t dst_num_blocks,
                    void* stream) {
  if (num_pairs < 0 || block_bytes <= 0 || src_num_blocks < 0 || dst_num_blocks < 0)
    return PKV_E_INVALID_ARGUMENT;
  if (num_pairs == 0) return PKV_OK;
  if (!src || !dst || !block_mapping_h) return PKV_E_INVALID_ARGUMENT;
  for (int i = 0; i < num_pairs; ++i) {
    const int64_t s = block_mapping_h[2 * i], d = block_mapping_h[2 * i + 1];
    if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks) return PKV_E_INVALID_ARGUMENT;
  }
  return hip_status(pkv::swap_blocks(src, dst, block_mapping_h, num_pairs, block_bytes,
                                     (hipStream_t)stream));
}

}  // extern "C"
