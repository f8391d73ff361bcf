// Paged decode for callers that cannot allocate (code under graph capture, tight serving loops,
// harnesses that forbid allocation): the split-KV partials live in a device array the library
// holds instead of a caller workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/pkv.h"
#include "api_internal.h"

namespace {

// Each GPU the library runs on holds its own copy of this array until the process ends. In host
// code `scratch` is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that address is passed
// to kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, which `stream` must belong to (any stream
// of it, or the null stream).
int scratch_address(void* stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return PKV_E_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return PKV_E_HIP;
    if ((int)sdev != cur) return PKV_E_INVALID_ARGUMENT;
  }
  if (cur < 0 || cur >= kMaxDevices) return PKV_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[cur] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PKV_E_HIP;
    g_scratch[cur] = p;
  }
  *out = g_scratch[cur];
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_paged_attn_decode_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* seq_lens, void* out, float* lse, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_seq_len, float scale, int32_t partition_tokens,
    void* stream) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
      partition_tokens < -1)
    return PKV_E_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return PKV_E_INVALID_ARGUMENT;
  // the partials the call needs (0 on the direct path); beyond the array: rejected before launch
  const size_t need = batch > 0 ? pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                             head_dim, max_seq_len,
                                                             partition_tokens)
                                : 0;
  if (need > kScratchBytes) return PKV_E_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(stream, &ws);
    if (st != PKV_OK) return st;
  }
  return pkv::decode_checked(q, k_cache, v_cache, block_tables, seq_lens, out, lse, batch,
                             num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_seq_len, scale, partition_tokens, ws,
                             need > 0 ? kScratchBytes : 0, 0, 1.f, 1.f, 0, 0, stream);
}
