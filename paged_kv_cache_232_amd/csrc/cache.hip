// reshape_and_cache: bit copy of new tokens' K/V rows into their paged-cache slots.
// Operation as the vLLM-derived paged_attn.py page defines it (PagedAttention.write_to_paged_cache):
// row [t, h, :] of key/value goes to cache[slot / block_size, h, slot % block_size, :] for
// slot = slot_mapping[t]; negative slots are skipped.
//
// HBM-bound copy: each thread moves 16-byte units; consecutive threads walk one token's
// [Hkv, D] rows, so reads are contiguous and each (block, head, offset) row is written as
// D * 2 contiguous bytes.
#include "common.h"
#include "kernels.h"

namespace pkv {

__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                         u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                         const int64_t* __restrict__ slot_mapping, int64_t num_units,
                         int units_per_token, int units_per_row, int block_size,
                         int64_t num_slots) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < num_units; u += stride) {
    const int64_t t = u / units_per_token;
    const int r = (int)(u - t * units_per_token);  // unit within the token: head * units_per_row + c
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int h = r / units_per_row;
    const int c = r - h * units_per_row;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const int heads = units_per_token / units_per_row;
    const int64_t dst = ((blk * heads + h) * block_size + off) * units_per_row + c;
    const u32x4 kv = k[u];
    const u32x4 vv = v[u];
    k_cache[dst] = kv;
    v_cache[dst] = vv;
  }
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks,
                                    hipStream_t stream) {
  const int units_per_row = head_dim / 8;
  const int units_per_token = units_per_row * num_kv_heads;
  const int64_t num_units = (int64_t)num_tokens * units_per_token;
  if (num_units == 0) return hipSuccess;
  const int threads = 256;
  int64_t blocks = (num_units + threads - 1) / threads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const u32x4*)k, (const u32x4*)v, (u32x4*)k_cache, (u32x4*)v_cache,
                     slot_mapping, num_units, units_per_token, units_per_row, block_size,
                     (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

}  // namespace pkv
