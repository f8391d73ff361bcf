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

template <bool POW2>
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                         u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                         const int64_t* __restrict__ slot_mapping, int64_t num_units,
                         int units_per_token, int units_per_row, int block_size,
                         int64_t num_slots, int upt_shift, int upr_shift, int bs_shift) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int heads = units_per_token / units_per_row;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < num_units; u += stride) {
    // POW2: units per token, units per row and block size are powers of two (shifts and masks
    // instead of 64-bit divisions, which the GPU emulates with dozens of instructions)
    int64_t t, blk, off;
    int h, c;
    if constexpr (POW2) {
      t = u >> upt_shift;
    } else {
      t = u / units_per_token;
    }
    const int r = (int)(u - t * units_per_token);  // unit within the token: head * units_per_row + c
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    if constexpr (POW2) {
      h = r >> upr_shift;
      c = r & (units_per_row - 1);
      blk = slot >> bs_shift;
      off = slot & (block_size - 1);
    } else {
      h = r / units_per_row;
      c = r - h * units_per_row;
      blk = slot / block_size;
      off = slot - blk * block_size;
    }
    const int64_t dst = ((blk * heads + h) * block_size + off) * units_per_row + c;
    const u32x4 kv = k[u];
    const u32x4 vv = v[u];
    k_cache[dst] = kv;
    v_cache[dst] = vv;
  }
}

static bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

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
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (is_pow2(units_per_token) && is_pow2(units_per_row) && is_pow2(block_size))
    hipLaunchKernelGGL((reshape_and_cache_kernel<true>), dim3((unsigned)blocks), dim3(threads), 0,
                       stream, (const u32x4*)k, (const u32x4*)v, (u32x4*)k_cache, (u32x4*)v_cache,
                       slot_mapping, num_units, units_per_token, units_per_row, block_size,
                       num_slots, __builtin_ctz((unsigned)units_per_token),
                       __builtin_ctz((unsigned)units_per_row), __builtin_ctz((unsigned)block_size));
  else
    hipLaunchKernelGGL((reshape_and_cache_kernel<false>), dim3((unsigned)blocks), dim3(threads), 0,
                       stream, (const u32x4*)k, (const u32x4*)v, (u32x4*)k_cache, (u32x4*)v_cache,
                       slot_mapping, num_units, units_per_token, units_per_row, block_size,
                       num_slots, 0, 0, 0);
  return hipGetLastError();
}

// fp8 (OCP e4m3) cache: each thread writes one 16-byte unit of 16 codes, code = e4m3(x / scale)
// with x the bf16 input widened to fp32 and an IEEE fp32 division; the hardware conversion rounds
// to nearest even, magnitudes beyond 448 are clamped to 448 first (it would give NaN), and a NaN
// input is stored as 0x7F.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  float x[4] = {a, b, c, d};
  uint32_t nan_mask = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (x[j] != x[j]) nan_mask |= 0xFFu << (8 * j);
    x[j] = x[j] > 448.f ? 448.f : (x[j] < -448.f ? -448.f : x[j]);  // NaN passes unchanged
  }
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], r, true);
  return (r & ~nan_mask) | (0x7F7F7F7Fu & nan_mask);
}

__device__ __forceinline__ u32x4 quantize16(u32x4 lo, u32x4 hi, float scale) {
  // lo / hi: 16 bf16 values (8 each); bf16 -> fp32 is a 16-bit shift
  float f[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __builtin_bit_cast(float, lo[j] << 16) / scale;
    f[2 * j + 1] = __builtin_bit_cast(float, lo[j] & 0xFFFF0000u) / scale;
    f[8 + 2 * j] = __builtin_bit_cast(float, hi[j] << 16) / scale;
    f[8 + 2 * j + 1] = __builtin_bit_cast(float, hi[j] & 0xFFFF0000u) / scale;
  }
  return u32x4{e4m3x4(f[0], f[1], f[2], f[3]), e4m3x4(f[4], f[5], f[6], f[7]),
               e4m3x4(f[8], f[9], f[10], f[11]), e4m3x4(f[12], f[13], f[14], f[15])};
}

__global__ void __launch_bounds__(256)
reshape_and_cache_fp8_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                             u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                             const int64_t* __restrict__ slot_mapping, int64_t num_units,
                             int units_per_token, int units_per_row, int block_size,
                             int64_t num_slots, float k_scale, float v_scale) {
  // unit u = 16 elements: input units 2u, 2u+1 (16 bytes of bf16 each), output unit (16 codes)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < num_units; u += stride) {
    const int64_t t = u / units_per_token;
    const int r = (int)(u - t * units_per_token);
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int h = r / units_per_row;
    const int c = r - h * units_per_row;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const int heads = units_per_token / units_per_row;
    const int64_t dst = ((blk * heads + h) * block_size + off) * units_per_row + c;
    k_cache[dst] = quantize16(k[2 * u], k[2 * u + 1], k_scale);
    v_cache[dst] = quantize16(v[2 * u], v[2 * u + 1], v_scale);
  }
}

hipError_t launch_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                        const int64_t* slot_mapping, int num_tokens,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, float k_scale, float v_scale,
                                        hipStream_t stream) {
  const int units_per_row = head_dim / 16;
  const int units_per_token = units_per_row * num_kv_heads;
  const int64_t num_units = (int64_t)num_tokens * units_per_token;
  if (num_units == 0) return hipSuccess;
  const int threads = 256;
  int64_t blocks = (num_units + threads - 1) / threads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(reshape_and_cache_fp8_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const u32x4*)k, (const u32x4*)v, (u32x4*)k_cache, (u32x4*)v_cache,
                     slot_mapping, num_units, units_per_token, units_per_row, block_size,
                     (int64_t)num_blocks * block_size, k_scale, v_scale);
  return hipGetLastError();
}

}  // namespace pkv
