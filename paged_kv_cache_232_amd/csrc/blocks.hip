// Block management around the paged cache: copy_blocks (inside each layer's caches, on the GPU)
// and swap_blocks (between caches in different memories).
//
// Operations as the vLLM-derived paged_attn.py page defines them (PagedAttention.copy_blocks and
// PagedAttention.swap_blocks): for every (src, dst) pair, block dst of the destination cache becomes
// a copy of block src of the source cache, for the key and the value cache of every layer. A block
// of one cache is the contiguous [num_kv_heads, block_size, head_dim] run of the cache layout.
//
// copy_blocks is one launch for all layers and pairs: work-group (pair, layer, K|V) copies one
// block in 16-byte units, every load of a thread issued before its stores (an HBM-bound copy).
// Loads and stores are non-temporal: nothing in the copy re-reads a line (3-4 % faster).
// swap_blocks runs the same block copy when the GPU can address both caches (pinned host memory is
// read and written over PCIe by the kernel itself), else one HIP copy per run of consecutive pairs.
#include "common.h"
#include "kernels.h"

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;  // 16-byte units per thread in flight

__global__ void __launch_bounds__(kCopyThreads)
copy_blocks_kernel(const uint64_t* __restrict__ k_ptrs, const uint64_t* __restrict__ v_ptrs,
                   const int64_t* __restrict__ mapping, int64_t units_per_block, int num_blocks) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const int64_t src = mapping[2 * (int64_t)pair];
  const int64_t dst = mapping[2 * (int64_t)pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const uint64_t base = blockIdx.z == 0 ? k_ptrs[layer] : v_ptrs[layer];
  const u32x4* s = reinterpret_cast<const u32x4*>(base) + src * units_per_block;
  u32x4* d = reinterpret_cast<u32x4*>(base) + dst * units_per_block;
  for (int64_t u0 = threadIdx.x; u0 < units_per_block; u0 += kCopyThreads * kCopyUnroll) {
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t u = u0 + (int64_t)j * kCopyThreads;
      if (u < units_per_block) x[j] = __builtin_nontemporal_load(s + u);
    }
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t u = u0 + (int64_t)j * kCopyThreads;
      if (u < units_per_block) __builtin_nontemporal_store(x[j], d + u);
    }
  }
}

hipError_t launch_copy_blocks(const uint64_t* k_ptrs, const uint64_t* v_ptrs, int num_layers,
                              const int64_t* mapping, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream) {
  if (num_pairs == 0 || num_layers == 0) return hipSuccess;
  const dim3 grid(num_pairs, num_layers, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, k_ptrs, v_ptrs,
                     mapping, block_bytes / 16, num_blocks);
  return hipGetLastError();
}

// swap_blocks between two memories the GPU can address (device memory, pinned host memory): one
// work-group per block, the pairs passed by value in batches of kSwapBatch per launch.
constexpr int kSwapBatch = 240;
struct SwapPairs {
  int64_t src[kSwapBatch];
  int64_t dst[kSwapBatch];
};

__global__ void __launch_bounds__(kCopyThreads)
swap_blocks_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, SwapPairs pairs, int n,
                   int64_t units_per_block) {
  const int i = blockIdx.x;
  if (i >= n) return;
  const u32x4* s = src + pairs.src[i] * units_per_block;
  u32x4* d = dst + pairs.dst[i] * units_per_block;
  for (int64_t u0 = threadIdx.x; u0 < units_per_block; u0 += kCopyThreads * kCopyUnroll) {
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t u = u0 + (int64_t)j * kCopyThreads;
      if (u < units_per_block) x[j] = s[u];
    }
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t u = u0 + (int64_t)j * kCopyThreads;
      if (u < units_per_block) d[u] = x[j];
    }
  }
}

// Device address of p when the GPU can read and write it directly (device memory, managed memory,
// pinned host memory mapped into the GPU's address space); null otherwise (pageable host memory).
static void* gpu_address(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // pageable memory is not an error for the caller
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged ||
      a.type == hipMemoryTypeHost)
    return a.devicePointer;
  return nullptr;
}

hipError_t swap_blocks(const void* src, void* dst, const int64_t* mapping_h, int num_pairs,
                       int64_t block_bytes, hipStream_t stream) {
  const void* src_d = gpu_address(src);
  void* dst_d = gpu_address(dst);
  if (src_d != nullptr && dst_d != nullptr && block_bytes % 16 == 0) {
    for (int i0 = 0; i0 < num_pairs; i0 += kSwapBatch) {
      const int n = num_pairs - i0 < kSwapBatch ? num_pairs - i0 : kSwapBatch;
      SwapPairs pairs;
      for (int i = 0; i < n; ++i) {
        pairs.src[i] = mapping_h[2 * (i0 + i)];
        pairs.dst[i] = mapping_h[2 * (i0 + i) + 1];
      }
      hipLaunchKernelGGL(swap_blocks_kernel, dim3(n), dim3(kCopyThreads), 0, stream,
                         static_cast<const u32x4*>(src_d), static_cast<u32x4*>(dst_d), pairs, n,
                         block_bytes / 16);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // pageable host memory: HIP copies, with runs of pairs whose source and destination blocks both
  // advance by one moved as one copy
  int i = 0;
  while (i < num_pairs) {
    const int64_t s0 = mapping_h[2 * i], d0 = mapping_h[2 * i + 1];
    int n = 1;
    while (i + n < num_pairs && mapping_h[2 * (i + n)] == s0 + n && mapping_h[2 * (i + n) + 1] == d0 + n)
      ++n;
    hipError_t e = hipMemcpyAsync(static_cast<char*>(dst) + d0 * block_bytes,
                                  static_cast<const char*>(src) + s0 * block_bytes,
                                  (size_t)n * block_bytes, hipMemcpyDefault, stream);
    if (e != hipSuccess) return e;
    i += n;
  }
  return hipSuccess;
}

}  // namespace pkv
