// Internal helpers shared by the HIP kernels of the paged-KV attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16x16x32 bf16 MFMA, fp32 accumulate. Operand layout (wave64):
//   A [16 x 32]: lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B [32 x 16]: lane l holds B[8 * (l / 16) + j][l % 16]
//   C [16 x 16]: lane l holds C[4 * (l / 16) + r][l % 16], r = 0..3
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA, fp32 accumulate. Operand layout (wave64):
//   A [32 x 16]: lane l holds A[l % 32][8 * (l / 32) + j]
//   B [16 x 32]: lane l holds B[8 * (l / 32) + j][l % 32]
//   C [32 x 32]: lane l holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32], r = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  u32x4 r;
  r[0] = pack_bf16x2(v[0], v[1]);
  r[1] = pack_bf16x2(v[2], v[3]);
  r[2] = pack_bf16x2(v[4], v[5]);
  r[3] = pack_bf16x2(v[6], v[7]);
  return as_bf16x8(r);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group, lanes 4r..4r+3
// each supply the address of 4 consecutive 16-bit elements; together they form row r (16
// elements) of a 4 x 16 block, and lane i of the group receives column i: the 4 values
// (row0[i], row1[i], row2[i], row3[i]).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across lanes l and l ^ 16 (resp. l ^ 32) with gfx950's v_permlane16_swap /
// v_permlane32_swap: with both operands holding x, the two results hold x of rows {0,2} and of
// rows {1,3} (resp. of the low and high half), so combining them reduces over the partner lanes in
// VALU only. The second operand is passed through an empty asm so the compiler cannot treat the
// two operands as one value (it otherwise folds the swap of identical operands away).
__device__ __forceinline__ uint2 swap16(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("" : "+v"(b));
  const auto p = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  return uint2{p[0], p[1]};
}
__device__ __forceinline__ uint2 swap32(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("" : "+v"(b));
  const auto p = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return uint2{p[0], p[1]};
}
__device__ __forceinline__ float max_xor16(float x) {
  const uint2 p = swap16(x);
  return fmaxf(__builtin_bit_cast(float, p.x), __builtin_bit_cast(float, p.y));
}
__device__ __forceinline__ float max_xor32(float x) {
  const uint2 p = swap32(x);
  return fmaxf(__builtin_bit_cast(float, p.x), __builtin_bit_cast(float, p.y));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const uint2 p = swap16(x);
  return __builtin_bit_cast(float, p.x) + __builtin_bit_cast(float, p.y);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint2 p = swap32(x);
  return __builtin_bit_cast(float, p.x) + __builtin_bit_cast(float, p.y);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Non-temporal 16-byte store (global_store ... nt): for outputs no later kernel of the same pass
// re-reads soon. Prefill output written this way streams to HBM while the (compute-bound) kernel
// runs, instead of lingering dirty in the caches and being written back during the next kernel.
__device__ __forceinline__ void store16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Raw buffer resource over memory starting at a wave-uniform address (no bounds limit: callers
// keep every offset inside their tensors). Loads through it take a 32-bit per-lane byte offset,
// so a tile's addresses cost one VALU op per unit instead of a 64-bit add per load.
// The address is made explicitly uniform (the compiler would otherwise loop over lanes whenever
// it cannot prove that itself).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0, -1, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Direct-to-LDS 16-byte load (gfx950 global_load_lds_dwordx4): lane i reads the 16 bytes at
// base + voff_i and writes them to LDS bytes [lds + 16 i, lds + 16 i + 16), so one instruction
// fills 1 KiB of LDS contiguously. base and lds are made wave-uniform (SGPR base, M0). The load is
// written as asm so that the compiler's wait-count pass does not track it: it would otherwise wait
// for every such load in flight before any LDS read, and a fence at a barrier waits for all of them
// too. Callers wait with wait_vm_barrier() below. M0 is saved and restored around the load. The
// instruction has no destination register, so nothing in registers is written behind the
// compiler's back.
__device__ __forceinline__ void dma_load16(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(u), "s"(l)
      : "memory");
}

// Waits until at most N of this wave's vector-memory loads (dma_load16 included) are still in
// flight and all its LDS operations are done, then joins the work-group barrier. Vector loads
// complete in issue order, so N counts the most recent loads that may stay outstanding.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// acc + the sum of 8 bf16 values (two per v_dot2_f32_bf16 against (1, 1); the products are exact)
__device__ __forceinline__ float sum_bf16x8(bf16x8 p, float acc) {
  const u32x4 u = __builtin_bit_cast(u32x4, p);
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // copied out first: a bit_cast applied directly to a vector element reads element 0
    const uint32_t x = u[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
  }
  return acc;
}

__device__ __forceinline__ u32x2 load8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// 8 fp8 (OCP e4m3) codes -> 8 bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1: every e4m3 value,
// subnormals and NaN included, is exactly representable in bf16). Element order is kept: byte j of
// the input becomes bf16 j of the result.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 x) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true));
  return r;
}

// Keeps the compiler from moving memory operations across this point. Loads that a loop keeps in
// flight across iterations must be issued in the same order before the loop as inside it, or the
// wait-count pass cannot tell their order at the loop head and waits for all of them.
__device__ __forceinline__ void memory_order_point() { asm volatile("" ::: "memory"); }

template <typename T>
__device__ __forceinline__ T clampi(T x, T lo, T hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// A wave's sliding view of one block-table row: 64 consecutive entries held one per lane, with the
// next 64 already loaded. Block ids come out with v_readlane (a scalar), so forming a page address
// never waits on a table load issued behind in-flight data loads. Indices passed to get() must be
// wave-uniform and non-decreasing. Entries past the row width read as 0.
struct TableWindow {
  const int32_t* row;
  int width;
  int base;
  int cur;
  int nxt;

  __device__ __forceinline__ void init(const int32_t* r, int w, int first_index, int lane) {
    row = r;
    width = w;
    base = first_index & ~63;
    const int j0 = base + lane, j1 = base + 64 + lane;
    cur = j0 < width ? row[j0] : 0;
    nxt = j1 < width ? row[j1] : 0;
  }
  __device__ __forceinline__ int get(int index, int lane) {
    while (index >= base + 64) {
      base += 64;
      cur = nxt;
      const int j = base + 64 + lane;
      nxt = j < width ? row[j] : 0;
    }
    return __builtin_amdgcn_readlane(cur, index - base);
  }
};

}  // namespace pkv
