// Device helpers shared by the gfx950 kernels of the denoise-step library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tt {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

// Two fp32 -> packed fp16x2 (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 32x32x16 bf16 MFMA, fp32 accumulate. Operand layout (wave64): A row = lane % 32, B column =
// lane % 32, both holding 8 consecutive k values selected by lane / 32. Result: lane holds column
// lane % 32 and, in register i, row (i / 4) * 8 + (lane / 32) * 4 + (i % 4).
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld_global_16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// Stores of results that a later kernel reads (from any XCD) go through a buffer resource over a
// wave-uniform base with the write-through policy (sc1): they reach memory while the kernel runs
// instead of staying dirty in this XCD's L2 until the write-back at the kernel's end (a plain
// 256 x 32 KB store kernel: 2.8 instead of 3.3 us).
constexpr int kWriteThrough = 16;  // cache-policy operand: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ void st_wt_16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kWriteThrough);
}

__device__ __forceinline__ u32x4 ld_lds_16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void st_lds_16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Value held by lane (lane ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over the lane pair (lane, lane ^ 32), in every lane, without LDS: one
// v_permlane32_swap gives each lane both halves' values.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

#define TT_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8); expcnt and
// lgkmcnt are left at their maxima so only vector-memory operations are waited for. Issued through
// the builtin so that the compiler's own wait insertion knows about them.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Work-group barrier for LDS hand-offs: this wave's LDS operations are complete, then s_barrier.
// (No memory fence: outstanding global loads, including direct-to-LDS ones, are waited for
// explicitly with waitcnt_vm.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// XOR key of the 16-byte chunk swizzle for LDS rows of 128 bytes: the 8 (32-bank) and 16
// (64-bank, two rows per bank line) consecutive rows read by one operand load hit distinct slots.
__device__ __forceinline__ int key128(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

}  // namespace tt
