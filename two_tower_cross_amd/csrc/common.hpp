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

__device__ __forceinline__ u32x4 ld_lds_16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void st_lds_16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Value held by lane (lane ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace tt
