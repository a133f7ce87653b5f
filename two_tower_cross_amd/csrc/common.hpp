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


// Returns v unchanged, as the output of an (empty) asm statement at this point of the program:
// nothing can be computed from v before it, so the wait for the load that produced v is placed
// here and not right after the load (a flag read at kernel start and used much later).
__device__ __forceinline__ uint32_t defer_use(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ u32x4 ld_lds_16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void st_lds_16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

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

// Phase stamps of the profiling build (compiled with TT_PHASE_STAMPS; the product library has
// none): wave 0 of a work-group records wall_clock64() (a constant 100 MHz counter) at up to 6
// phases of its kernel and clock64() (shader cycles) at 2 more points; its first lane stores the
// 8 values in the file's stamp array, row = flat work-group id.
#ifdef TT_PHASE_STAMPS
#define TT_STAMPS_DECL unsigned long long tt_st_[8] = {0, 0, 0, 0, 0, 0, 0, 0}
#define TT_STAMP(i) do { if (threadIdx.x < 64) tt_st_[i] = wall_clock64(); } while (0)
#define TT_CYCLES(i) do { if (threadIdx.x < 64) tt_st_[i] = clock64(); } while (0)
#define TT_STAMP_DRAINED(i) do { __builtin_amdgcn_s_waitcnt(0); TT_STAMP(i); } while (0)
#define TT_STAMPS_STORE(arr, id) \
  do { if (threadIdx.x == 0 && (id) < 8192) for (int i_ = 0; i_ < 8; ++i_) arr[id][i_] = tt_st_[i_]; } while (0)
#else
#define TT_STAMPS_DECL do {} while (0)
#define TT_STAMP(i) do {} while (0)
#define TT_CYCLES(i) do {} while (0)
#define TT_STAMP_DRAINED(i) do {} while (0)
#define TT_STAMPS_STORE(arr, id) do {} while (0)
#endif

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

// Arrival of member s of a group of n work-groups (1 <= n <= 16) at the group's counter, called by
// one thread of the work-group once every store of the work-group that the others read has
// completed. Returns the set of shares (bit i: share i) this work-group must merge: its own share
// once every member has arrived, plus, for the member that completes the count, the shares of
// members that gave up waiting; 0 when it gave up itself. No member waits for anything that might
// never run: a member that has polled max_polls times without seeing the count complete hands its
// share over and leaves, so the group finishes even when its members cannot all be resident at
// once (another kernel holding compute units, on another stream), only more slowly.
// The counter is a 64-bit word in device memory (alone in its 128-byte line): tag << 32 |
// given-up mask << 16 | count, where `tag` (nonzero) identifies the launch. A word holding another
// tag, or a complete count, is left over from an earlier launch (or is arbitrary memory): the first
// member to arrive starts a new round with a compare-and-swap, every other member adds 1 (one
// atomic round trip each, whatever the contention), so the word needs no reset between launches:
// a new launch brings a new tag, and replays of one recorded launch, which share their tag, find
// the previous replay's complete count. A member gives up with a compare-and-swap that sets its
// bit only while the count is incomplete, so the completing member's add returns every bit set
// before it; a give-up that loses that race finds the count complete and merges its own share.
// Visibility without cache-wide maintenance (a release or acquire fence at device scope writes back
// or invalidates this XCD's whole L2, which costs tens of microseconds when 32 work-groups of an
// XCD do it in turn): what the members exchange is stored write-through (sc1) and every wave of
// the work-group has waited for its stores to complete (vmcnt 0, then a work-group barrier)
// before the arrival; the merging work-groups read it with device-coherent loads (sc1), issued
// only once the complete count has been observed. The arrival and the polls are device-scope
// atomics (relaxed: the ordering comes from those completions).
__device__ __forceinline__ uint32_t group_arrive(unsigned long long *ctr, uint32_t tag, int n, int s,
                                                 int max_polls) {
  const unsigned long long base = (unsigned long long)tag << 32;
  const unsigned long long nn = (unsigned long long)n;
  unsigned long long v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if ((v >> 32) == tag && (v & 0xFFFFull) < nn) {
      v = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
      break;
    }
    // left over from before: start this launch's round (v is reloaded when another member did)
    if (__hip_atomic_compare_exchange_strong(ctr, &v, base | 1ull, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
      v = base | 1ull;
      break;
    }
  }
  const uint32_t own = 1u << s;
  if ((v & 0xFFFFull) == nn) return own | (uint32_t)((v >> 16) & 0xFFFFull);  // completed it
  for (int polls = 0;;) {
    if ((v & 0xFFFFull) == nn) return own;  // every member has arrived
    if (polls >= max_polls) {
      // hand the share to the member that completes the count (a failed swap reloads v)
      if (__hip_atomic_compare_exchange_strong(ctr, &v, v | (1ull << (16 + s)), __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        return 0;
      continue;
    }
    __builtin_amdgcn_s_sleep(16);
    v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ++polls;
  }
}

// Device-coherent (sc1) loads through a buffer resource: they do not hit lines an XCD's L2 or a
// compute unit's cache may hold from before the data was written.
__device__ __forceinline__ u32x4 ld_coherent_16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kWriteThrough));
}

// XOR key of the 16-byte chunk swizzle for LDS rows of 128 bytes: the 8 (32-bank) and 16
// (64-bank, two rows per bank line) consecutive rows read by one operand load hit distinct slots.
__device__ __forceinline__ int key128(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

}  // namespace tt
