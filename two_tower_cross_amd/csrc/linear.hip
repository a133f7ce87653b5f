// Skinny bf16 products Y = X W^T (X [M, K] with M = batch * S <= a few hundred rows, W [N, K])
// for the synthetic denoiser's projections and lm-head, on gfx950.
//
// The weights dominate the bytes (M = 128 against N, K in the thousands), so the kernel streams W
// once: a work-group owns 64 output features and up to 128 rows, walks K in chunks of 64 with
// X and W chunks double-buffered in LDS (16-byte loads, chunks XOR-swizzled by row & 7), and
// computes Y^T = W X^T with 32x32x16 bf16 MFMA in fp32. Four waves split the tile as 2 feature
// blocks x 2 row halves. When N alone gives too few work-groups to fill the GPU, K is also
// partitioned (fp32 partials + one reduce pass, fixed summation order, no atomics).
// Epilogues: fp32 store (logits), Q/K/V scatter into the attention layouts (bf16), and residual
// add (bf16).
#include "common.hpp"
#include "kernels.hpp"

namespace tt {

constexpr int kLN = 64;
constexpr int kLM = 128;
constexpr int kLK = 64;
constexpr int kLThreads = 256;

__device__ __forceinline__ void epilogue4(const LinearParams &p, int m, int n, f32x4 v) {
  if (p.epi == EPI_F32) {
    *reinterpret_cast<f32x4 *>(p.y + (size_t)m * p.ldy + n) = v;
  } else if (p.epi == EPI_RESIDUAL) {
    const uint16_t *res = static_cast<const uint16_t *>(p.residual) + (size_t)m * p.N + n;
    const uint2 rr = *reinterpret_cast<const uint2 *>(res);
    const float r0 = __uint_as_float(rr.x << 16), r1 = __uint_as_float(rr.x & 0xFFFF0000u);
    const float r2 = __uint_as_float(rr.y << 16), r3 = __uint_as_float(rr.y & 0xFFFF0000u);
    uint2 o;
    o.x = pack_bf16x2(r0 + v[0], r1 + v[1]);
    o.y = pack_bf16x2(r2 + v[2], r3 + v[3]);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.y_bf16) + (size_t)m * p.N + n) = o;
  } else {  // EPI_QKV
    const int b = m / p.S, i = m % p.S;
    const int qn = p.Hq * p.D, kn = p.Hkv * p.D;
    if (n < qn) {
      const int h = n / p.D, d = n % p.D;
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.q) + (((size_t)b * p.S + i) * p.Hq + h) * p.D + d) = o;
    } else if (n < qn + kn) {
      const int g = (n - qn) / p.D, d = (n - qn) % p.D;
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.k_blk) + (((size_t)b * p.Hkv + g) * p.S + i) * p.D + d) = o;
    } else {
      const int g = (n - qn - kn) / p.D, d = (n - qn - kn) % p.D;
      uint16_t *vb = static_cast<uint16_t *>(p.v_blk) + (((size_t)b * p.Hkv + g) * p.D + d) * p.S + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) vb[(size_t)j * p.S] = f32_to_bf16(v[j]);
    }
  }
}

struct LinearRegs {
  u32x4 x[kLM * kLK / 8 / kLThreads];  // 4
  u32x4 w[kLN * kLK / 8 / kLThreads];  // 2
};

__device__ __forceinline__ void linear_fetch(LinearRegs &r, const LinearParams &p, int m0, int n0,
                                             int k, int k1, int tid) {
  const uint16_t *x = static_cast<const uint16_t *>(p.x);
  const uint16_t *w = static_cast<const uint16_t *>(p.w);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int idx = tid + c * kLThreads;
    const int row = idx / 8, ch = idx % 8;
    const int kk = k + ch * 8;
    u32x4 z = {0u, 0u, 0u, 0u};
    r.x[c] = (m0 + row < p.M && kk < k1) ? ld_global_16(x + (size_t)(m0 + row) * p.K + kk) : z;
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int idx = tid + c * kLThreads;
    const int row = idx / 8, ch = idx % 8;
    const int kk = k + ch * 8;
    u32x4 z = {0u, 0u, 0u, 0u};
    r.w[c] = (n0 + row < p.N && kk < k1) ? ld_global_16(w + (size_t)(n0 + row) * p.K + kk) : z;
  }
}

__device__ __forceinline__ void linear_store(const LinearRegs &r, uint16_t *xs, uint16_t *ws,
                                             int tid) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int idx = tid + c * kLThreads;
    const int row = idx / 8, ch = idx % 8;
    st_lds_16(xs + row * kLK + ((ch ^ (row & 7)) << 3), r.x[c]);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int idx = tid + c * kLThreads;
    const int row = idx / 8, ch = idx % 8;
    st_lds_16(ws + row * kLK + ((ch ^ (row & 7)) << 3), r.w[c]);
  }
}

__global__ __launch_bounds__(kLThreads) void linear_kernel(LinearParams p, int kc) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kLM * kLK];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kLN * kLK];
  const int n0 = blockIdx.x * kLN;
  const int m0 = blockIdx.y * kLM;
  const int kz = blockIdx.z;
  const int k0 = kz * kc;
  const int k1 = min(p.K, k0 + kc);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int nb = wave & 1, mh = wave >> 1;

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  const int nchunks = k1 > k0 ? (k1 - k0 + kLK - 1) / kLK : 0;
  LinearRegs regs;
  if (nchunks > 0) {
    linear_fetch(regs, p, m0, n0, k0, k1, tid);
    linear_store(regs, xs[0], ws[0], tid);
    if (nchunks > 1) linear_fetch(regs, p, m0, n0, k0 + kLK, k1, tid);
    __syncthreads();
  }
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const uint16_t *wsb = ws[buf];
    const uint16_t *xsb = xs[buf];
    const int wrow = nb * 32 + col;
#pragma unroll
    for (int ks = 0; ks < kLK / 16; ++ks) {
      const int ch = ks * 2 + hh;
      const u32x4 a = ld_lds_16(wsb + wrow * kLK + ((ch ^ (wrow & 7)) << 3));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int xrow = mh * 64 + mb * 32 + col;
        const u32x4 bx = ld_lds_16(xsb + xrow * kLK + ((ch ^ (xrow & 7)) << 3));
        acc[mb] = mfma32x32x16(a, bx, acc[mb]);
      }
    }
    if (c + 1 < nchunks) linear_store(regs, xs[buf ^ 1], ws[buf ^ 1], tid);
    if (c + 2 < nchunks) linear_fetch(regs, p, m0, n0, k0 + (c + 2) * kLK, k1, tid);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + mh * 64 + mb * 32 + col;
    if (m >= p.M) continue;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int n = n0 + nb * 32 + q4 * 8 + hh * 4;
      if (n >= p.N) continue;
      f32x4 v;
      v[0] = acc[mb][q4 * 4 + 0];
      v[1] = acc[mb][q4 * 4 + 1];
      v[2] = acc[mb][q4 * 4 + 2];
      v[3] = acc[mb][q4 * 4 + 3];
      if (p.ksplit > 1)
        *reinterpret_cast<f32x4 *>(p.part + ((size_t)kz * p.M + m) * p.N + n) = v;
      else
        epilogue4(p, m, n, v);
    }
  }
}

__global__ __launch_bounds__(256) void linear_reduce_kernel(LinearParams p) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.M * (p.N / 4);
  if (e >= total) return;
  const int m = (int)(e / (p.N / 4));
  const int n = (int)(e % (p.N / 4)) * 4;
  f32x4 s = *reinterpret_cast<const f32x4 *>(p.part + (size_t)m * p.N + n);
  for (int z = 1; z < p.ksplit; ++z)
    s += *reinterpret_cast<const f32x4 *>(p.part + ((size_t)z * p.M + m) * p.N + n);
  epilogue4(p, m, n, s);
}

hipError_t launch_linear(const LinearParams &p, hipStream_t stream) {
  const int kc = ((p.K + p.ksplit - 1) / p.ksplit + kLK - 1) / kLK * kLK;
  dim3 grid((p.N + kLN - 1) / kLN, (p.M + kLM - 1) / kLM, p.ksplit);
  hipLaunchKernelGGL(linear_kernel, grid, dim3(kLThreads), 0, stream, p, kc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.ksplit == 1) return e;
  const size_t total = (size_t)p.M * (p.N / 4);
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace tt
