// Skinny bf16 products Y = X W^T (X [M, K] with M = batch * S <= a few hundred rows, W [N, K])
// for the synthetic denoiser's projections and lm-head, on gfx950.
//
// The weights dominate the bytes (M = 128 against N, K in the thousands), so the kernel streams W
// once: a work-group owns 64 or 256 output features and up to 128 rows and walks K in chunks of
// 64.
// W and X chunks go straight from global memory into a 3-stage LDS ring (direct-to-LDS loads,
// 16-byte chunks XOR-swizzled per 128-byte row, two chunks in flight, explicit vmcnt waits), and
// Y^T = W X^T is computed with 32x32x16 bf16 MFMA in fp32. When N alone gives too few
// work-groups to fill the GPU, K is also partitioned (fp32 partials + one reduce pass, fixed
// summation order, no atomics).
// Epilogues: fp32 store (logits), Q/K/V scatter into the attention layouts (bf16), and residual
// add (bf16).
#include "common.hpp"
#include "kernels.hpp"

namespace tt {

constexpr int kLM = 128;         // rows per work-group
constexpr int kLK = 64;          // K per chunk (128-byte LDS rows)
constexpr int kLStages = 3;      // LDS ring depth (two chunks in flight)

// Two tile shapes. NARROW: 64 output features, 4 waves = 2 feature blocks x 2 row halves, 72 KB
// of LDS (two work-groups per compute unit) -- for the small projections, with K partitioned
// across work-groups. WIDE: 256 output features, 8 waves of 32 features x all 128 rows, 144 KB of
// LDS -- for the lm-head, so that each X chunk read through L2 serves 4x more weights.
template <int NB>
struct LTile {
  static constexpr int N = NB * 32;                       // features per work-group
  static constexpr int WAVES = NB == 2 ? 4 : NB;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int MB = NB == 2 ? 2 : 4;              // 32-row blocks per wave
  static constexpr int WBYTES = N * kLK * 2;
  static constexpr int XBYTES = kLM * kLK * 2;
  static constexpr int STAGE = WBYTES + XBYTES;
  static constexpr int WLOADS = WBYTES / 1024 / WAVES;    // DMA instructions per wave per chunk
  static constexpr int XLOADS = XBYTES / 1024 / WAVES;
  static constexpr int LOADS = WLOADS + XLOADS;
  static constexpr int LDS = kLStages * STAGE;
};

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

// Chunk of 64 K-columns of W rows n0.. and X rows m0.. -> LDS stage (direct-to-LDS, 16 B per
// lane). Rows past N or M read a valid row instead (their results are never stored); the K range
// [k, k + 64) must lie inside the row.
template <int NB>
__device__ __forceinline__ void linear_dma(char *stage, const LinearParams &p, int n0, int m0,
                                           int k, int wave, int lane) {
  using T = LTile<NB>;
  const uint16_t *w = static_cast<const uint16_t *>(p.w);
  const uint16_t *x = static_cast<const uint16_t *>(p.x);
#pragma unroll
  for (int j = 0; j < T::WLOADS; ++j) {
    const int seg = j * T::WAVES + wave, f = seg * 64 + lane;
    const int r = f / 8, c = (f % 8) ^ key128(f / 8);
    const int n = min(n0 + r, p.N - 1);
    __builtin_amdgcn_global_load_lds(w + (size_t)n * p.K + k + c * 8, TT_LDS_PTR(stage + seg * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < T::XLOADS; ++j) {
    const int seg = j * T::WAVES + wave, f = seg * 64 + lane;
    const int r = f / 8, c = (f % 8) ^ key128(f / 8);
    const int m = min(m0 + r, p.M - 1);
    __builtin_amdgcn_global_load_lds(x + (size_t)m * p.K + k + c * 8,
                                     TT_LDS_PTR(stage + T::WBYTES + seg * 1024), 16, 0, 0);
  }
}

// Partial last chunk (k1 - k < 64 columns) through registers, zero past k1.
template <int NB>
__device__ void linear_tail(char *stage, const LinearParams &p, int n0, int m0, int k, int k1,
                            int tid) {
  using T = LTile<NB>;
  const uint16_t *w = static_cast<const uint16_t *>(p.w);
  const uint16_t *x = static_cast<const uint16_t *>(p.x);
  const u32x4 z = {0u, 0u, 0u, 0u};
  constexpr int NW = T::N * 8 / T::THREADS, NX = kLM * 8 / T::THREADS;
  u32x4 vw[NW], vx[NX];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int f = tid + j * T::THREADS, r = f / 8, c = f % 8;
    const int n = min(n0 + r, p.N - 1);
    vw[j] = k + c * 8 < k1 ? ld_global_16(w + (size_t)n * p.K + k + c * 8) : z;
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int f = tid + j * T::THREADS, r = f / 8, c = f % 8;
    const int m = min(m0 + r, p.M - 1);
    vx[j] = k + c * 8 < k1 ? ld_global_16(x + (size_t)m * p.K + k + c * 8) : z;
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int f = tid + j * T::THREADS, r = f / 8, c = f % 8;
    st_lds_16(stage + r * 128 + ((c ^ key128(r)) << 4), vw[j]);
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int f = tid + j * T::THREADS, r = f / 8, c = f % 8;
    st_lds_16(stage + T::WBYTES + r * 128 + ((c ^ key128(r)) << 4), vx[j]);
  }
}

// Y^T[n][m] += W[n][k] X[m][k] over one LDS chunk: this wave's 32 features x (MB * 32) rows.
template <int NB>
__device__ __forceinline__ void linear_chunk(const char *stage, f32x16 *acc, int nb, int mrow0,
                                             int lane) {
  using T = LTile<NB>;
  const int col = lane & 31, hh = lane >> 5;
  const int wr = nb * 32 + col;
  u32x4 a[4], bx[T::MB][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = ks * 2 + hh;
    a[ks] = ld_lds_16(stage + wr * 128 + ((ch ^ key128(wr)) << 4));
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
      const int xr = mrow0 + mb * 32 + col;
      bx[mb][ks] = ld_lds_16(stage + T::WBYTES + xr * 128 + ((ch ^ key128(xr)) << 4));
    }
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) acc[mb] = mfma32x32x16(a[ks], bx[mb][ks], acc[mb]);
}

template <int NB>
__global__ __launch_bounds__(LTile<NB>::THREADS) void linear_kernel(LinearParams p, int kc) {
  using T = LTile<NB>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int n0 = blockIdx.x * T::N;
  const int m0 = blockIdx.y * kLM;
  const int kz = blockIdx.z;
  const int k0 = kz * kc;
  const int k1 = min(p.K, k0 + kc);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int nb = NB == 2 ? (wave & 1) : wave;
  const int mrow0 = NB == 2 ? (wave >> 1) * 64 : 0;

  f32x16 acc[T::MB];
#pragma unroll
  for (int mb = 0; mb < T::MB; ++mb) acc[mb] = f32x16{};
  const int nk = k1 > k0 ? k1 - k0 : 0;
  const int n_full = nk / kLK;
  const bool tail = nk % kLK != 0;

#pragma unroll
  for (int i = 0; i < kLStages - 1; ++i)
    if (i < n_full) linear_dma<NB>(smem + i * T::STAGE, p, n0, m0, k0 + i * kLK, wave, lane);
  for (int c = 0; c < n_full; ++c) {
    if (c + 1 < n_full) __builtin_amdgcn_s_waitcnt(waitcnt_vm(T::LOADS));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();  // chunk c is in LDS for every wave; the stage of chunk c - 1 is free
    const int cn = c + kLStages - 1;
    if (cn < n_full)
      linear_dma<NB>(smem + (cn % kLStages) * T::STAGE, p, n0, m0, k0 + cn * kLK, wave, lane);
    linear_chunk<NB>(smem + (c % kLStages) * T::STAGE, acc, nb, mrow0, lane);
  }
  if (tail) {
    lds_barrier();
    char *st = smem + (n_full % kLStages) * T::STAGE;
    linear_tail<NB>(st, p, n0, m0, k0 + n_full * kLK, k1, tid);
    lds_barrier();
    linear_chunk<NB>(st, acc, nb, mrow0, lane);
  }

#pragma unroll
  for (int mb = 0; mb < T::MB; ++mb) {
    const int m = m0 + mrow0 + mb * 32 + col;
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

template <int NB>
static hipError_t launch_tile(const LinearParams &p, hipStream_t stream, int kc) {
  using T = LTile<NB>;
  dim3 grid((p.N + T::N - 1) / T::N, (p.M + kLM - 1) / kLM, p.ksplit);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&linear_kernel<NB>),
      hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(linear_kernel<NB>, grid, dim3(T::THREADS), T::LDS, stream, p, kc);
  return hipGetLastError();
}

hipError_t launch_linear(const LinearParams &p, hipStream_t stream) {
  const int kc = ((p.K + p.ksplit - 1) / p.ksplit + kLK - 1) / kLK * kLK;
  hipError_t e = p.wide ? launch_tile<8>(p, stream, kc) : launch_tile<2>(p, stream, kc);
  if (e != hipSuccess || p.ksplit == 1) return e;
  const size_t total = (size_t)p.M * (p.N / 4);
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace tt
