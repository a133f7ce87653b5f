// Skinny bf16 products Y = X W^T (X [M, K] with M = batch * S <= a few hundred rows, W [N, K])
// for the synthetic denoiser's projections and lm-head, on gfx950.
//
// The weights dominate the bytes (M = 128 against N, K in the thousands) and are read once per
// product, so they are stored pre-packed in the A-operand order of v_mfma_f32_32x32x16_bf16: a
// 32-feature x 16-column block is 1 KB, lane-contiguous; 32-feature slabs are grouped by 8 and a
// group's blocks are stored step-major (see pack_weight_kernel). A work-group owns NB slabs of one
// group (64 or 256 features) and all rows of an M tile, and walks its K range in chunks of 64
// columns:
//   * W chunks (one 32 KB run for 256 features, four 2 KB runs for 64) stream into an LDS ring
//     with non-temporal direct-to-LDS loads (several chunks in flight: a compute unit keeps
//     ~64 KB of loads in flight, and deeper rings only queue behind that limit);
//   * X chunks (128 rows x 64 columns, re-read by every work-group, so served by L2) go through a
//     second ring, 16-byte chunks XOR-swizzled per 128-byte row, deep enough to cover the L2
//     latency under load;
//   * Y^T = W X^T with 32x32x16 bf16 MFMA in fp32; the W operand reads are lane-contiguous.
// When N alone gives too few work-groups to fill the GPU, K is also partitioned: fp32 partials,
// written through to memory and summed in partition order (no floating-point atomics), inside the
// product kernel once a tile's partitions have arrived at its counter (each sums a share of the
// tile's rows), or by a second kernel.
// Epilogues: fp32 store (logits), Q/K/V scatter into the attention layouts (bf16), residual add
// (bf16), and the unmasking triples of the lm-head (lm_unmask_kernel when the logits are not
// kept: persistent, 256-feature tiles computed in pairs that share each 32-column X chunk, the
// pairs' chunks as one ring stream).
#include <algorithm>
#include <mutex>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "launch_util.hpp"
#include "triple.hpp"

namespace tt {

#ifdef TT_PHASE_STAMPS
__device__ unsigned long long linear_phase_stamps[8192][8];
#endif

constexpr int kLM = 128;         // rows per work-group
constexpr int kLK = 64;          // K columns per chunk
// Cache policy of the weight streams. The lm-head's weight (hundreds of MB, read once per step) is
// streamed non-temporally (about 20% more read bandwidth than the default policy for a streaming
// read on gfx950). The projections' weights keep the default policy: a step reads every layer's
// W_qkv and W_o once (216 MB at hidden 2048 and 6 layers), and with the KV caches and the
// lm-head read non-temporally they stay in the 256 MB last-level cache from one step to the next
// (the 32K-context loop ran 1.9% faster than with non-temporal projection weights). The 256-feature
// tiles (products with a vocabulary-sized N: the lm-head with its logits kept) stream their weight
// non-temporally. X stays cached: every work-group reads it.
constexpr int kNonTemporal = 2;
constexpr int kProjectionWeights = 0;

// Two tile shapes, 8 waves each (a wave issues a 1 KB load only every ~100 cycles and stalls
// meanwhile, so the ring's loads are spread over as many waves as possible). NB = 2: 64 output
// features, the waves are 2 slabs x 4 blocks of 32 rows, a 6-deep W ring (48 KB) and a 4-deep X
// ring (64 KB) -- for the projections, with K partitioned across work-groups. NB = 8: 256 output
// features, 8 waves of one slab x all 128 rows, 3-deep rings (96 + 48 KB) -- for the lm-head,
// where each X chunk read through L2 then serves 4x more weights.
template <int NB>
struct LTile {
  static constexpr int N = NB * 32;                       // features per work-group
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int MB = NB == 2 ? 1 : 4;              // 32-row blocks per wave
  static constexpr int WST = NB == 2 ? 6 : 3;             // W ring depth
  static constexpr int XST = NB == 2 ? 4 : 3;             // X ring depth (<= WST)
  static constexpr int WBYTES = NB * 4096;                // one W chunk
  static constexpr int XBYTES = kLM * kLK * 2;            // one X chunk
  static constexpr int XBASE = WST * WBYTES;
  static constexpr int WLOADS = NB * 4 / WAVES;           // DMA instructions per wave per chunk
  static constexpr int XLOADS = XBYTES / 1024 / WAVES;
  static constexpr int LDS = XBASE + XST * XBYTES;
  // DMA instructions issued after X(i) once X(i) is due (see linear_kernel)
  static constexpr int AFTER = (XST - 2) * (WLOADS + XLOADS);
};

// ----------------------------------------------------------------------------- weight packing
// Packed layout: slabs of 32 features, grouped by 8 (group gi = nb / 8 of gsize = min(8, NS - 8 gi)
// slabs, NS = ceil(N / 32)); 1 KB unit U = 8 gi Ks + s gsize + nb % 8 holds the 32 x 16 block
// (slab nb, K step s), Ks = ceil(K / 16):
// P[(U * 64 + lane) * 8 + e] = W[nb * 32 + lane % 32][s * 16 + (lane / 32) * 8 + e], zero outside W.
// One thread per 16-byte piece, read in slab order.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t *w, int N, int K,
                                                          uint16_t *out, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int Ks = (K + 15) / 16;
  const int NS = (N + 31) / 32;
  const int lane = (int)(u % 64);
  const int64_t blk = u / 64;
  const int s = (int)(blk % Ks);
  const int nb = (int)(blk / Ks);
  const int gi = nb / 8, gsize = min(8, NS - 8 * gi);
  const int64_t unit = (int64_t)8 * gi * Ks + (int64_t)s * gsize + nb % 8;
  const int n = nb * 32 + lane % 32;
  const int k0 = s * 16 + (lane / 32) * 8;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (n < N) {
    const uint16_t *row = w + (size_t)n * K;
    if (k0 + 8 <= K) {
      v = ld_global_16(row + k0);  // K % 8 == 0: 16-byte aligned
    } else {
      uint16_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = k0 + i < K ? row[k0 + i] : (uint16_t)0;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
    }
  }
  *reinterpret_cast<u32x4 *>(out + ((size_t)unit * 64 + lane) * 8) = v;
}

hipError_t launch_pack_weight(const void *w, int N, int K, void *out, hipStream_t stream) {
  const int64_t units = (int64_t)((N + 31) / 32) * ((K + 15) / 16) * 64;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t *>(w), N, K, static_cast<uint16_t *>(out),
                     units);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------- epilogues
__device__ __forceinline__ uint2 load_residual4(const LinearParams &p, int m, int n) {
  return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.residual) +
                                          (size_t)m * p.N + n);
}

// rr: the residual's 4 bf16 at (m, n) when already loaded (EPI_RESIDUAL), else ignored.
__device__ __forceinline__ void epilogue4(const LinearParams &p, int m, int n, f32x4 v,
                                          const uint2 *rr_pre = nullptr) {
  if (p.epi == EPI_F32) {
    *reinterpret_cast<f32x4 *>(p.y + (size_t)m * p.ldy + n) = v;
  } else if (p.epi == EPI_RESIDUAL) {
    const uint2 rr = rr_pre ? *rr_pre : load_residual4(p, m, n);
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

// ------------------------------------------------------------------------------------ loads
// Buffer resource over the packed block of slab group gi (gsize x Ks KB); loads past it return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(const void *w, int gi, int gsize,
                                                             int Ks) {
  const char *base = static_cast<const char *>(w) + (size_t)8 * gi * Ks * 1024;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, gsize * Ks * 1024,
                                           0x00020000);
}

// W chunk c (K columns 64c .. 64c + 63, steps 4c .. 4c + 3) of this work-group's NB slabs, slots
// gs0 .. gs0 + NB - 1 of the group behind `gr` -> W stage (block-major: slab j at j * 4 KB, step i
// at i * 1 KB). For a whole group (NB = 8) the chunk is one contiguous 32 KB run of the packed
// weight. Slots past the group's gsize (features past N), and every load when real is false, go
// through `none` (a resource with no records: nothing moves); steps past Ks fall outside `gr`.
template <int NB>
__device__ __forceinline__ void w_dma(char *stage, __amdgpu_buffer_rsrc_t gr, int gsize, int gs0,
                                      bool real, __amdgpu_buffer_rsrc_t none, int c, int wave,
                                      int lane) {
  using T = LTile<NB>;
#pragma unroll
  for (int j = 0; j < T::WLOADS; ++j) {
    const int t = j * T::WAVES + wave;  // instruction index: slab t / 4, step t % 4
    const int gs = gs0 + t / 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(real && gs < gsize ? gr : none,
                                             TT_LDS_PTR(stage + t * 1024), 16, lane * 16,
                                             ((4 * c + t % 4) * gsize + gs) * 1024, 0,
                                             NB == 2 ? kProjectionWeights : kNonTemporal);
  }
}

// X chunk (rows m0 .. m0 + 127, columns k .. k + 63) -> X stage (direct-to-LDS through a buffer
// resource over X, so that no load leaves the tensor). Rows past M read row M - 1 instead (their
// results are never stored).
template <int NB>
__device__ __forceinline__ void x_dma(char *stage, __amdgpu_buffer_rsrc_t xr, const LinearParams &p,
                                      int m0, int k, int wave, int lane) {
  using T = LTile<NB>;
#pragma unroll
  for (int j = 0; j < T::XLOADS; ++j) {
    const int seg = j * T::WAVES + wave, f = seg * 64 + lane;
    const int r = f / 8, c = (f % 8) ^ key128(f / 8);
    const int m = min(m0 + r, p.M - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, TT_LDS_PTR(stage + seg * 1024), 16,
                                             (m * p.K + k + c * 8) * 2, 0, 0, 0);
  }
}

// Partial last X chunk (k1 - k < 64 columns) through registers, zero past k1.
template <int NB>
__device__ void x_tail(char *stage, const LinearParams &p, int m0, int k, int k1, int tid) {
  using T = LTile<NB>;
  const uint16_t *x = static_cast<const uint16_t *>(p.x);
  const u32x4 z = {0u, 0u, 0u, 0u};
  constexpr int NX = kLM * 8 / T::THREADS;
  u32x4 vx[NX];
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int f = tid + j * T::THREADS, r = f / 8, c = f % 8;
    const int m = min(m0 + r, p.M - 1);
    vx[j] = k + c * 8 < k1 ? ld_global_16(x + (size_t)m * p.K + k + c * 8) : z;
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int f = tid + j * T::THREADS, r = f / 8, c = f % 8;
    st_lds_16(stage + r * 128 + ((c ^ key128(r)) << 4), vx[j]);
  }
}

// Y^T[n][m] += W[n][k] X[m][k] over one chunk: this wave's slab (32 features) x (MB * 32) rows.
template <int NB>
__device__ __forceinline__ void linear_chunk(const char *ws, const char *xs, f32x16 *acc, int slab,
                                             int mrow0, int lane) {
  using T = LTile<NB>;
  const int col = lane & 31, hh = lane >> 5;
  u32x4 a[4], bx[T::MB][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    a[ks] = ld_lds_16(ws + slab * 4096 + ks * 1024 + lane * 16);
    const int ch = ks * 2 + hh;
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
      const int xr = mrow0 + mb * 32 + col;
      bx[mb][ks] = ld_lds_16(xs + xr * 128 + ((ch ^ key128(xr)) << 4));
    }
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) acc[mb] = mfma32x32x16(a[ks], bx[mb][ks], acc[mb]);
}

// Fused lm-head epilogue feeding the unmasking: the fp32 tile [128 rows][256 features] is in LDS
// (16-byte chunk c of row r at chunk slot c ^ (r & 63)). Optionally stores it as logits; then
// four threads per row each reduce 64 consecutive features to (maximum, its first position, sum
// of exp(y - max)), merge their triples with two lane exchanges, and the first writes the row's
// triple for this tile. Rows committed already (masked == 0, read at kernel start into `live`)
// write nothing. A thread whose features run past the vocabulary takes them one by one.
template <int NB>
__device__ void unmask_epilogue(const LinearParams &p, const float *tile, int m0, int n0, int tid,
                                bool live) {
  using T = LTile<NB>;
  static_assert(T::THREADS == 4 * kLM, "four threads per row");
  constexpr int NCH = T::N / 4;
  if (p.y) {
    for (int u = tid; u < kLM * NCH; u += T::THREADS) {
      const int r = u / NCH, c = u % NCH;
      const int m = m0 + r, nn = n0 + c * 4;
      if (m >= p.M || nn >= p.N) continue;
      *reinterpret_cast<f32x4 *>(p.y + (size_t)m * p.ldy + nn) =
          *reinterpret_cast<const f32x4 *>(tile + r * T::N + ((c ^ (r & (NCH - 1))) << 2));
    }
  }
  const int r = tid >> 2, q = tid & 3;
  const int m = m0 + r;
  Triple t = empty_triple();
  const int nq = n0 + q * (NCH / 4) * 4;  // first feature of this thread's 64
  if (live && nq + (NCH / 4) * 4 <= p.N) {
    // All 64 features inside the vocabulary: the maximum by a max tree, its first position by a
    // backward scan, then the sum of exp2(y log2 e - max log2 e) in four independent chains.
    f32x4 v[NCH / 4];
    float m4[NCH / 4];
#pragma unroll
    for (int j = 0; j < NCH / 4; ++j) {
      const int c = q * (NCH / 4) + j;
      v[j] = *reinterpret_cast<const f32x4 *>(tile + r * T::N + ((c ^ (r & (NCH - 1))) << 2));
      m4[j] = fmaxf(fmaxf(v[j][0], v[j][1]), fmaxf(v[j][2], v[j][3]));
    }
#pragma unroll
    for (int w = NCH / 8; w >= 1; w /= 2)
#pragma unroll
      for (int j = 0; j < w; ++j) m4[j] = fmaxf(m4[j], m4[j + w]);
    const float mx = m4[0];
    if (mx > -INFINITY) {  // else no feature is above -inf (or all are NaN): the empty triple
      int idx = 0;
#pragma unroll
      for (int j = NCH / 4 - 1; j >= 0; --j)
#pragma unroll
        for (int e = 3; e >= 0; --e) idx = v[j][e] == mx ? j * 4 + e : idx;
      constexpr float kLog2e = 1.4426950408889634f;
      const float mc = mx * kLog2e;
      float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NCH / 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] += __builtin_amdgcn_exp2f(fmaf(v[j][e], kLog2e, -mc));
      t.m = mx;
      t.idx = nq + idx;
      t.z = (z[0] + z[1]) + (z[2] + z[3]);
    }
  } else if (live) {
    f32x4 v[NCH / 4];
#pragma unroll
    for (int j = 0; j < NCH / 4; ++j) {
      const int c = q * (NCH / 4) + j;
      v[j] = *reinterpret_cast<const f32x4 *>(tile + r * T::N + ((c ^ (r & (NCH - 1))) << 2));
    }
#pragma unroll
    for (int j = 0; j < NCH / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = n0 + (q * (NCH / 4) + j) * 4 + e;
        if (n < p.N && v[j][e] > t.m) {
          t.m = v[j][e];
          t.idx = n;
        }
      }
    float z = 0.f;
    if (t.m > -INFINITY) {
#pragma unroll
      for (int j = 0; j < NCH / 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n0 + (q * (NCH / 4) + j) * 4 + e < p.N) z += __expf(v[j][e] - t.m);
    }
    t.z = z;
  }
  t = merge(t, shfl_xor_triple(t, 1));
  t = merge(t, shfl_xor_triple(t, 2));
  if (q == 0 && live) {
    float *o = p.triples + ((size_t)m * ((p.N + T::N - 1) / T::N) + blockIdx.x) * 4;
    o[0] = t.m;
    o[1] = __int_as_float(t.idx);
    o[2] = t.z;
  }
}

// Sum of the K partials of outputs (m, n .. n + 3) in partition order, 8 partials requested at a
// time (clamped loads, no branches, so that they are all in flight together), then the epilogue.
// COHERENT: the partials were written by other work-groups of the same kernel (the in-kernel
// merge), so they are read with device-coherent loads (sc1) through a resource over the partials
// (which then span less than 4 GiB).
template <bool COHERENT>
__device__ __forceinline__ void reduce_partials4(const LinearParams &p, int m, int n) {
  const float *src = p.part + (size_t)m * p.N + n;
  const size_t zstride = (size_t)p.M * p.N;
  const __amdgpu_buffer_rsrc_t pr =
      buf_rsrc(p.part, COHERENT ? (uint32_t)(p.ksplit * zstride * 4) : 0u);
  uint2 rr = {0u, 0u};
  if (p.epi == EPI_RESIDUAL) rr = load_residual4(p, m, n);  // in flight with the partials
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < p.ksplit; z0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t e = (size_t)min(z0 + j, p.ksplit - 1) * zstride;
      if (COHERENT)
        v[j] = __builtin_bit_cast(f32x4, ld_coherent_16(pr, (uint32_t)(((size_t)m * p.N + n + e) * 4)));
      else
        v[j] = *reinterpret_cast<const f32x4 *>(src + e);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (z0 + j < p.ksplit) s = z0 + j == 0 ? v[j] : s + v[j];
  }
  epilogue4(p, m, n, s, &rr);
}

// Grid: (ceil(N / (32 NB)), ceil(M / 128), ksplit); the work-group's K range is chunks
// [z * cpz, min(nch, (z + 1) * cpz)) of the ceil(K / 64) chunks.
template <int NB>
__global__ __launch_bounds__(LTile<NB>::THREADS) void linear_kernel(LinearParams p, int cpz) {
  using T = LTile<NB>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  TT_STAMPS_DECL;
  TT_STAMP(0);  // phase stamps (profiling build): start
  TT_CYCLES(6);
  const int nb0 = blockIdx.x * NB;
  const int m0 = blockIdx.y * kLM;
  const int kz = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int slab = NB == 2 ? (wave & 1) : wave;
  const int mrow0 = NB == 2 ? (wave >> 1) * 32 : 0;
  // Fused unmasking: whether this thread's epilogue row (m0 + tid / 4) is still masked, read now
  // so that the load is long done when the epilogue needs it.
  uint32_t row_flag = 0;
  if (NB == 8 && p.epi == EPI_UNMASK) row_flag = p.masked[min(m0 + (tid >> 2), p.M - 1)];

  const int nch = (p.K + kLK - 1) / kLK;
  const int Ks = (p.K + 15) / 16;
  const int c0 = kz * cpz;
  const int n = max(0, min(nch, c0 + cpz) - c0);   // chunks of this work-group
  const bool tail = p.K % kLK != 0 && c0 + n == nch;  // its last chunk is partial
  const int n_dma_x = tail ? n - 1 : n;            // chunks whose X comes by DMA

  // This tile's slabs are slots nb0 % 8 .. of slab group nb0 / 8 (8 % NB == 0); slots past the
  // group's size (the last tile of an N that is not a multiple of the tile width) load nothing.
  const int nslabs = (p.N + 31) / 32;
  const int gi = nb0 / 8, gs0 = nb0 % 8, gsize = min(8, nslabs - 8 * gi);
  const __amdgpu_buffer_rsrc_t gr = group_rsrc(p.w, gi, gsize, Ks);

  f32x16 acc[T::MB];
#pragma unroll
  for (int mb = 0; mb < T::MB; ++mb) acc[mb] = f32x16{};

  char *wring = smem;
  char *xring = smem + T::XBASE;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(p.x), (short)0, p.M * p.K * 2, 0x00020000);
  // Every step issues the same DMA: W(c) (c = step + WST - 1) and X(c') (c' = step + XST - 1).
  // Chunks past the end are still "loaded" (phantom loads that move no data, into the stage they
  // would occupy, which nobody reads again); so the number of DMA instructions issued after X(i)
  // when chunk i is due is always T::AFTER and one vmcnt immediate serves every step. W(i) is
  // issued before X(i) (WST >= XST), so the wait covers both.
  // Phantom loads go through a resource of zero records: out of range, so they move no data
  // (the LDS stage gets zeros) while still counting as issued loads.
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(p.x), (short)0, 0, 0x00020000);
  auto w_issue = [&](int c) {
    w_dma<NB>(wring + (c % T::WST) * T::WBYTES, gr, gsize, gs0, c < n, none, c0 + min(c, n - 1),
              wave, lane);
  };
  auto x_issue = [&](int c) {
    x_dma<NB>(xring + (c % T::XST) * T::XBYTES, c < n_dma_x ? xr : none, p, m0,
              c < n_dma_x ? (c0 + c) * kLK : 0, wave, lane);
  };
  if (n > 0) {
    // Prologue: W(0 .. WST-XST-1), then the pairs W(WST-XST+j), X(j) for j < XST-1, so that
    // W(0 .. WST-2) and X(0 .. XST-2) are in flight and step 0 goes on with W(WST-1), X(XST-1).
#pragma unroll
    for (int c = 0; c < T::WST - T::XST; ++c) w_issue(c);
#pragma unroll
    for (int j = 0; j < T::XST - 1; ++j) {
      w_issue(T::WST - T::XST + j);
      x_issue(j);
    }
  }
  for (int i = 0; i < n; ++i) {
    if (i < n_dma_x) __builtin_amdgcn_s_waitcnt(waitcnt_vm(T::AFTER));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();  // chunk i is in LDS for every wave; the stages of chunk i - 1 are free
    if (i == 0) TT_STAMP(1);  // chunk 0 has landed
    w_issue(i + T::WST - 1);
    x_issue(i + T::XST - 1);
    char *xs = xring + (i % T::XST) * T::XBYTES;
    if (i >= n_dma_x) {  // the partial last chunk: X through registers, zero past K
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no DMA into this stage is still in flight
      x_tail<NB>(xs, p, m0, (c0 + i) * kLK, p.K, tid);
      lds_barrier();
    }
    linear_chunk<NB>(wring + (i % T::WST) * T::WBYTES, xs, acc, slab, mrow0, lane);
  }

  // Epilogue: the fp32 tile [128 rows][32 NB features] goes through LDS (16-byte chunks of row r
  // XOR-swizzled by r, so that the 32 rows one store touches fall in distinct banks), then every
  // thread handles 4 consecutive features of one row, consecutive threads along the row: the global
  // stores cover whole rows instead of 32-byte pieces of 32 rows.
  constexpr int NCH = T::N / 4;  // 16-byte chunks per tile row
  TT_STAMP(2);  // the K loop is done
  // The last steps issued phantom loads into the rings (zeros); they must land before the rings
  // are reused for the output tile.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();                 // every wave is done with the rings
  TT_STAMP(3);
  float *tile = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int mb = 0; mb < T::MB; ++mb) {
    const int r = mrow0 + mb * 32 + col;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ch = (slab * 32 + q4 * 8 + hh * 4) / 4;
      const f32x4 v = {acc[mb][q4 * 4 + 0], acc[mb][q4 * 4 + 1], acc[mb][q4 * 4 + 2],
                       acc[mb][q4 * 4 + 3]};
      *reinterpret_cast<f32x4 *>(tile + r * T::N + ((ch ^ (r & (NCH - 1))) << 2)) = v;
    }
  }
  lds_barrier();
  const int n0 = nb0 * 32;
  if constexpr (NB == 8) {
    if (p.epi == EPI_UNMASK) {
      unmask_epilogue<NB>(p, tile, m0, n0, tid, m0 + (tid >> 2) < p.M && defer_use(row_flag) != 0);
      return;
    }
  }
  // K partials: rows m0 .. of partition kz, written through (the reduce reads them from any XCD)
  const __amdgpu_buffer_rsrc_t pr =
      buf_rsrc(p.part + ((size_t)kz * p.M + m0) * p.N, (uint32_t)(min(kLM, p.M - m0) * p.N * 4));
  for (int u = tid; u < kLM * NCH; u += T::THREADS) {
    const int r = u / NCH, c = u % NCH;
    const int m = m0 + r, nn = n0 + c * 4;
    if (m >= p.M || nn >= p.N) continue;
    const f32x4 v = *reinterpret_cast<const f32x4 *>(tile + r * T::N + ((c ^ (r & (NCH - 1))) << 2));
    if (p.ksplit > 1)
      st_wt_16(pr, (uint32_t)((r * p.N + nn) * 4), __builtin_bit_cast(u32x4, v));
    else
      epilogue4(p, m, nn, v);
  }
  if (p.ksplit > 1 && p.sync) {
    // Merge of the K partials inside the kernel: once the tile's ksplit work-groups have stored
    // their partials and arrived at the tile's counter, partition kz sums rows
    // [kz * rows / ksplit, (kz + 1) * rows / ksplit) of the tile, as linear_reduce_kernel would
    // (and the shares of partitions that gave up waiting, when it is the last to arrive).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's partial stores have completed
    __syncthreads();
    uint32_t *shares = reinterpret_cast<uint32_t *>(smem + T::LDS - 4);
    if (tid == 0)
      shares[0] = group_arrive(p.sync + (blockIdx.x + gridDim.x * blockIdx.y) * kSyncWords,
                               p.sync_tag, p.ksplit, kz, p.sync_polls);
    __syncthreads();
    const int rows = min(kLM, p.M - m0);
    for (uint32_t left = __builtin_amdgcn_readfirstlane(shares[0]); left != 0; left &= left - 1) {
      const int sh = __builtin_ctz(left);
      const int lo = sh * rows / p.ksplit, hi = (sh + 1) * rows / p.ksplit;
      for (int u = tid; u < (hi - lo) * NCH; u += T::THREADS) {
        const int nn = n0 + (u % NCH) * 4;
        if (nn < p.N) reduce_partials4<true>(p, m0 + lo + u / NCH, nn);
      }
    }
  }
  TT_STAMP(4);  // stores issued
  TT_STAMP_DRAINED(5);  // stores done
  TT_CYCLES(7);
  TT_STAMPS_STORE(linear_phase_stamps,
                  blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
}

// ---------------------------------------------------------------- lm-head fused with unmasking
// The step's lm-head when its logits are not kept. Persistent: work-group g of a 128-row block
// takes the 256-feature tiles g, g + G, g + 2G, ... (G = gridDim.x) two at a time: the tiles of a
// pair are computed together, chunk by chunk of 32 K columns, so every X chunk read through L2
// serves both (X is re-read per tile pair instead of per tile: 1 instead of 2 X bytes per 4 weight
// bytes), and the pairs stream through the ring as one sequence, so the first chunks of the next
// pair are in flight while the (max, first argmax, sum of exp) of the previous one are reduced.
// The reduction reads the accumulators in registers (no staging of the fp32 tiles): each lane's 16
// features of a row, the lane pair (the other 16 of the wave's 32-feature slab), then the 8 slabs
// through an LDS area after the rings.
struct LPair {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KC = 32;                      // K columns per chunk (2 MFMA K-steps)
  static constexpr int WST = 3, XST = 3;             // ring depths
  static constexpr int TBYTES = 8 * 2 * 1024;        // one tile's chunk: 8 slabs x 2 steps x 1 KB
  static constexpr int WBYTES = 2 * TBYTES;          // both tiles
  static constexpr int XBYTES = kLM * KC * 2;        // 128 rows x 64 bytes
  static constexpr int XBASE = WST * WBYTES;
  static constexpr int RED = XBASE + XST * XBYTES;
  static constexpr int REDBYTES = 2 * 8 * kLM * 3 * 4;  // [tile][slab][row] (m, idx, z)
  static constexpr int LDS = RED + REDBYTES;
  static constexpr int WLOADS = WBYTES / 1024 / WAVES;  // DMA instructions per wave per chunk
  static constexpr int XLOADS = XBYTES / 1024 / WAVES;
  static constexpr int AFTER = (XST - 2) * (WLOADS + XLOADS);
};
static_assert(LPair::WST == LPair::XST, "the prologue issues W and X chunks in pairs");
static_assert(LPair::LDS <= 160 * 1024, "LDS");

// XOR key of the 16-byte chunk swizzle for LDS rows of 64 bytes: the 8 (32-bank) and 16 (64-bank)
// consecutive rows read by one operand load hit distinct slots.
__device__ __forceinline__ int key64(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// X chunk (rows m0 .. m0 + 127, columns k .. k + 31) -> X stage, direct-to-LDS through a buffer
// resource over X (16-byte slot q of row r holds columns k + 8 (q ^ key64(r)) ..); rows past M
// read row M - 1 (their results are never stored).
__device__ __forceinline__ void x_dma32(char *stage, __amdgpu_buffer_rsrc_t xr, const LinearParams &p,
                                        int m0, int k, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < LPair::XLOADS; ++j) {
    const int seg = j * LPair::WAVES + wave, f = seg * 64 + lane;
    const int r = f >> 2, c = (f & 3) ^ key64(r);
    const int m = min(m0 + r, p.M - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, TT_LDS_PTR(stage + seg * 1024), 16,
                                             (m * p.K + k + c * 8) * 2, 0, 0, 0);
  }
}

// Partial last X chunk (k1 - k < 32 columns) through registers, zero past k1 (K % 8 == 0).
__device__ void x_tail32(char *stage, const LinearParams &p, int m0, int k, int k1, int tid) {
  const uint16_t *x = static_cast<const uint16_t *>(p.x);
  const u32x4 z = {0u, 0u, 0u, 0u};
  static_assert(kLM * 4 == LPair::THREADS, "one 16-byte slot per thread");
  const int r = tid >> 2, q = tid & 3, c = q ^ key64(r);
  const int m = min(m0 + r, p.M - 1);
  const u32x4 v = k + c * 8 < k1 ? ld_global_16(x + (size_t)m * p.K + k + c * 8) : z;
  st_lds_16(stage + r * 64 + q * 16, v);
}

// One 32-column chunk of both tiles: this wave's slab (32 features) of each tile x 128 rows;
// the X operand fragments are read once and used for both tiles.
__device__ __forceinline__ void pair_chunk(const char *ws, const char *xs, f32x16 (*acc)[4],
                                           int wave, int lane) {
  const int col = lane & 31, hh = lane >> 5;
  u32x4 a[2][2], bx[4][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      a[t][ks] = ld_lds_16(ws + t * LPair::TBYTES + (wave * 2 + ks) * 1024 + lane * 16);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int xr = mb * 32 + col, ch = ks * 2 + hh;
      bx[mb][ks] = ld_lds_16(xs + xr * 64 + ((ch ^ key64(xr)) << 4));
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[t][mb] = mfma32x32x16(a[t][ks], bx[mb][ks], acc[t][mb]);
}

// (max, first argmax, sum of exp(y - max)) of the 16 accumulator values a lane holds for one
// row: register i is feature f0 + (i / 4) * 8 + i % 4; features at or past N are left out.
__device__ __forceinline__ Triple lane_triple(const f32x16 &a, int f0, int N) {
  float v[16];
  const bool full = f0 + 28 < N;  // (the lane's last feature is f0 + 27)
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = full || f0 + (i / 4) * 8 + i % 4 < N ? a[i] : -INFINITY;
  float m4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) m4[j] = fmaxf(fmaxf(v[4 * j], v[4 * j + 1]), fmaxf(v[4 * j + 2], v[4 * j + 3]));
  const float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  Triple t = empty_triple();
  if (mx > -INFINITY) {
    int idx = 0;
#pragma unroll
    for (int i = 15; i >= 0; --i) idx = v[i] == mx ? (i / 4) * 8 + i % 4 : idx;
    constexpr float kLog2e = 1.4426950408889634f;
    const float mc = mx * kLog2e;
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      z0 += __builtin_amdgcn_exp2f(fmaf(v[i], kLog2e, -mc));
      z1 += __builtin_amdgcn_exp2f(fmaf(v[i + 1], kLog2e, -mc));
    }
    t.m = mx;
    t.idx = f0 + idx;
    t.z = z0 + z1;
  }
  return t;
}

__global__ __launch_bounds__(LPair::THREADS) void lm_unmask_kernel(LinearParams p, int ntiles) {
  using T = LPair;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int m0 = blockIdx.y * kLM;
  const int G = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  // the final merge: four threads per row; whether the row is still masked, requested now and
  // used only at the first pair's merge (the ring does not wait for it)
  const int rr = tid >> 2, q = tid & 3;
  const uint32_t flag = p.masked[min(m0 + rr, p.M - 1)];

  const int mine = (ntiles - (int)blockIdx.x + G - 1) / G;  // tiles of this work-group
  const int pairs = (mine + 1) / 2;                       // pair j: tiles j-th and (j+1)-th of mine
  const int nch = (p.K + T::KC - 1) / T::KC;
  const int Ks = (p.K + 15) / 16;
  const int nslabs = (p.N + 31) / 32;
  const bool tail = p.K % T::KC != 0;  // the last chunk of every pair is partial
  const int total = pairs * nch;

  f32x16 acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[t][mb] = f32x16{};

  char *wring = smem;
  char *xring = smem + T::XBASE;
  float *red = reinterpret_cast<float *>(smem + T::RED);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(p.x), (short)0, p.M * p.K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(p.x), (short)0, 0, 0x00020000);
  // Tile t (0, 1) of pair j (the whole slab group of 256 features), or -1 past the last tile.
  auto pair_tile = [&](int j, int t) {
    const int tile = (int)blockIdx.x + (2 * j + t) * G;
    return tile < ntiles ? tile : -1;
  };
  // Chunk g of the sequence is chunk g % nch of pair g / nch. As in linear_kernel every step
  // issues the same DMA (phantom loads through `none` past the end and for a pair's missing
  // second tile), so T::AFTER is exact for every chunk whose X comes by DMA. Instruction i of a
  // wave loads 1 KB block (slab u / 2, step u % 2), u = (i % 2) * 8 + wave, of tile i / 2.
  auto w_issue = [&](int g) {
    const int gg = min(g, total - 1);
    const int j = gg / nch, c = gg % nch;
#pragma unroll
    for (int i = 0; i < T::WLOADS; ++i) {
      const int t = i >> 1, u = (i & 1) * 8 + wave, slab = u >> 1, step = u & 1;
      const int tile = pair_tile(j, t);
      const int gsize = tile >= 0 ? min(8, nslabs - 8 * tile) : 0;
      const bool real = g < total && slab < gsize;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          real ? group_rsrc(p.w, tile, gsize, Ks) : none,
          TT_LDS_PTR(wring + (g % T::WST) * T::WBYTES + t * T::TBYTES + (slab * 2 + step) * 1024),
          16, lane * 16, real ? ((2 * c + step) * gsize + slab) * 1024 : 0, 0, kNonTemporal);
    }
  };
  auto x_issue = [&](int g) {
    const int c = g % nch;
    const bool real = g < total && !(tail && c == nch - 1);
    x_dma32(xring + (g % T::XST) * T::XBYTES, real ? xr : none, p, m0, real ? c * T::KC : 0, wave,
            lane);
  };
  if (total > 0) {
#pragma unroll
    for (int j = 0; j < T::XST - 1; ++j) {
      w_issue(j);
      x_issue(j);
    }
  }
  for (int g = 0; g < total; ++g) {
    const int c = g % nch;
    const bool x_by_regs = tail && c == nch - 1;
    if (!x_by_regs) __builtin_amdgcn_s_waitcnt(waitcnt_vm(T::AFTER));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();  // chunk g is in LDS for every wave; the stages of chunk g - 1 are free
    w_issue(g + T::WST - 1);
    x_issue(g + T::XST - 1);
    char *xs = xring + (g % T::XST) * T::XBYTES;
    if (x_by_regs) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no DMA into this stage is still in flight
      x_tail32(xs, p, m0, c * T::KC, p.K, tid);
      lds_barrier();
    }
    pair_chunk(wring + (g % T::WST) * T::WBYTES, xs, acc, wave, lane);
    if (c == nch - 1) {
      // Pair done: per tile, this wave's slab, per row: lane triple, lane pair, then the 8 slabs.
      const int j = g / nch;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int tile = pair_tile(j, t);
        const int f0 = max(tile, 0) * 256 + wave * 32 + hh * 4;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          Triple tr = lane_triple(acc[t][mb], f0, tile >= 0 ? p.N : 0);
          tr = merge(tr, shfl_xor_triple(tr, 32));
          if (hh == 0) {
            float *o = red + ((t * 8 + wave) * kLM + mb * 32 + col) * 3;
            o[0] = tr.m;
            o[1] = __int_as_float(tr.idx);
            o[2] = tr.z;
          }
          acc[t][mb] = f32x16{};
        }
      }
      lds_barrier();
      const bool live = m0 + rr < p.M && defer_use(flag) != 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int tile = pair_tile(j, t);
        Triple tr, u;
        const float *a = red + ((t * 8 + 2 * q) * kLM + rr) * 3;
        const float *b = red + ((t * 8 + 2 * q + 1) * kLM + rr) * 3;
        tr.m = a[0];
        tr.idx = __float_as_int(a[1]);
        tr.z = a[2];
        u.m = b[0];
        u.idx = __float_as_int(b[1]);
        u.z = b[2];
        tr = merge(tr, u);
        tr = merge(tr, shfl_xor_triple(tr, 1));
        tr = merge(tr, shfl_xor_triple(tr, 2));
        if (q == 0 && live && tile >= 0) {
          float *o = p.triples + ((size_t)(m0 + rr) * ntiles + tile) * 4;
          o[0] = tr.m;
          o[1] = __int_as_float(tr.idx);
          o[2] = tr.z;
        }
      }
      // (the next write of `red` follows at least one more ring barrier)
    }
  }
  // The last steps issued phantom loads into the rings; they must land before the work-group
  // ends and its LDS is handed to another.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

__global__ __launch_bounds__(256) void linear_reduce_kernel(LinearParams p) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.M * (p.N / 4);
  if (e >= total) return;
  reduce_partials4<false>(p, (int)(e / (p.N / 4)), (int)(e % (p.N / 4)) * 4);
}

template <int NB>
static hipError_t launch_tile(const LinearParams &p, hipStream_t stream, int cpz) {
  using T = LTile<NB>;
  dim3 grid((p.N + T::N - 1) / T::N, (p.M + kLM - 1) / kLM, p.ksplit);
  const hipError_t attr =
      allow_dynamic_lds(reinterpret_cast<const void *>(&linear_kernel<NB>), T::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(linear_kernel<NB>, grid, dim3(T::THREADS), T::LDS, stream, p, cpz);
  return hipGetLastError();
}

// Persistent fused lm-head: as many work-groups as compute units (or tile pairs, if fewer), spread
// over the 128-row blocks.
static hipError_t launch_lm_unmask(const LinearParams &p, hipStream_t stream) {
  using T = LPair;
  const hipError_t attr =
      allow_dynamic_lds(reinterpret_cast<const void *>(&lm_unmask_kernel), T::LDS);
  if (attr != hipSuccess) return attr;
  const int cus = current_device_cus();
  if (cus < 1) return hipErrorInvalidDevice;
  const int ntiles = (p.N + 255) / 256;
  const int rows = (p.M + kLM - 1) / kLM;
  const int G = std::max(1, std::min((ntiles + 1) / 2, cus / rows));
  hipLaunchKernelGGL(lm_unmask_kernel, dim3(G, rows), dim3(T::THREADS), T::LDS, stream, p, ntiles);
  return hipGetLastError();
}

// Whether every work-group of launch_tile<NB>'s grid for p can be resident on the current device at
// once (occupancy at the tile's LDS size times the compute units): the condition for merging the K
// partials inside the kernel.
template <int NB>
static bool tile_grid_resident(const LinearParams &p) {
  using T = LTile<NB>;
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int64_t cap[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (cap[dev] == 0) {
    int per_cu = 0;
    const int cus = current_device_cus();
    if (cus < 1 ||
        allow_dynamic_lds(reinterpret_cast<const void *>(&linear_kernel<NB>), T::LDS) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, linear_kernel<NB>, T::THREADS,
                                                     T::LDS) != hipSuccess)
      return false;
    const int64_t c = (int64_t)per_cu * cus;
    cap[dev] = c > 0 ? c : -1;  // -1: not even one (never merged inside)
  }
  const int64_t grid =
      (int64_t)((p.N + T::N - 1) / T::N) * ((p.M + kLM - 1) / kLM) * p.ksplit;
  return grid <= cap[dev];
}

hipError_t launch_linear(const LinearParams &p_in, hipStream_t stream) {
  if (p_in.epi == EPI_UNMASK && p_in.y == nullptr) return launch_lm_unmask(p_in, stream);
  LinearParams p = p_in;
  // merged inside the kernel: at most 16 partitions (the counter's mask), the grid resident at
  // once (else the partitions would mostly hand their shares over), the partials addressable by
  // 32-bit offsets
  if (p.ksplit == 1 || p.ksplit > 16 || (size_t)p.ksplit * p.M * p.N * 4 >= ((size_t)1 << 32) ||
      !(p.wide ? tile_grid_resident<8>(p) : tile_grid_resident<2>(p)))
    p.sync = nullptr;
  const int nch = (p.K + kLK - 1) / kLK;
  const int cpz = (nch + p.ksplit - 1) / p.ksplit;
  hipError_t e = p.wide ? launch_tile<8>(p, stream, cpz) : launch_tile<2>(p, stream, cpz);
  if (e != hipSuccess || p.ksplit == 1 || p.sync) return e;
  const size_t total = (size_t)p.M * (p.N / 4);
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

#ifdef TT_PHASE_STAMPS
// Profiling build only: copies (or, with clear != 0, zeroes) the projection kernel's phase stamps.
extern "C" int tt_phase_stamps_linear(void *dst, size_t bytes, int clear) {
  if (clear) {
    static unsigned long long zero[8192][8];
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(linear_phase_stamps), zero, sizeof(zero), 0,
                                  hipMemcpyHostToDevice);
  }
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(linear_phase_stamps), bytes, 0,
                                  hipMemcpyDeviceToHost);
}
#endif

}  // namespace tt
