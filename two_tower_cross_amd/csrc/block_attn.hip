// Block attention of the denoiser tower for gfx950.
//
// The S block queries of every (sequence b, KV head g) attend, under one softmax, to the context
// tower's same-layer KV rows 0..ctx_lens[b]-1 and to the block's own S KV rows ("Nemotron-
// TwoTower" explainer, sections "Architektur" and "Generierungsprozess"; gotburnout.io,
// "2. Denoiser Tower"). The G = Hq/Hkv query heads sharing KV head g are packed with the S block
// positions into G*S query rows, so one pass over the KV rows serves all of them.
//
// bf16 path (one work-group = 8 waves = up to 256 query rows of one (b, g), one context
// partition):
//   * 64-token K and V tiles are contiguous 16 KB blocks of 16-byte chunks in HBM, K as
//     [D/8 dimension chunks][64 tokens][8] and V as [8 token chunks][D][8], the order in which
//     the MFMA operands read them; they are copied into LDS unchanged with 16-byte loads, and the
//     operand reads of 32 lanes touch 32 consecutive chunks (no bank conflict).
//   * Each wave owns 32 query rows and computes S^T = K Q^T with 32x32x16 bf16 MFMA: a lane then
//     holds one query column and 16 token rows, so the softmax max/sum is in-lane plus one swap
//     between the two wave halves. The token order inside a 32-token sub-tile is permuted (bits 2
//     and 3 of the row swapped) so that the exponentials a lane holds are exactly the B operand of
//     the next product O^T += V^T P^T, with no LDS round trip for P.
//   * Online softmax in base 2 with the scale folded into one FMA; O^T is rescaled only when a
//     row maximum moved.
//   * Partition 0 also folds in the S block keys; with several partitions each one writes its
//     normalized output rows in fp16, each row scaled by a power of two 2^k that puts its largest
//     magnitude in [2^14, 2^15) (so no finite bf16 value overflows and small rows keep fp16's
//     relative precision), with (log-sum-exp, k) beside it; attn_reduce_kernel merges them
//     exactly.
// fp32 path: one work-group per (b, query head, block position), plain fp32 arithmetic.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "launch_util.hpp"

namespace tt {

#ifdef TT_PHASE_STAMPS
__device__ unsigned long long attn_phase_stamps[8192][8];
#endif

constexpr int kTile = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 4;             // LDS ring depth: up to 3 tiles in flight per work-group
constexpr float kRescaleLog2 = 8.0f;   // the running max moves only when it grows by > 2^8
constexpr float kLaneSumMax = 4096.f;  // pipelined loop: bound on a lane's 16 weights of a sub-tile
constexpr int kMaxPartTiles = 4096;    // tile indices of one partition staged in LDS (16 KB)

#define LDS_PTR(p) TT_LDS_PTR(p)

__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Keep the first n (0..8) bf16 elements of a 16-byte chunk, zero the rest.
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int n) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t m = (2 * w < n ? 0x0000FFFFu : 0u) | (2 * w + 1 < n ? 0xFFFF0000u : 0u);
    r[w] = v[w] & m;
  }
  return r;
}

// LDS map of the bf16 kernel: K stages, then V stages, each a 64-token tile in the cache's own
// 16-byte-chunk order (K [D/8][64 tokens][8], V [8 token chunks][D][8]), then the partition's
// tile indices. Every K offset, and every V offset relative to VBASE (which the lanes' V offsets
// include), stays within the 16-bit immediate of ds_read, so with the stage known at compile time
// each operand read is one VGPR plus an immediate.
template <int D>
struct Geom {
  static constexpr int KBYTES = kTile * D * 2;
  static constexpr int VBYTES = D * kTile * 2;
  static constexpr int VBASE = kStages * KBYTES;
  static constexpr int IDS = VBASE + kStages * VBYTES;
  static constexpr int FLAGS = IDS + kMaxPartTiles * 4;  // one word per wave
  static constexpr int LDS = FLAGS + kWaves * 4;
  static constexpr int KCH = KBYTES / 16 / kThreads;  // 16-byte K chunks per thread per tile
  static constexpr int VCH = VBYTES / 16 / kThreads;
  static constexpr int LOADS = KCH + VCH;             // DMA instructions per thread per tile
  static __device__ __forceinline__ constexpr int koff(int s) { return s * KBYTES; }
  static __device__ __forceinline__ constexpr int voff(int s) { return VBASE + s * VBYTES; }
};

// Per-lane constants of one wave. The tiles are chunk-major in HBM and in LDS, so an operand read
// of 32 lanes (32 tokens of one 8-dimension chunk for K, 32 dimensions of one 8-token chunk for V)
// covers 32 consecutive 16-byte slots (no bank conflict, no swizzle) and every address is one
// register plus an immediate: the K operand of K-step kk of the sub-tile in tokens 32h .. 32h + 31
// of a stage is at kb + kk * 2048 + h * 512; the V operand of (sub-tile sub, 16-token half kc) for
// dimensions 32mb .. 32mb + 31 at vb + (4 sub + 2 kc) * D * 16 + mb * 512. The DMA is a straight
// copy: a lane's j-th 16-byte chunk of a tile is byte (j * kThreads + wave * 64 + lane) * 16 of
// the source and of the stage.
template <int D>
struct LaneMap {
  int kb, vb;
  uint32_t kdma, vdma;
  int wave;

  __device__ __forceinline__ void init(int lane, int wave_) {
    wave = wave_;
    const int col = lane & 31, hh = lane >> 5;
    const int tok = swap_bits23(col);
    kb = hh * 1024 + tok * 16;                   // chunk 2kk + hh of token tok
    vb = Geom<D>::VBASE + hh * D * 16 + col * 16;  // token chunk 4sub + 2kc + hh of dimension col
    kdma = vdma = (uint32_t)(wave * 64 + lane) * 16u;
  }
  __device__ __forceinline__ int k(int kk) const { return kb + kk * 2048; }
  __device__ __forceinline__ int v(int sub, int kc) const { return vb + (sub * 4 + kc * 2) * D * 16; }
};

// Cache policy of the streaming loads: non-temporal (the KV caches are read once per step; the
// hint lets the memory system stream them, about 20% more read bandwidth than the default
// policy in a plain copy of this access pattern on gfx950).
constexpr int kNonTemporal = 2;

// Buffer resource over one 16 KB tile (raw, 32-bit data format; loads past the tile return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, bytes, 0x00020000);
}

// Full 64-token context tile -> LDS stage s, asynchronously (buffer_load ... lds, 16 B per lane).
// Each instruction fills 1024 contiguous LDS bytes lane by lane from the same 1024 bytes of the
// tile. The tile base goes into the (scalar) buffer resource, so a lane's source is a 32-bit
// offset.
template <int D>
__device__ __forceinline__ void dma_tile(char *smem, int s, const char *kb, const char *vb,
                                         const LaneMap<D> &lm) {
  const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kb, Geom<D>::KBYTES);
  const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vb, Geom<D>::VBYTES);
#pragma unroll
  for (int j = 0; j < Geom<D>::KCH; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        kr, LDS_PTR(smem + Geom<D>::koff(s) + (j * kWaves + lm.wave) * 1024), 16, lm.kdma,
        j * kThreads * 16, 0, kNonTemporal);
#pragma unroll
  for (int j = 0; j < Geom<D>::VCH; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        vr, LDS_PTR(smem + Geom<D>::voff(s) + (j * kWaves + lm.wave) * 1024), 16, lm.vdma,
        j * kThreads * 16, 0, kNonTemporal);
}

// Partial context tile (`valid` < 64 tokens) -> LDS stage s through registers, zero-filling the
// tokens past the end so that whatever the page holds there never reaches the MFMA. The tile is
// copied in its own chunk order (16-byte unit u: K token u % 64, V tokens 8 (u / D) ..); all of a
// thread's loads are issued before its first store, so the tile costs one memory round trip.
template <int D>
__device__ void load_tail_tile(char *smem, int s, const uint16_t *kbase, const uint16_t *vbase,
                               int valid, int tid) {
  constexpr int NU = kTile * D / 8 / kThreads;  // 16-byte units per thread (K and V alike)
  char *ks = smem + Geom<D>::koff(s);
  char *vs = smem + Geom<D>::voff(s);
  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4 xk[NU], xv[NU];
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int u = tid + j * kThreads;
    xk[j] = (u & 63) < valid ? ld_global_16(kbase + (size_t)u * 8) : z;
    xv[j] = (u / D) * 8 < valid ? ld_global_16(vbase + (size_t)u * 8) : z;
  }
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int u = tid + j * kThreads;
    const int n = valid - (u / D) * 8;
    st_lds_16(ks + u * 16, xk[j]);
    st_lds_16(vs + u * 16, keep_first(xv[j], n < 0 ? 0 : (n > 8 ? 8 : n)));
  }
}

// The block's own keys/values of (b, g), 64 at a time, through registers into LDS stage s; tokens
// past the count are zero. K rows are contiguous ([S][D]); a V row holds S tokens ([D][S]),
// 16-byte aligned when S % 8 == 0, else gathered element by element. The fetch is split from the
// store so that the first tile's loads can be in flight with the kernel's other first loads.
template <int D>
struct BlockRegs {
  static constexpr int NK = kTile * (D / 8) / kThreads, NV = D * 8 / kThreads;
  u32x4 xk[NK], xv[NV];
};

// Block keys/values rows 0 .. S-1 (S <= 64) into registers, zero past S.
template <int D>
__device__ __forceinline__ void fetch_block_tile(BlockRegs<D> &br, const uint16_t *kblk,
                                                 const uint16_t *vblk, int S, int vstride, int tid) {
  constexpr int KC = D / 8;
  constexpr int NK = BlockRegs<D>::NK, NV = BlockRegs<D>::NV;
  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4 *xk = br.xk, *xv = br.xv;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int f = tid + j * kThreads, r = f / KC, c = f % KC;
    xk[j] = r < S ? ld_global_16(kblk + (size_t)r * D + c * 8) : z;
  }
  if ((S & 7) == 0 && (vstride & 7) == 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int f = tid + j * kThreads, d = f / 8, c = f % 8;
      xv[j] = c * 8 < S ? ld_global_16(vblk + (size_t)d * vstride + c * 8) : z;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int f = tid + j * kThreads, d = f / 8, c = f % 8;
      uint16_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        e[i] = c * 8 + i < S ? vblk[(size_t)d * vstride + c * 8 + i] : (uint16_t)0;
#pragma unroll
      for (int w = 0; w < 4; ++w) xv[j][w] = (uint32_t)e[2 * w] | ((uint32_t)e[2 * w + 1] << 16);
    }
  }
}

// ... then into LDS stage s (in the chunk-major order of the ring's tiles).
template <int D>
__device__ __forceinline__ void store_block_tile(char *smem, int s, const BlockRegs<D> &br, int tid) {
  constexpr int KC = D / 8;
  constexpr int NK = BlockRegs<D>::NK, NV = BlockRegs<D>::NV;
  char *ks = smem + Geom<D>::koff(s);
  char *vs = smem + Geom<D>::voff(s);
  const u32x4 *xk = br.xk, *xv = br.xv;
#pragma unroll
  for (int j = 0; j < NK; ++j) {  // chunk c of row r -> K unit c * 64 + r
    const int f = tid + j * kThreads, r = f / KC, c = f % KC;
    st_lds_16(ks + (c * kTile + r) * 16, xk[j]);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {  // tokens 8c .. of dimension d -> V unit c * D + d
    const int f = tid + j * kThreads, d = f / 8, c = f % 8;
    st_lds_16(vs + (c * D + d) * 16, xv[j]);
  }
}

// Wait until at most `tiles_in_flight` tiles of DMA (LOADS instructions each) are outstanding.
template <int LOADS>
__device__ __forceinline__ void wait_dma(int tiles_in_flight) {
  if (tiles_in_flight >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LOADS));
  else if (tiles_in_flight == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// One 64-token LDS tile (at byte offsets kst / vst of K and V) into the running softmax state of
// this wave's 32 query rows. Two phases, each one basic block: (1) S^T of both 32-token
// sub-tiles (two independent MFMA chains) and their row maximum; (2) the exponentials of
// sub-tile 0, its PV product, then those of sub-tile 1 and its PV product, so the VALU work of one
// sub-tile can issue under the MFMAs of the other. m is a reference maximum in raw score units
// that only moves when some row's maximum exceeds it by more than 2^kRescaleLog2 in
// probability, so every exponential stays <= 2^8.
template <int D, bool FULL>
__device__ __forceinline__ void attend_tile(const char *smem, int kst, int vst, int valid,
                                            const LaneMap<D> &lm, const u32x4 *qreg,
                                            f32x16 *oacc, float &m, float &lpart, float c,
                                            int lane) {
  const int hh = lane >> 5;
  f32x16 s0 = {}, s1 = {};
  u32x4 a0[D / 16], a1[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    a0[kk] = ld_lds_16(smem + kst + lm.k(kk));
    a1[kk] = ld_lds_16(smem + kst + 32 * 16 + lm.k(kk));
  }
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    s0 = mfma32x32x16(a0[kk], qreg[kk], s0);
    s1 = mfma32x32x16(a1[kk], qreg[kk], s1);
  }
  // Operand reads run four K-steps ahead of the MFMAs that consume them.
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < D / 16 - 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  if (!FULL) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = (i >> 3) * 16 + hh * 8 + (i & 7);
      if (t >= valid) s0[i] = -INFINITY;
      if (t + 32 >= valid) s1[i] = -INFINITY;
    }
  }
  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
  mx = pair_max(mx);
  if (__ballot((mx - m) * c > kRescaleLog2)) {
    const float mnew = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
    lpart *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
    m = mnew;
  }
  const float mc = m * c;
  float psum = 0.f;
  u32x4 pa, pb;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s0[2 * w], c, -mc));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s0[2 * w + 1], c, -mc));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(s0[8 + 2 * w], c, -mc));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(s0[8 + 2 * w + 1], c, -mc));
    psum += (e0 + e1) + (e2 + e3);
    pa[w] = pack_bf16x2(e0, e1);
    pb[w] = pack_bf16x2(e2, e3);
  }
  u32x4 v0[D / 16], v1[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    v0[2 * mb] = ld_lds_16(smem + vst + mb * 32 * 16 + lm.v(0, 0));
    v0[2 * mb + 1] = ld_lds_16(smem + vst + mb * 32 * 16 + lm.v(0, 1));
  }
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    v1[2 * mb] = ld_lds_16(smem + vst + mb * 32 * 16 + lm.v(1, 0));
    v1[2 * mb + 1] = ld_lds_16(smem + vst + mb * 32 * 16 + lm.v(1, 1));
  }
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    oacc[mb] = mfma32x32x16(v0[2 * mb], pa, oacc[mb]);
    oacc[mb] = mfma32x32x16(v0[2 * mb + 1], pb, oacc[mb]);
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s1[2 * w], c, -mc));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s1[2 * w + 1], c, -mc));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(s1[8 + 2 * w], c, -mc));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(s1[8 + 2 * w + 1], c, -mc));
    psum += (e0 + e1) + (e2 + e3);
    pa[w] = pack_bf16x2(e0, e1);
    pb[w] = pack_bf16x2(e2, e3);
  }
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    oacc[mb] = mfma32x32x16(v1[2 * mb], pa, oacc[mb]);
    oacc[mb] = mfma32x32x16(v1[2 * mb + 1], pb, oacc[mb]);
  }
  lpart += psum;
  // The exponentials of sub-tile 1 issue between the PV MFMAs of sub-tile 0.
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
  }
}

// Software pipeline over the 32-token sub-tiles of the full context tiles. Window u consists of
// a matrix half M(u), which issues the PV product of sub-tile u-1 and the QK product of sub-tile
// u+1 and prefetches from LDS the operands of M(u+1) (V of sub-tile u, K of sub-tile u+2), and a
// vector half V(u), the softmax of sub-tile u, which depends on neither, so the two overlap (a
// window is one basic block apart from a rarely taken branch). Between halves the registers
// carry:
template <int D>
struct PipeRegs {
  f32x16 s;          // S^T of the sub-tile whose softmax is next (raw scores)
  f32x16 sn;         // S^T of the sub-tile after it
  u32x4 k[D / 16];   // K operand of the next QK
  u32x4 v[D / 16];   // V operand of the next PV, [32-dim block][16-token half]
  u32x4 pa, pb;      // P^T of the next PV (bf16), token halves 0 and 1
};

// M(u). KS/KH: stage and half of sub-tile u+2 (its K is loaded); VS/VH: of sub-tile u (its V is
// loaded). Adds the PV of sub-tile u-1 to O.
template <int D, int KS, int KH, int VS, int VH>
__device__ __forceinline__ void pipe_mma(const char *smem, const LaneMap<D> &lm, const u32x4 *qreg,
                                         PipeRegs<D> &r, f32x16 *oacc) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
      oacc[mb] = mfma32x32x16(r.v[2 * mb + kc], kc ? r.pb : r.pa, oacc[mb]);
  f32x16 sn = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) sn = mfma32x32x16(r.k[kk], qreg[kk], sn);
  r.sn = sn;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
      r.v[2 * mb + kc] = ld_lds_16(smem + (Geom<D>::voff(VS) - Geom<D>::VBASE) +
                                   mb * 32 * 16 + lm.v(VH, kc));
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    r.k[kk] = ld_lds_16(smem + Geom<D>::koff(KS) + KH * 32 * 16 + lm.k(kk));
  // Each operand read follows the MFMA that last used its registers.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Exponentials of the 16 scores a lane holds against the reference mc = m * c (base 2), packed to
// bf16 as the B operand of the PV product, and their sum (of the rounded values, so that the
// normalizer sums exactly the weights the product applies; one dot product with ones per pair).
__device__ __forceinline__ float exp_pack(const f32x16 &s, float c, float mc, u32x4 &pa,
                                          u32x4 &pb) {
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16x2 (1, 1)
  float ps0 = 0.f, ps1 = 0.f;
  // (The sums are taken on the packed words before they are inserted into the operand vectors:
  // applied to an element of the vector, the dot product was compiled to read element 0 only.)
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[2 * w], c, -mc)),
                                   __builtin_amdgcn_exp2f(fmaf(s[2 * w + 1], c, -mc)));
    const uint32_t b = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[8 + 2 * w], c, -mc)),
                                   __builtin_amdgcn_exp2f(fmaf(s[8 + 2 * w + 1], c, -mc)));
    ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                          __builtin_bit_cast(bf16x2, kOnes), ps0, false);
    ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, b),
                                          __builtin_bit_cast(bf16x2, kOnes), ps1, false);
    pa[w] = a;
    pb[w] = b;
  }
  return ps0 + ps1;
}

// V(u): softmax of sub-tile u against the reference maximum m. The exponentials are first taken
// against the current m; only when some lane's 16 of them sum to more than kLaneSumMax (or to inf /
// NaN, as for the first sub-tile, when m = -inf) does the wave take the rare branch that moves m to
// the row maximum (never down), rescales l and O (which, after M(u), holds everything through
// sub-tile u-1) and recomputes them, so every weight stays <= kLaneSumMax.
template <int D>
__device__ __forceinline__ void pipe_softmax(PipeRegs<D> &r, f32x16 *oacc, float &m, float &lpart,
                                             float c) {
  float ps = exp_pack(r.s, c, m * c, r.pa, r.pb);
  if (__ballot(!(ps <= kLaneSumMax))) {
    float t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t[j] = fmaxf(fmaxf(r.s[4 * j], r.s[4 * j + 1]), fmaxf(r.s[4 * j + 2], r.s[4 * j + 3]));
    const float mx = pair_max(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
    const float mnew = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);  // 0 while m = -inf
    m = mnew;
    lpart *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
    ps = exp_pack(r.s, c, mnew * c, r.pa, r.pb);
  }
  lpart += ps;
  r.s = r.sn;
}

// Pipeline start: sub-tile 0 (stage 0, half 0) is in LDS. Computes S^T of sub-tile 0, loads the K
// of sub-tile 1 and clears the PV operands so that window 0 adds nothing for sub-tile -1.
template <int D>
__device__ __forceinline__ void pipe_start(const char *smem, const LaneMap<D> &lm,
                                           const u32x4 *qreg, PipeRegs<D> &r) {
  u32x4 k0[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) k0[kk] = ld_lds_16(smem + Geom<D>::koff(0) + lm.k(kk));
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    r.k[kk] = ld_lds_16(smem + Geom<D>::koff(0) + 32 * 16 + lm.k(kk));
  r.s = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) r.s = mfma32x32x16(k0[kk], qreg[kk], r.s);
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < D / 16; ++j) r.v[j] = z;
  r.pa = z;
  r.pb = z;
}

// Pipeline end: the PV product of the last sub-tile.
template <int D>
__device__ __forceinline__ void pipe_finish(const PipeRegs<D> &r, f32x16 *oacc) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
      oacc[mb] = mfma32x32x16(r.v[2 * mb + kc], kc ? r.pb : r.pa, oacc[mb]);
}

// ------------------------------------------------------------------ balanced partition plan
// With the automatic partition count the context of each (sequence, KV head) is cut so that the
// work-groups get nearly equal shares whatever the mix of lengths: sequence b's T_b =
// ceil(L_b / 64) tiles go into n_b = max(1, ceil(T_b / c)) partitions of nearly equal size
// (partition s holds tiles floor(s T_b / n_b) .. floor((s + 1) T_b / n_b) - 1; partition 0 also
// takes the block keys), with c the smallest tile count >= kMinPartTiles for which
// sum_b n_b <= p.parts (the host's target per KV head and row group: one work-group per compute
// unit); when one partition per sequence already exceeds the target, c = kMaxPartTiles. A
// sequence that the caller marks finished (p.active given and no nonzero flag of the sequence)
// gets no partition; one with an invalid length counts as empty (its outputs become NaN). Work
// item k of a KV head and row group is partition k - E_b of the sequence b with E_b <= k <
// E_b + n_b (E_b = sum of n over the sequences before b), ordered (b, KV head, partition) so that
// equal lengths give the same items, in the same order, as a uniform split. Every wave of the
// attention kernel computes the plan from the lengths (at most kPlanMaxB sequences, kPlanPerLane
// per lane), except when every sequence is active at max_ctx_len: then the plan is that uniform
// split, known beforehand, and one ballot replaces the computation. Work-group 0 writes the plan
// record that the merge reads.
constexpr int kPlanMaxB = 256;
constexpr int kPlanPerLane = kPlanMaxB / 64;
constexpr int kMinPartTiles = 1;  // short contexts: one tile per work-group, more of the GPU busy

// Inclusive prefix sum over the 64 lanes of a wave: sums of 4 within each row of 16 lanes by row
// shifts, then rows completed with shifts by 4 and 8, then carried across rows by the row
// broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_incl_scan(int x) {
  int v = x + __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);         // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xf, 0xf, true);         // row_shr:3
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, true);         // row_shr:4, lanes 4-15
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, true);         // row_shr:8, lanes 8-15
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, true);         // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, true);         // row_bcast:31, rows 2, 3
  return v;
}

__device__ __forceinline__ int wave_total(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

// ceil(a / c) for 0 <= a < 2^24, 1 <= c < 2^24: a float estimate, then corrected exactly.
__device__ __forceinline__ int ceil_div24(int a, int c) {
  int q = (int)ceilf((float)a / (float)c);
  while (q > 0 && (q - 1) * c >= a) --q;
  while (q * c < a) ++q;
  return q;
}

// Lane l's sequences b = l + 64 j: their tile counts, activity, and (after plan_partitions)
// partition counts and exclusive prefix sums.
struct PlanLanes {
  int T[kPlanPerLane];
  int n[kPlanPerLane];
  int excl[kPlanPerLane];
  bool act[kPlanPerLane];
};

// A sequence counts as active unless the caller's flags say it has no masked position left.
// Whether sequence b has a nonzero flag. The flags are read in batches of 8 words (or bytes) whose
// loads are all issued before any is used (indices clamped to the row, so a batch past its end
// re-reads the row's last word): one memory round trip per batch, 1 for S <= 32.
__device__ __forceinline__ bool seq_active(const AttnParams &p, int b) {
  if (!p.active) return true;
  const uint8_t *m = p.active + (size_t)b * p.S;
  uint32_t any = 0;
  if ((p.S & 3) == 0 && (reinterpret_cast<uintptr_t>(p.active) & 3) == 0) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(m);
    const int nw = p.S >> 2;
    for (int i0 = 0; i0 < nw; i0 += 8) {
      uint32_t v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = w[min(i0 + k, nw - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) any |= v[k];
    }
  } else {
    for (int i0 = 0; i0 < p.S; i0 += 8) {
      uint32_t v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = m[min(i0 + k, p.S - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) any |= v[k];
    }
  }
  return any != 0;
}

// Requests the lengths (and activity flags) of lane's sequences; nothing is used yet.
__device__ __forceinline__ void plan_load(const AttnParams &p, int lane, int (&L)[kPlanPerLane],
                                          bool (&act)[kPlanPerLane]) {
#pragma unroll
  for (int j = 0; j < kPlanPerLane; ++j) {
    const int b = lane + 64 * j;
    L[j] = b < p.B ? p.ctx_lens[b] : 0;
    act[j] = b < p.B && seq_active(p, b);
  }
}

__device__ __forceinline__ int plan_count(const PlanLanes &pl, int c) {
  int s = 0;
#pragma unroll
  for (int j = 0; j < kPlanPerLane; ++j)
    if (pl.act[j]) s += max(1, ceil_div24(pl.T[j], c));
  return wave_total(s);
}

// The partition size c (tiles) and every lane's n and exclusive prefix; returns the total count.
__device__ int plan_partitions(const AttnParams &p, const int (&L)[kPlanPerLane],
                               const bool (&act)[kPlanPerLane], PlanLanes &pl) {
  int tot = 0, nact = 0;
#pragma unroll
  for (int j = 0; j < kPlanPerLane; ++j) {
    const bool ok = L[j] >= 0 && L[j] <= p.max_ctx_len;
    pl.T[j] = ok ? (L[j] + kTile - 1) / kTile : 0;
    pl.act[j] = act[j];
    if (act[j]) {
      tot += pl.T[j];
      ++nact;
    }
  }
  tot = wave_total(tot);
  nact = wave_total(nact);
  int lo = min(max(kMinPartTiles, (tot + p.parts - 1) / p.parts), kMaxPartTiles);
  int c = lo;
  if (plan_count(pl, lo) > p.parts) {
    if (nact >= p.parts) {
      c = kMaxPartTiles;
    } else {
      // feasible: sum_b n_b <= tot / hi + nact <= parts (or hi is the largest partition allowed)
      int hi = min(kMaxPartTiles, max(lo + 1, (tot + p.parts - nact - 1) / (p.parts - nact)));
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (plan_count(pl, mid) <= p.parts) hi = mid;
        else lo = mid;
      }
      c = hi;
    }
  }
  int carry = 0;
#pragma unroll
  for (int j = 0; j < kPlanPerLane; ++j) {
    pl.n[j] = pl.act[j] ? max(1, ceil_div24(pl.T[j], c)) : 0;
    const int incl = wave_incl_scan(pl.n[j]) + carry;
    pl.excl[j] = incl - pl.n[j];
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  return carry;
}

// The sequence, KV head and partition of work unit q (units ordered (b, KV head, partition)), or
// b = -1 when q lies past the last one.
struct PlanItem {
  int b, g, split, n, excl;
};

__device__ __forceinline__ PlanItem plan_item(const AttnParams &p, const PlanLanes &pl, int q) {
  PlanItem it = {-1, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kPlanPerLane; ++j) {
    const bool mine = q >= pl.excl[j] * p.Hkv && q < (pl.excl[j] + pl.n[j]) * p.Hkv;
    const uint64_t hit = __ballot(mine);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      it.b = l + 64 * j;
      it.n = __builtin_amdgcn_readlane(pl.n[j], l);
      it.excl = __builtin_amdgcn_readlane(pl.excl[j], l);
      const int r = q - it.excl * p.Hkv;
      it.g = r / it.n;
      it.split = r - it.g * it.n;
    }
  }
  return it;
}

// Tokens [t_begin, t_end) of partition s of n over a sequence of L tokens (T tiles).
__device__ __forceinline__ void part_range(int s, int n, int L, int &t_begin, int &t_end) {
  const int T = (L + kTile - 1) / kTile;
  t_begin = (int)(((int64_t)s * T) / n) * kTile;
  t_end = min(L, (int)(((int64_t)(s + 1) * T) / n) * kTile);
}

template <int D>
__global__ __launch_bounds__(kThreads) void block_attn_bf16_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // Work-groups are dealt to the 8 XCDs round robin (work-group id mod 8). The row groups of one
  // (sequence, KV head, partition) read the same KV, so they get ids 8 apart: one XCD, adjacent
  // in its dispatch order, one L2 serving them all.
  const int id = blockIdx.x, R = p.row_groups;
  const int q = (id >> 3) / R * 8 + (id & 7);  // (sequence, KV head, partition) unit
  const int rg = (id >> 3) % R;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  TT_STAMPS_DECL;
  TT_STAMP(0);  // phase stamps (profiling build): start
  const int per_b = p.Hkv * p.splits;
  if (!p.balanced && q >= p.B * per_b) return;

  // The unit's sequence, KV head and partition, first as if every sequence had max_ctx_len tokens
  // (and were active): the uniform split, and with the balanced plan the plan of that case, which
  // is the actual one whenever the lengths are equal. Everything that depends on them is requested
  // at once with the lengths (one memory round trip): this wave's query rows, the first block
  // tile (partition 0) and the page of every tile the partition can hold (clamped to the table;
  // entries past the sequence's end are loaded but not used). With the balanced plan the actual
  // unit follows from the lengths, and what differs is requested again.
  int b = min(q / per_b, p.B - 1);
  int g = (q % per_b) / p.splits, split = q % p.splits;
  int t_begin, t_end_b;
  if (p.balanced) part_range(split, p.splits, p.max_ctx_len, t_begin, t_end_b);
  else t_begin = split * p.chunk;
  int n_b = p.splits, excl_b = b * p.splits;  // the sequence's partitions, and those before it
  int Lp[kPlanPerLane];
  bool actp[kPlanPerLane];
  int L = 0;

  const int col = lane & 31, hh = lane >> 5;
  const int r_local = wave * 32 + col;
  const int r = rg * p.rows_per_group + r_local;
  const bool row_ok = r < p.rows && r_local < p.rows_per_group;
  const bool wave_active =
      wave * 32 < p.rows_per_group && rg * p.rows_per_group + wave * 32 < p.rows;
  const int jq = row_ok ? r / p.S : 0, iq = row_ok ? r % p.S : 0;
  u32x4 qreg[D / 16];
  BlockRegs<D> br;
  const int n_spec = p.chunk / kTile;               // tiles of the largest partition
  // Up to 64 tiles, every wave requests all of the pages (lane i: tile i) and keeps the tile
  // indices in a register; beyond, the work-group requests them once and stages them in LDS.
  const bool ids_in_regs = n_spec <= 64;
  const int li = ids_in_regs ? lane : tid;
  int spec_page = 0;
  auto load_unit = [&]() {
    const uint16_t *qrow =
        static_cast<const uint16_t *>(p.q) + (((size_t)b * p.S + iq) * p.Hq + g * p.G + jq) * D;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qreg[kk] = row_ok ? ld_global_16(qrow + kk * 16 + hh * 8) : z;
    const size_t bg = (size_t)b * p.Hkv + g;
    if (split == 0)
      fetch_block_tile<D>(br, static_cast<const uint16_t *>(p.k_blk) + bg * p.S * D,
                          static_cast<const uint16_t *>(p.v_blk) + bg * D * p.S, min(p.S, kTile),
                          p.S, tid);
    const int32_t *btab = p.block_table + (size_t)b * p.max_pages;
    if (li < n_spec) spec_page = btab[min((t_begin + li * kTile) / p.page_size, p.max_pages - 1)];
  };
  // The unit's loads go first: the plan's lengths and flags are used (waited for) at once.
  load_unit();
  if (p.balanced) plan_load(p, lane, Lp, actp);
  else L = p.ctx_lens[b];

  bool spec_exact = false;
  if (p.balanced) {
    // Every sequence active at max_ctx_len: the plan is the speculated one (the uniform split).
    bool full = true;
#pragma unroll
    for (int j = 0; j < kPlanPerLane; ++j)
      if (lane + 64 * j < p.B) full = full && actp[j] && Lp[j] == p.max_ctx_len;
    spec_exact = __ballot(!full) == 0;
  }
  if (spec_exact) {
    if (id == 0 && wave == 0 && p.plan_rec) {
#pragma unroll
      for (int j = 0; j < kPlanPerLane; ++j) {
        const int bb = lane + 64 * j;
        if (bb < p.B) *reinterpret_cast<int2 *>(p.plan_rec + 2 * bb) = make_int2(p.splits, bb * p.splits);
      }
    }
    if (q >= p.B * per_b) return;  // past the last unit (the same for every wave)
    L = p.max_ctx_len;
  } else if (p.balanced) {
    PlanLanes pl;
    plan_partitions(p, Lp, actp, pl);
    if (id == 0 && wave == 0 && p.plan_rec) {  // the merge reads the plan instead of recomputing it
#pragma unroll
      for (int j = 0; j < kPlanPerLane; ++j) {
        const int bb = lane + 64 * j;
        if (bb < p.B) *reinterpret_cast<int2 *>(p.plan_rec + 2 * bb) = make_int2(pl.n[j], pl.excl[j]);
      }
    }
    const PlanItem it = plan_item(p, pl, q);
    if (it.b < 0) return;                        // past the last unit (the same for every wave)
#pragma unroll
    for (int j = 0; j < kPlanPerLane; ++j)
      if (it.b >= 64 * j && it.b < 64 * (j + 1)) L = __builtin_amdgcn_readlane(Lp[j], it.b - 64 * j);
    const bool ok = L >= 0 && L <= p.max_ctx_len;
    int tb, te;
    part_range(it.split, it.n, ok ? L : 0, tb, te);
    n_b = it.n;
    excl_b = it.excl;
    if (it.b != b || it.g != g || it.split != split || tb != t_begin) {
      b = it.b;
      g = it.g;
      split = it.split;
      t_begin = tb;
      load_unit();
    }
    t_end_b = te;
  }
  const int h = g * p.G + jq;
  const bool has_block = split == 0;
  const size_t bg = (size_t)b * p.Hkv + g;
  const uint16_t *kblk = static_cast<const uint16_t *>(p.k_blk) + bg * p.S * D;
  const uint16_t *vblk = static_cast<const uint16_t *>(p.v_blk) + bg * D * p.S;
  const int32_t *btab = p.block_table + (size_t)b * p.max_pages;

  bool bad = L < 0 || L > p.max_ctx_len;
  const int Lc = bad ? 0 : L;
  const int t_end = p.balanced ? t_end_b : min(Lc, t_begin + p.chunk);
  if (!p.balanced && !has_block && t_begin >= Lc && !bad) return;  // partition past the context

  const int n_ctx = t_end > t_begin ? t_end - t_begin : 0;
  const int n_full = n_ctx / kTile;            // full tiles: asynchronous ring
  const int tail = n_ctx - n_full * kTile;     // tokens of the last, partial tile

  // K and V pools are both sequences of 16 KB tiles (chunk-major 64-token tiles); context tile n of
  // this partition (tokens t_begin + 64n ...) is tile (page * Hkv + g) * (page_size / 64) + (offset
  // in page) / 64 of either pool. The partition's tile indices are computed once (in a register of
  // every wave up to 64 tiles, else in LDS), so the ring issues no vector load of its own besides
  // the DMA. A page id outside the pool makes the sequence bad: nothing is loaded through it and
  // its outputs become NaN.
  int *tile_ids = reinterpret_cast<int *>(smem + Geom<D>::IDS);
  const int n_tiles = (n_ctx + kTile - 1) / kTile;
  const int tpp = p.page_size / kTile;
  int my_tile = 0;  // register path: the index of tile `lane`
  if (ids_in_regs) {
    // Every wave sees every page, so each reaches the same verdict without a barrier.
    int page_bad = 0;
    if (lane < n_tiles) {
      page_bad = spec_page < 0 || spec_page >= p.num_pages;
      my_tile = (spec_page * p.Hkv + g) * tpp + ((t_begin + lane * kTile) % p.page_size) / kTile;
    }
    if (__ballot(page_bad) != 0) bad = true;
  } else {
    int page_bad = 0;
    for (int i = tid; i < n_tiles; i += kThreads) {
      const int t = t_begin + i * kTile;
      const int page = i < kThreads ? spec_page : btab[t / p.page_size];
      page_bad |= page < 0 || page >= p.num_pages;
      tile_ids[i] = (page * p.Hkv + g) * tpp + (t % p.page_size) / kTile;
    }
    int *flags = reinterpret_cast<int *>(smem + Geom<D>::FLAGS);
    const bool wave_bad = __ballot(page_bad) != 0;
    if (lane == 0) flags[wave] = wave_bad;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any |= flags[w];
    if (any) bad = true;
  }
  // Index of context tile n (n uniform); on the LDS path it is read after a barrier, when this
  // wave has no LDS read in flight.
  auto tile_index = [&](int n) {
    return ids_in_regs ? __builtin_amdgcn_readlane(my_tile, n)
                       : __builtin_amdgcn_readfirstlane(tile_ids[n]);
  };
  TT_STAMP(1);  // the partition's tile indices are known
  const int n_full_ok = bad ? 0 : n_full;
  const int tail_ok = bad ? 0 : tail;
  const char *kpool = static_cast<const char *>(p.k_pages);
  const char *vpool = static_cast<const char *>(p.v_pages);
  constexpr size_t kTileBytes = (size_t)kTile * D * 2;

  LaneMap<D> lm;
  lm.init(lane, wave);
  // DMA of context tile n into stage n % kStages.
  auto dma_ctx_tile = [&](int n, int stage) {
    const size_t off = (size_t)tile_index(n) * kTileBytes;
    dma_tile<D>(smem, stage, kpool + off, vpool + off, lm);
  };

  // Start the ring: context tiles 0 .. kStages-2 into stages 0 .. kStages-2, then the first block
  // tile (already in registers) into the last stage; the block tile is attended while the ring's
  // first tiles are in flight.
#pragma unroll
  for (int n = 0; n < kStages - 1; ++n)
    if (n < n_full_ok) dma_ctx_tile(n, n);
  if (has_block) store_block_tile<D>(smem, kStages - 1, br, tid);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16{};
  float m = -INFINITY, lpart = 0.f;
  const float c = p.scale * kLog2e;

  if (has_block) {
    for (int j0 = 0; j0 < p.S; j0 += kTile) {
      const int nj = min(kTile, p.S - j0);
      if (j0 > 0) {
        fetch_block_tile<D>(br, kblk + (size_t)j0 * D, vblk + j0, nj, p.S, tid);
        lds_barrier();  // every wave is done with the previous block tile
        store_block_tile<D>(smem, kStages - 1, br, tid);
      }
      lds_barrier();
      if (wave_active)
        attend_tile<D, false>(smem, Geom<D>::koff(kStages - 1), Geom<D>::voff(kStages - 1) -
                              Geom<D>::VBASE, nj, lm, qreg, oacc, m, lpart, c, lane);
    }
  }

  TT_STAMP(2);  // the ring's first DMA is issued (and the block tile attended)
  if (n_full_ok > 0) {
    // Tile 0 is in LDS for every wave.
    wait_dma<Geom<D>::LOADS>(min(kStages - 2, n_full_ok - 1));
    lds_barrier();
    TT_STAMP(3);  // tile 0 has landed
    TT_CYCLES(6);
    PipeRegs<D> pr;
    if (wave_active) pipe_start<D>(smem, lm, qreg, pr);
    // Tile T is consumed by M(2T) and M(2T+1) (its V) after M(2T-2) and M(2T-1) read its K.
    // Before M(2T): wait for tile T+1, then refill the stage of tile T-1, which every wave is done
    // with. The ring is unrolled by its depth so that all LDS offsets are immediates.
    auto ring_step = [&](auto stage_tag, int T) {
      constexpr int ST = decltype(stage_tag)::value;
      constexpr int NX = (ST + 1) % kStages;
      if (T + 1 < n_full_ok) {
        wait_dma<Geom<D>::LOADS>(min(1, n_full_ok - 2 - T));
        lds_barrier();
        if (T + kStages - 1 < n_full_ok) dma_ctx_tile(T + kStages - 1, (ST + kStages - 1) % kStages);
      }
      if (wave_active) {
        pipe_mma<D, NX, 0, ST, 0>(smem, lm, qreg, pr, oacc);
        pipe_softmax<D>(pr, oacc, m, lpart, c);
        pipe_mma<D, NX, 1, ST, 1>(smem, lm, qreg, pr, oacc);
        pipe_softmax<D>(pr, oacc, m, lpart, c);
      }
    };
    for (int T = 0; T < n_full_ok; T += kStages) {
      ring_step(std::integral_constant<int, 0>{}, T);
      if (T + 1 < n_full_ok) ring_step(std::integral_constant<int, 1>{}, T + 1);
      if (T + 2 < n_full_ok) ring_step(std::integral_constant<int, 2>{}, T + 2);
      if (T + 3 < n_full_ok) ring_step(std::integral_constant<int, 3>{}, T + 3);
    }
    if (wave_active) pipe_finish<D>(pr, oacc);
    TT_STAMP(4);  // the ring is done
    TT_CYCLES(7);
  }

  if (tail_ok > 0) {
    lds_barrier();  // every wave is done with the ring before a stage is overwritten
    const int st = n_full_ok % kStages;
    const size_t off = (size_t)tile_index(n_full_ok) * kTileBytes;
    load_tail_tile<D>(smem, st, reinterpret_cast<const uint16_t *>(kpool + off),
                      reinterpret_cast<const uint16_t *>(vpool + off), tail_ok, tid);
    lds_barrier();
    if (wave_active)
      attend_tile<D, false>(smem, Geom<D>::koff(st), Geom<D>::voff(st) - Geom<D>::VBASE, tail_ok,
                            lm, qreg, oacc, m, lpart, c, lane);
  }

  // Epilogue. Each wave stages its normalized 32 x D output block in a private LDS slice (the
  // ring is idle once every wave has passed this barrier) and writes it back row by row, so
  // every store instruction covers whole contiguous rows. In the slice the 16-byte chunks of row
  // r are XOR-swizzled by r, so that the 32 rows one LDS store touches fall in distinct banks.
  lds_barrier();
  if (!wave_active) return;
  const float l = pair_sum(lpart);
  const float inv = bad ? NAN : 1.0f / l;
  const float lse_val = bad ? NAN : m * p.scale + logf(l);
  const bool to_part = n_b > 1;
  // Partial rows go out in fp16 scaled by 2^kexp, kexp chosen so that the row's largest |O_p|
  // lands in [2^14, 2^15): |O_p| <= max|V| may be any finite bf16 value, far outside fp16's range
  // without the scale. The row's 2 x D/2 values sit in the lane pair (col, col + 32).
  int kexp = 0;
  float fac = inv;
  if (to_part) {
    float amax = 0.f;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(oacc[mb][i]));
    amax = pair_max(amax) * inv;
    if (amax > 0.f) kexp = 15 - __builtin_amdgcn_frexp_expf(amax);  // amax in [2^(e-1), 2^e)
    kexp = min(max(kexp, -126), 126);  // inv <= 1, so inv * 2^kexp stays finite
    fac = __builtin_amdgcn_ldexpf(inv, kexp);
  }
  const bool half_out = to_part || p.out_bf16;     // 2-byte elements (fp16 partial / bf16 out)
  const int row_bytes = D * (half_out ? 2 : 4);
  const int cpr = row_bytes / 16;                 // 16-byte chunks per row (a power of two)
  char *slice = smem + wave * (32 * D * 4);
  char *rowp = slice + col * row_bytes;
  if (half_out) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + q4 * 8 + hh * 4;
        const float o0 = oacc[mb][q4 * 4 + 0] * fac, o1 = oacc[mb][q4 * 4 + 1] * fac;
        const float o2 = oacc[mb][q4 * 4 + 2] * fac, o3 = oacc[mb][q4 * 4 + 3] * fac;
        uint2 pk;
        if (to_part) {
          pk.x = pack_f16x2(o0, o1);
          pk.y = pack_f16x2(o2, o3);
        } else {
          pk.x = pack_bf16x2(o0, o1);
          pk.y = pack_bf16x2(o2, o3);
        }
        const int byte = d * 2;
        *reinterpret_cast<uint2 *>(rowp + (((byte >> 4) ^ (col & (cpr - 1))) << 4) + (byte & 15)) = pk;
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + q4 * 8 + hh * 4;
        f32x4 o;
        o[0] = oacc[mb][q4 * 4 + 0] * inv;
        o[1] = oacc[mb][q4 * 4 + 1] * inv;
        o[2] = oacc[mb][q4 * 4 + 2] * inv;
        o[3] = oacc[mb][q4 * 4 + 3] * inv;
        *reinterpret_cast<f32x4 *>(rowp + ((((d * 4) >> 4) ^ (col & (cpr - 1))) << 4)) = o;
      }
  }
  // chunk cc of slice row rr (the un-swizzled source of a contiguous row store)
  auto slice_chunk = [&](int rr, int cc) {
    return ld_lds_16(slice + rr * row_bytes + ((cc ^ (rr & (cpr - 1))) << 4));
  };
  if (to_part) {
    // partial slot: the sequence's partitions sit together, per (KV head, row group)
    const size_t item = (size_t)excl_b * p.Hkv * R + (size_t)(g * R + rg) * n_b + split;
    const size_t slots = p.balanced ? (size_t)p.items * p.Hkv * R : (size_t)p.B * p.Hkv * R * p.splits;
    if (item >= slots) return;  // never taken: the plan keeps every slot inside the workspace
    // rows wave*32 .. wave*32+31 of this partition are contiguous in the partial buffer
    char *dst = reinterpret_cast<char *>(p.part_o) + (item * p.rows_per_group + wave * 32) * (size_t)row_bytes;
    const int nrows = min(32, p.rows_per_group - wave * 32);
    for (int f = lane; f < nrows * cpr; f += 64)
      *reinterpret_cast<u32x4 *>(dst + (size_t)f * 16) = slice_chunk(f / cpr, f % cpr);
    if (hh == 0 && r_local < p.rows_per_group)
      reinterpret_cast<float2 *>(p.part_lse)[item * p.rows_per_group + r_local] =
          make_float2(lse_val, (float)kexp);
  } else {
    char *obase = static_cast<char *>(p.out);
    for (int f = lane; f < 32 * cpr; f += 64) {
      const int rr = f / cpr, cc = f % cpr;
      const int rg_row = rg * p.rows_per_group + wave * 32 + rr;
      if (wave * 32 + rr >= p.rows_per_group || rg_row >= p.rows) continue;
      const int j2 = rg_row / p.S, i2 = rg_row % p.S;
      const size_t orow = ((size_t)b * p.S + i2) * p.Hq + (g * p.G + j2);
      *reinterpret_cast<u32x4 *>(obase + orow * row_bytes + cc * 16) = slice_chunk(rr, cc);
    }
    if (p.lse && hh == 0 && row_ok) p.lse[((size_t)b * p.Hq + h) * p.S + iq] = lse_val;
  }
  TT_STAMP_DRAINED(5);  // outputs written
  TT_STAMPS_STORE(attn_phase_stamps, blockIdx.x);
}

// Exact merge of the partitions of each query row: with lse* = max_p lse_p and
// w_p = exp(lse_p - lse*), out = sum_p w_p O_p / sum_p w_p and lse = lse* + ln(sum_p w_p).
// A partition's row is stored as fp16 O_p * 2^k_p with (lse_p, k_p) beside it, so its term is
// (w_p * 2^-k_p) times the stored value (the power of two is exact).
//
// A work-group of 256 threads covers RPB query rows of one (b, KV head, row group); a row's D
// outputs are spread over TPR = D/8 threads (8 dimensions each) and its partitions over PG thread
// groups (group pg takes partitions pg, pg + PG, ...), so that the grid grows with the partition
// count and not only with the rows (a single 131072-token sequence has only 2 x 256 rows). Each
// thread requests the LSE pair and the 16-byte chunk of its first kRedBatch partitions together
// with the lengths before using any of them (one memory round trip); partitions past the
// sequence's last one are loaded (the workspace holds them) but not used. The PG groups'
// (max, sum, 8 accumulators) are combined through LDS in a fixed order.
constexpr int kRedBatch = 16;

template <int D, int PG>
__global__ __launch_bounds__(256) void attn_reduce_kernel(AttnParams p) {
  constexpr int TPR = D / 8;                 // threads per row and partition group
  constexpr int RPB = 256 / (TPR * PG);      // rows per work-group
  __shared__ float red[PG > 1 ? 256 * 10 : 1];
  const int item_bgr = blockIdx.x;
  const int rg = item_bgr % p.row_groups;
  const int g = (item_bgr / p.row_groups) % p.Hkv;
  const int b = item_bgr / (p.row_groups * p.Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const uint16_t *part = static_cast<const uint16_t *>(p.part_o);
  const int d8 = tid % TPR, pg = (tid / TPR) % PG, rr = tid / (TPR * PG);
  const int r_local = blockIdx.y * RPB + rr;
  const bool live = r_local < p.rows_per_group && rg * p.rows_per_group + r_local < p.rows;
  const int r_ld = live ? r_local : 0;       // rows past the end load row 0 (never stored)

  // This (sequence, KV head, row group)'s partials: slots item0 .. item0 + n - 1, first as in the
  // case that every sequence has max_ctx_len tokens (the uniform split); with the balanced plan
  // the actual slots follow from the sequence's plan record (written by the attention kernel,
  // requested in the same round trip), and the first batch is requested again if they differ.
  size_t item0 = (size_t)item_bgr * p.splits;
  int n = p.splits;
  int2 rec = make_int2(0, 0);
  if (p.balanced) rec = *reinterpret_cast<const int2 *>(p.plan_rec + 2 * b);
  float2 ls[kRedBatch];
  u32x4 v[kRedBatch];
  auto batch_loads = [&](int s0) {
    // partitions per thread in this batch (the same for the whole work-group); a group whose
    // last one lies past the end loads the sequence's last partition instead (never used)
    const int nb = min(kRedBatch, (n - s0 + PG - 1) / PG);
#pragma unroll
    for (int sp = 0; sp < kRedBatch; ++sp) {
      if (sp < nb) {
        const int sidx = min(s0 + pg + sp * PG, n - 1);
        const size_t it = (item0 + sidx) * p.rows_per_group + r_ld;
        ls[sp] = reinterpret_cast<const float2 *>(p.part_lse)[it];
        v[sp] = ld_global_16(part + it * D + d8 * 8);
      }
    }
  };
  batch_loads(0);
  asm volatile("" ::: "memory");  // keeps the length loads behind the batch's loads
  const int L = p.ctx_lens[b];
  const bool bad = L < 0 || L > p.max_ctx_len;
  int nact;                       // partitions of this sequence that hold context
  if (p.balanced) {
    const int nb = __builtin_amdgcn_readfirstlane(rec.x), ex = __builtin_amdgcn_readfirstlane(rec.y);
    // one partition: the attention kernel wrote the output itself; none: a finished sequence
    if (nb <= 1) return;
    const size_t real0 = (size_t)ex * p.Hkv * p.row_groups + (size_t)(g * p.row_groups + rg) * nb;
    // never taken: the plan keeps every slot inside the workspace
    if (real0 + nb > (size_t)p.items * p.Hkv * p.row_groups) return;
    if (real0 != item0 || nb != n) {
      item0 = real0;
      n = nb;
      batch_loads(0);
    }
    nact = n;
  } else {
    nact = min(bad || L == 0 ? 1 : (L + p.chunk - 1) / p.chunk, p.splits);
  }

  float mx = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nact; s0 += kRedBatch * PG) {
    if (s0 > 0) batch_loads(s0);
    float bmx = mx;
#pragma unroll
    for (int sp = 0; sp < kRedBatch; ++sp)
      if (s0 + pg + sp * PG < nact) bmx = fmaxf(bmx, ls[sp].x);
    if (bmx > mx) {                 // first active partition: mx = -inf, the factor is 0
      const float rescale = __expf(mx - bmx);
      wsum *= rescale;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= rescale;
      mx = bmx;
    }
#pragma unroll
    for (int sp = 0; sp < kRedBatch; ++sp) {
      if (s0 + pg + sp * PG < nact) {
        const float w = __expf(ls[sp].x - mx);
        wsum += w;
        const float wk = __builtin_amdgcn_ldexpf(w, -(int)ls[sp].y);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += wk * f16_to_f32(v[sp][e] & 0xFFFFu);
          acc[2 * e + 1] += wk * f16_to_f32(v[sp][e] >> 16);
        }
      }
    }
  }
  if (PG > 1) {
    // groups 1 .. PG-1 hand (max, sum, accumulators) to group 0 of the same row and dimensions
    float *mine = red + tid * 10;
    mine[0] = mx;
    mine[1] = wsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) mine[2 + e] = acc[e];
    __syncthreads();
    if (pg != 0) return;
    float gm = mx;
#pragma unroll
    for (int q = 1; q < PG; ++q) gm = fmaxf(gm, red[(tid + q * TPR) * 10]);
    const float f0 = __expf(mx - gm);
    wsum *= f0;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= f0;
#pragma unroll
    for (int q = 1; q < PG; ++q) {
      const float *o = red + (tid + q * TPR) * 10;
      const float f = o[0] > -INFINITY ? __expf(o[0] - gm) : 0.f;  // a group with no partition
      wsum += f * o[1];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += f * o[2 + e];
    }
    mx = gm;
  }
  if (!live) return;
  const float inv = bad ? NAN : 1.0f / wsum;
  const int r = rg * p.rows_per_group + r_local;
  const int jq = r / p.S, iq = r % p.S, h = g * p.G + jq;
  const size_t o_off = (((size_t)b * p.S + iq) * p.Hq + h) * D + d8 * 8;
  if (p.out_bf16) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(p.out) + o_off) = o;
  } else {
    float *o = static_cast<float *>(p.out) + o_off;
    const f32x4 lo = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    const f32x4 hi = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    *reinterpret_cast<f32x4 *>(o) = lo;
    *reinterpret_cast<f32x4 *>(o + 4) = hi;
  }
  if (p.lse && d8 == 0) p.lse[((size_t)b * p.Hq + h) * p.S + iq] = bad ? NAN : mx + logf(wsum);
}

// fp32 path: one work-group per (position i, query head h, sequence b); keys in tiles of 256,
// each tile's values staged in LDS.
__device__ __forceinline__ float block_max_256(float x, float *red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum_256(float x, float *red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <int D>
__global__ __launch_bounds__(256) void block_attn_f32_kernel(AttnParams p) {
  // LDS: the query, the tile's 256 weights, the reduction words, the partial weighted sums of the
  // key groups, then the tile's values staged token-major [256][D] (dynamic), so that the
  // weighted sum reads LDS instead of scattered global loads.
  constexpr int KG = 256 / D;  // key groups of the weighted sum: thread t takes dimension t % D
  __shared__ float qs[D];
  __shared__ float pw[256];
  __shared__ float red[4];
  __shared__ float part[256];
  __shared__ int vpage[256];  // page of each context key of the tile
  extern __shared__ float vs[];
  const int iq = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int g = h / p.G;
  const float *q = static_cast<const float *>(p.q) + (((size_t)b * p.S + iq) * p.Hq + h) * D;
  const float *kp = static_cast<const float *>(p.k_pages);
  const float *vp = static_cast<const float *>(p.v_pages);
  const float *kb = static_cast<const float *>(p.k_blk) + ((size_t)b * p.Hkv + g) * p.S * D;
  const float *vb = static_cast<const float *>(p.v_blk) + ((size_t)b * p.Hkv + g) * D * p.S;
  const int32_t *btab = p.block_table + (size_t)b * p.max_pages;
  if (tid < D) qs[tid] = q[tid];
  const int L = p.ctx_lens[b];
  bool bad = L < 0 || L > p.max_ctx_len;
  const int Lc = bad ? 0 : L;
  const int N = p.S + Lc;  // block keys first, then the context
  float m = -INFINITY, l = 0.f, o = 0.f;
  __syncthreads();
  for (int base = 0; base < N; base += 256) {
    const int nt = min(256, N - base);
    // Page of every key of the tile first (one round trip), then this thread's key row and its
    // share of the tile's values requested together (one more), so that the tile costs two memory
    // round trips instead of one per dependent step.
    const int j = base + tid;
    int mypage = -1;
    if (j >= p.S && j < N) mypage = btab[(j - p.S) / p.page_size];
    vpage[tid] = mypage;
    __syncthreads();
    const bool key_ok = j < N && (j < p.S || (mypage >= 0 && mypage < p.num_pages));
    const float *key = nullptr;
    if (key_ok)
      key = j < p.S ? kb + (size_t)j * D
                    : kp + ((size_t)mypage * p.Hkv + g) * p.page_size * D;  // (page, head) block
    const int ko = (j - p.S) % p.page_size;
    f32x4 krow[D / 4];
#pragma unroll
    for (int d = 0; d < D; d += 4)
      krow[d / 4] = key ? *reinterpret_cast<const f32x4 *>(
                              key + (j < p.S ? (size_t)d : k_elem(ko, d, D)))
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    // the tile's values, token-major: element e = tid + 256 i is (key e / D, dimension e % D); a
    // page id outside the pool reads nothing (0). The first NV0 of a thread's D elements are
    // requested with its key row, the rest (D = 128) after those are stored.
    constexpr int NV0 = D < 64 ? D : 64;
    auto load_v = [&](int i) {
      const int e = tid + 256 * i, jl = e / D, d = e % D, jj = base + jl;
      float v = 0.f;
      if (jl < nt) {
        if (jj < p.S) {
          v = vb[(size_t)d * p.S + jj];
        } else {
          const int page = vpage[jl];
          if (page >= 0 && page < p.num_pages)
            v = vp[((size_t)page * p.Hkv + g) * p.page_size * D + v_elem((jj - p.S) % p.page_size, d, D)];
        }
      }
      return v;
    };
    float vreg[NV0];
#pragma unroll
    for (int i = 0; i < NV0; ++i) vreg[i] = load_v(i);
    // score (four independent partial dot products)
    float s = -INFINITY;
    if (j < N) {
      if (key) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          float &a = acc[(d / 4) & 3];
          a = fmaf(qs[d], krow[d / 4][0], a);
          a = fmaf(qs[d + 1], krow[d / 4][1], a);
          a = fmaf(qs[d + 2], krow[d / 4][2], a);
          a = fmaf(qs[d + 3], krow[d / 4][3], a);
        }
        s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * p.scale;
      } else {
        s = NAN;
      }
    }
    __syncthreads();  // every wave is done with the previous tile's values and weights
#pragma unroll
    for (int i = 0; i < NV0; ++i) vs[tid + 256 * i] = vreg[i];
#pragma unroll
    for (int i0 = NV0; i0 < D; i0 += NV0) {
#pragma unroll
      for (int i = 0; i < NV0; ++i) vreg[i] = load_v(i0 + i);
#pragma unroll
      for (int i = 0; i < NV0; ++i) vs[tid + 256 * (i0 + i)] = vreg[i];
    }
    const bool nan_here = s != s;
    if (__syncthreads_or(nan_here)) bad = true;
    if (nan_here) s = -INFINITY;
    const float tmax = block_max_256(s, red);
    const float mnew = fmaxf(m, tmax);
    const float alpha = expf(m - mnew);
    const float pj = j < N ? expf(s - mnew) : 0.f;
    pw[tid] = pj;
    const float psum = block_sum_256(pj, red);
    l = l * alpha + psum;
    // weighted sum: thread t sums dimension t % D over keys t / D, t / D + KG, ... of the tile
    // (four independent chains), then the KG groups are added in order
    {
      const int d = tid % D, kg = tid / D;
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
      int i = 0;
      for (int t = kg; t < nt; t += KG, ++i) a4[i & 3] = fmaf(pw[t], vs[t * D + d], a4[i & 3]);
      part[tid] = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    }
    __syncthreads();
    if (tid < D) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < KG; ++k) acc += part[k * D + tid];
      o = o * alpha + acc;
    }
    m = mnew;
    __syncthreads();
  }
  const float nanv = NAN;
  if (tid < D) {
    const float val = bad ? nanv : o / l;
    const size_t off = (((size_t)b * p.S + iq) * p.Hq + h) * D + tid;
    if (p.out_bf16)
      static_cast<uint16_t *>(p.out)[off] = f32_to_bf16(val);
    else
      static_cast<float *>(p.out)[off] = val;
  }
  if (p.lse && tid == 0) p.lse[((size_t)b * p.Hq + h) * p.S + iq] = bad ? nanv : m + logf(l);
}

hipError_t launch_block_attn_bf16(const AttnParams &p, hipStream_t stream, hipEvent_t ev_begin,
                                  hipEvent_t ev_end) {
  const int units = p.balanced ? p.Hkv * p.items : p.B * p.Hkv * p.splits;
  dim3 grid((unsigned)((units + 7) / 8 * 8 * p.row_groups));
  hipError_t e = hipSuccess;
  if (ev_begin && (e = hipEventRecord(ev_begin, stream)) != hipSuccess) return e;
  if (p.D == 128) {
    constexpr int lds = Geom<128>::LDS;
    const hipError_t attr =
        allow_dynamic_lds(reinterpret_cast<const void *>(&block_attn_bf16_kernel<128>), lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(block_attn_bf16_kernel<128>, grid, dim3(kThreads), lds, stream, p);
  } else {
    constexpr int lds = Geom<64>::LDS;
    const hipError_t attr =
        allow_dynamic_lds(reinterpret_cast<const void *>(&block_attn_bf16_kernel<64>), lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(block_attn_bf16_kernel<64>, grid, dim3(kThreads), lds, stream, p);
  }
  e = hipGetLastError();
  if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end, stream);
  return e;
}

hipError_t launch_block_attn_f32(const AttnParams &p, hipStream_t stream, hipEvent_t ev_begin,
                                 hipEvent_t ev_end) {
  dim3 grid(p.S, p.Hq, p.B);
  hipError_t e = hipSuccess;
  if (ev_begin && (e = hipEventRecord(ev_begin, stream)) != hipSuccess) return e;
  if (p.D == 128) {
    constexpr int lds = 256 * 128 * 4;
    const hipError_t attr =
        allow_dynamic_lds(reinterpret_cast<const void *>(&block_attn_f32_kernel<128>), lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(block_attn_f32_kernel<128>, grid, dim3(256), lds, stream, p);
  } else {
    constexpr int lds = 256 * 64 * 4;
    const hipError_t attr =
        allow_dynamic_lds(reinterpret_cast<const void *>(&block_attn_f32_kernel<64>), lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(block_attn_f32_kernel<64>, grid, dim3(256), lds, stream, p);
  }
  e = hipGetLastError();
  if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end, stream);
  return e;
}

// The merge's partition groups: one while a row has at most kRedBatch partitions (at 256 rows of
// 16 partitions, 256 work-groups of one round trip each were faster than 1024 of 4 groups: 6.5
// against 8.6 us); else the fewest (4 or 16) with at most kRedBatch partitions per thread.
template <int D, int PG>
static void launch_reduce_pg(const AttnParams &p, hipStream_t stream) {
  constexpr int rpb = 256 / (D / 8 * PG);
  dim3 grid(p.B * p.Hkv * p.row_groups, (p.rows_per_group + rpb - 1) / rpb);
  hipLaunchKernelGGL((attn_reduce_kernel<D, PG>), grid, dim3(256), 0, stream, p);
}

template <int D>
static void launch_reduce_d(const AttnParams &p, hipStream_t stream) {
  const int64_t units = (int64_t)p.B * p.Hkv * p.row_groups;
  auto groups = [&](int pg) {
    const int rpb = 256 / (D / 8 * pg);
    return units * ((p.rows_per_group + rpb - 1) / rpb);
  };
  // partitions of a sequence (with the balanced plan: when all lengths are equal; a sequence
  // with more takes more load batches)
  const int parts = p.splits;
  if (parts <= kRedBatch) launch_reduce_pg<D, 1>(p, stream);
  else if (parts <= 4 * kRedBatch && groups(4) >= 256) launch_reduce_pg<D, 4>(p, stream);
  else launch_reduce_pg<D, 16>(p, stream);
}

// Scratch of the no-allocation attention entry point: the split-KV partials live in this
// file-scope array instead of a caller workspace. Each device that loads the library holds its own
// copy until the process ends. Host code never uses the array's name as an address: the device
// address is looked up once per device with hipGetSymbolAddress (with that device current) and
// only that pointer is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attn_reduce(const AttnParams &p, hipStream_t stream) {
  if (p.D == 128) launch_reduce_d<128>(p, stream);
  else launch_reduce_d<64>(p, stream);
  return hipGetLastError();
}

#ifdef TT_PHASE_STAMPS
// Profiling build only: copies (or, with clear != 0, zeroes) the attention kernel's phase stamps.
extern "C" int tt_phase_stamps_attn(void *dst, size_t bytes, int clear) {
  if (clear) {
    static unsigned long long zero[8192][8];
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(attn_phase_stamps), zero, sizeof(zero), 0,
                                  hipMemcpyHostToDevice);
  }
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(attn_phase_stamps), bytes, 0,
                                  hipMemcpyDeviceToHost);
}
#endif

}  // namespace tt
