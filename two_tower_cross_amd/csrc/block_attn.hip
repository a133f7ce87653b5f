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
//   * K tiles [64 tokens][D] and V tiles [D][64 tokens] (V pages are dim-major) are staged in LDS
//     with 16-byte loads; chunks are XOR-swizzled by (row & 7) so the MFMA operand reads of 32
//     different rows hit distinct banks.
//   * Each wave owns 32 query rows and computes S^T = K Q^T with 32x32x16 bf16 MFMA: a lane then
//     holds one query column and 16 token rows, so the softmax max/sum is in-lane plus one swap
//     between the two wave halves. The token order inside a 32-token sub-tile is permuted (bits 2
//     and 3 of the row swapped) so that the exponentials a lane holds are exactly the B operand of
//     the next product O^T += V^T P^T, with no LDS round trip for P.
//   * Online softmax in base 2 with the scale folded into one FMA; O^T is rescaled only when a
//     row maximum moved.
//   * Partition 0 also folds in the S block keys; with several partitions each one writes a
//     normalized fp32 partial and its log-sum-exp, merged exactly by attn_reduce_kernel.
// fp32 path: one work-group per (b, query head, block position), plain fp32 arithmetic.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace tt {

constexpr int kTile = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 4;             // LDS ring depth: up to 3 tiles in flight per work-group
constexpr float kRescaleLog2 = 8.0f;   // the running max moves only when it grows by > 2^8
constexpr int kMaxPartPages = 4096;    // page ids of one partition staged in LDS (16 KB)

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// XOR keys of the 16-byte chunk swizzle. K rows (one token, D*2 bytes): the 32 lanes that read
// one MFMA operand hold tokens swap_bits23(lane) of a 32-token sub-tile, so keying on
// swap_bits23(token) gives every group of 8 (and of 16) consecutive lanes distinct chunk slots.
// V rows (one dimension, 128 bytes): distinct slots for 8 consecutive rows and, within each row
// parity, for 16 consecutive rows. Both hold for 32 and for 64 LDS banks.
template <int D>
__device__ __forceinline__ int kkey(int t) { return swap_bits23(t & 15) & (D / 8 - 1); }
__device__ __forceinline__ int vkey(int d) { return ((d >> 1) & 7) ^ ((d & 1) << 2); }

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

template <int D>
struct Geom {
  static constexpr int KBYTES = kTile * D * 2;
  static constexpr int VBYTES = D * kTile * 2;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KCH = KBYTES / 16 / kThreads;  // 16-byte K chunks per thread per tile
  static constexpr int VCH = VBYTES / 16 / kThreads;
  static constexpr int LOADS = KCH + VCH;             // DMA instructions per thread per tile
};

// Full 64-token context tile -> LDS stage, asynchronously (global_load_lds, 16 B per lane).
// Instruction j of wave w fills LDS bytes [(j*8 + w)*1024, +1024) lane by lane; the source of
// each lane is the logical chunk that the swizzle places in that slot.
template <int D>
__device__ __forceinline__ void dma_tile(char *stage, const uint16_t *kbase,
                                         const uint16_t *vbase, int page_size, int wave,
                                         int lane) {
  constexpr int KC = D / 8;
#pragma unroll
  for (int j = 0; j < Geom<D>::KCH; ++j) {
    const int seg = j * kWaves + wave;
    const int f = seg * 64 + lane;
    const int r = f / KC, p = f % KC;
    const int c = p ^ kkey<D>(r);
    __builtin_amdgcn_global_load_lds(kbase + (size_t)r * D + c * 8, LDS_PTR(stage + seg * 1024),
                                     16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < Geom<D>::VCH; ++j) {
    const int seg = j * kWaves + wave;
    const int f = seg * 64 + lane;
    const int d = f / 8, p = f % 8;
    const int c = p ^ vkey(d);
    __builtin_amdgcn_global_load_lds(vbase + (size_t)d * page_size + c * 8,
                                     LDS_PTR(stage + Geom<D>::KBYTES + seg * 1024), 16, 0, 0);
  }
}

// Partial context tile (`valid` < 64 tokens) -> LDS through registers, zero-filling the tokens
// past the end so that whatever the page holds there never reaches the MFMA.
template <int D>
__device__ void load_tail_tile(char *stage, const uint16_t *kbase, const uint16_t *vbase,
                               int page_size, int valid, int tid) {
  constexpr int KC = D / 8;
  uint16_t *ks = reinterpret_cast<uint16_t *>(stage);
  uint16_t *vs = reinterpret_cast<uint16_t *>(stage + Geom<D>::KBYTES);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int f = tid; f < kTile * KC; f += kThreads) {
    const int r = f / KC, c = f % KC;
    const u32x4 x = r < valid ? ld_global_16(kbase + (size_t)r * D + c * 8) : z;
    st_lds_16(ks + r * D + ((c ^ kkey<D>(r)) << 3), x);
  }
  for (int f = tid; f < D * 8; f += kThreads) {
    const int d = f / 8, c = f % 8;
    const int n = valid - c * 8;
    u32x4 x = n > 0 ? ld_global_16(vbase + (size_t)d * page_size + c * 8) : z;
    x = keep_first(x, n < 0 ? 0 : (n > 8 ? 8 : n));
    st_lds_16(vs + d * kTile + ((c ^ vkey(d)) << 3), x);
  }
}

// The block's own S keys/values of (b, g) into an LDS stage (element-wise; S need not be a
// multiple of 8). Tokens >= S are zero.
template <int D>
__device__ void load_block_tile(char *stage, const uint16_t *kblk, const uint16_t *vblk, int S,
                                int tid) {
  uint16_t *ks = reinterpret_cast<uint16_t *>(stage);
  uint16_t *vs = reinterpret_cast<uint16_t *>(stage + Geom<D>::KBYTES);
  for (int idx = tid; idx < kTile * D; idx += kThreads) {
    const int tok = idx / D, d = idx % D;
    const uint16_t x = tok < S ? kblk[tok * D + d] : (uint16_t)0;
    ks[tok * D + (((d >> 3) ^ kkey<D>(tok)) << 3) + (d & 7)] = x;
  }
  for (int idx = tid; idx < D * kTile; idx += kThreads) {
    const int d = idx / kTile, tok = idx % kTile;
    const uint16_t x = tok < S ? vblk[d * S + tok] : (uint16_t)0;
    vs[d * kTile + (((tok >> 3) ^ vkey(d)) << 3) + (tok & 7)] = x;
  }
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8); expcnt and
// lgkmcnt are left at their maxima so only vector-memory operations are waited for. Issued through
// the builtin so that the compiler's own wait insertion knows about them.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most `tiles_in_flight` tiles of DMA (LOADS instructions each) are outstanding.
template <int LOADS>
__device__ __forceinline__ void wait_dma(int tiles_in_flight) {
  if (tiles_in_flight >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LOADS));
  else if (tiles_in_flight == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// One LDS tile (`valid` tokens, <= 64) into the running softmax state of this wave's 32 rows.
// m is the (possibly stale) reference maximum in raw score units; it only moves when some row's
// maximum exceeds it by more than 2^kRescaleLog2 in probability, so exp2 stays <= 2^8.
template <int D, bool FULL>
__device__ __forceinline__ void attend_tile(const char *stage, int valid, const u32x4 *qreg,
                                            f32x16 *oacc, float &m, float &lpart, float c,
                                            int lane) {
  const uint16_t *ks = reinterpret_cast<const uint16_t *>(stage);
  const uint16_t *vts = reinterpret_cast<const uint16_t *>(stage + Geom<D>::KBYTES);
  const int col = lane & 31, hh = lane >> 5;
  const int kk_key = kkey<D>(swap_bits23(col));
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int base = sub * 32;
    if (!FULL && base >= valid) break;
    f32x16 s = {};
    const int tok = base + swap_bits23(col);
    const uint16_t *krow = ks + tok * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int ch = kk * 2 + hh;
      s = mfma32x32x16(ld_lds_16(krow + ((ch ^ kk_key) << 3)), qreg[kk], s);
    }
    if (!FULL) {
      const int nv = valid - base;
      if (nv < 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = (i >> 3) * 16 + hh * 8 + (i & 7);
          if (t >= nv) s[i] = -INFINITY;
        }
      }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, swap_halves(mx));
    if (__ballot((mx - m) * c > kRescaleLog2)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
      lpart *= alpha;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
      m = mnew;
    }
    const float mc = m * c;
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -mc));
      psum += p[i];
    }
    lpart += psum;
    u32x4 p0, p1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      p0[w] = pack_bf16x2(p[2 * w], p[2 * w + 1]);
      p1[w] = pack_bf16x2(p[8 + 2 * w], p[8 + 2 * w + 1]);
    }
    const int vk = vkey(col);
    const int ch0 = (sub * 4 + hh) ^ vk, ch1 = (sub * 4 + 2 + hh) ^ vk;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const uint16_t *vrow = vts + (mb * 32 + col) * kTile;
      oacc[mb] = mfma32x32x16(ld_lds_16(vrow + (ch0 << 3)), p0, oacc[mb]);
      oacc[mb] = mfma32x32x16(ld_lds_16(vrow + (ch1 << 3)), p1, oacc[mb]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void block_attn_bf16_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int split = blockIdx.x;
  const int item_bgr = blockIdx.y;
  const int rg = item_bgr % p.row_groups;
  const int g = (item_bgr / p.row_groups) % p.Hkv;
  const int b = item_bgr / (p.row_groups * p.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const int L = p.ctx_lens[b];
  bool bad = L < 0 || L > p.max_ctx_len;
  const int Lc = bad ? 0 : L;
  const int t_begin = split * p.chunk;
  const int t_end = min(Lc, t_begin + p.chunk);
  const bool has_block = split == 0;
  if (!has_block && t_begin >= Lc && !bad) return;  // partition past this sequence's context

  const int n_ctx = t_end > t_begin ? t_end - t_begin : 0;
  const int n_full = n_ctx / kTile;            // full tiles: asynchronous ring
  const int tail = n_ctx - n_full * kTile;     // tokens of the last, partial tile

  const uint16_t *kp = static_cast<const uint16_t *>(p.k_pages);
  const uint16_t *vp = static_cast<const uint16_t *>(p.v_pages);
  const int32_t *btab = p.block_table + (size_t)b * p.max_pages;
  // The partition's page ids are staged in LDS once (the ring loop then issues no vector load of
  // its own besides the DMA). Any id outside the pool makes the sequence bad: nothing is loaded
  // from it and its outputs become NaN.
  int *part_pages = reinterpret_cast<int *>(smem + kStages * Geom<D>::STAGE);
  const int pg0 = t_begin / p.page_size;
  const int n_pages = n_ctx > 0 ? (t_end - 1) / p.page_size - pg0 + 1 : 0;
  int page_bad = 0;
  for (int i = tid; i < n_pages; i += kThreads) {
    const int page = btab[pg0 + i];
    page_bad |= page < 0 || page >= p.num_pages;
    part_pages[i] = page;
  }
  if (__syncthreads_or(page_bad)) bad = true;
  const int n_full_ok = bad ? 0 : n_full;
  const int tail_ok = bad ? 0 : tail;

  auto tile_src = [&](int t0, const uint16_t *&kb, const uint16_t *&vb) {
    const int page = part_pages[t0 / p.page_size - pg0];
    const int off0 = t0 % p.page_size;
    const size_t ph = (size_t)page * p.Hkv + g;
    kb = kp + (ph * p.page_size + off0) * D;
    vb = vp + ph * D * p.page_size + off0;
  };

  // Query rows of this wave (B operand of S^T = K Q^T): row r -> (head j, position i).
  const int col = lane & 31, hh = lane >> 5;
  const int r_local = wave * 32 + col;
  const int r = rg * p.rows_per_group + r_local;
  const bool row_ok = r < p.rows && r_local < p.rows_per_group;
  const bool wave_active =
      wave * 32 < p.rows_per_group && rg * p.rows_per_group + wave * 32 < p.rows;
  const int jq = row_ok ? r / p.S : 0, iq = row_ok ? r % p.S : 0;
  const int h = g * p.G + jq;
  u32x4 qreg[D / 16];
  {
    const uint16_t *qrow =
        static_cast<const uint16_t *>(p.q) + (((size_t)b * p.S + iq) * p.Hq + h) * D;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = row_ok ? ld_global_16(qrow + kk * 16 + hh * 8) : z;
  }

  // The block's own keys (partition 0) go through the last stage, loaded before the ring starts
  // so that waiting for them never waits for context tiles.
  char *const block_stage = smem + (kStages - 1) * Geom<D>::STAGE;
  if (has_block) {
    const size_t bg = (size_t)b * p.Hkv + g;
    load_block_tile<D>(block_stage, static_cast<const uint16_t *>(p.k_blk) + bg * p.S * D,
                       static_cast<const uint16_t *>(p.v_blk) + bg * D * p.S, p.S, tid);
  }

  // Start the ring: context tiles 0 .. kStages-2 into stages 0 .. kStages-2.
#pragma unroll
  for (int n = 0; n < kStages - 1; ++n) {
    if (n < n_full_ok) {
      const uint16_t *kb, *vb;
      tile_src(t_begin + n * kTile, kb, vb);
      dma_tile<D>(smem + n * Geom<D>::STAGE, kb, vb, p.page_size, wave, lane);
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16{};
  float m = -INFINITY, lpart = 0.f;
  const float c = p.scale * kLog2e;

  // Q (and the first context tiles) have landed: inside the loop only the ring's own DMA is
  // ever waited for.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if (has_block) {
    lds_barrier();
    if (wave_active) attend_tile<D, false>(block_stage, p.S, qreg, oacc, m, lpart, c, lane);
  }

  for (int n = 0; n < n_full_ok; ++n) {
    wait_dma<Geom<D>::LOADS>(min(kStages - 2, n_full_ok - 1 - n));
    lds_barrier();  // tile n is in LDS for every wave; stage (n-1) % kStages is free again
    const int nn = n + kStages - 1;
    if (nn < n_full_ok) {
      const uint16_t *kb, *vb;
      tile_src(t_begin + nn * kTile, kb, vb);
      dma_tile<D>(smem + (nn % kStages) * Geom<D>::STAGE, kb, vb, p.page_size, wave, lane);
    }
    if (wave_active)
      attend_tile<D, true>(smem + (n % kStages) * Geom<D>::STAGE, kTile, qreg, oacc, m, lpart, c,
                           lane);
  }

  if (tail_ok > 0) {
    lds_barrier();  // every wave is done with the ring before a stage is overwritten
    const uint16_t *kb, *vb;
    tile_src(t_begin + n_full_ok * kTile, kb, vb);
    char *st = smem + (n_full_ok % kStages) * Geom<D>::STAGE;
    load_tail_tile<D>(st, kb, vb, p.page_size, tail_ok, tid);
    lds_barrier();
    if (wave_active) attend_tile<D, false>(st, tail_ok, qreg, oacc, m, lpart, c, lane);
  }

  if (!wave_active) return;
  const float l = lpart + swap_halves(lpart);
  const float inv = 1.0f / l;
  const float lse_val = bad ? NAN : m * p.scale + logf(l);
  const float nanv = NAN;
  if (p.splits == 1) {
    if (!row_ok) return;
    if (p.out_bf16) {
      uint16_t *orow = static_cast<uint16_t *>(p.out) + (((size_t)b * p.S + iq) * p.Hq + h) * D;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = mb * 32 + q4 * 8 + hh * 4;
          float o0 = bad ? nanv : oacc[mb][q4 * 4 + 0] * inv, o1 = bad ? nanv : oacc[mb][q4 * 4 + 1] * inv;
          float o2 = bad ? nanv : oacc[mb][q4 * 4 + 2] * inv, o3 = bad ? nanv : oacc[mb][q4 * 4 + 3] * inv;
          uint2 pk;
          pk.x = pack_bf16x2(o0, o1);
          pk.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<uint2 *>(orow + d) = pk;
        }
    } else {
      float *orow = static_cast<float *>(p.out) + (((size_t)b * p.S + iq) * p.Hq + h) * D;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = mb * 32 + q4 * 8 + hh * 4;
          f32x4 o;
          o[0] = bad ? nanv : oacc[mb][q4 * 4 + 0] * inv;
          o[1] = bad ? nanv : oacc[mb][q4 * 4 + 1] * inv;
          o[2] = bad ? nanv : oacc[mb][q4 * 4 + 2] * inv;
          o[3] = bad ? nanv : oacc[mb][q4 * 4 + 3] * inv;
          *reinterpret_cast<f32x4 *>(orow + d) = o;
        }
    }
    if (p.lse && hh == 0) p.lse[((size_t)b * p.Hq + h) * p.S + iq] = lse_val;
  } else {
    if (r_local >= p.rows_per_group) return;
    const size_t item = (size_t)item_bgr * p.splits + split;
    float *prow = p.part_o + (item * p.rows_per_group + r_local) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + q4 * 8 + hh * 4;
        f32x4 o;
        o[0] = bad ? nanv : oacc[mb][q4 * 4 + 0] * inv;
        o[1] = bad ? nanv : oacc[mb][q4 * 4 + 1] * inv;
        o[2] = bad ? nanv : oacc[mb][q4 * 4 + 2] * inv;
        o[3] = bad ? nanv : oacc[mb][q4 * 4 + 3] * inv;
        *reinterpret_cast<f32x4 *>(prow + d) = o;
      }
    if (hh == 0) p.part_lse[item * p.rows_per_group + r_local] = lse_val;
  }
}

// Exact merge of the partitions of each query row: with lse* = max_p lse_p and
// w_p = exp(lse_p - lse*), out = sum_p w_p O_p / sum_p w_p and lse = lse* + ln(sum_p w_p).
template <int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(AttnParams p) {
  const int item_bgr = blockIdx.x;
  const int rg = item_bgr % p.row_groups;
  const int g = (item_bgr / p.row_groups) % p.Hkv;
  const int b = item_bgr / (p.row_groups * p.Hkv);
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int r_local = e / (D / 4), d4 = e % (D / 4);
  if (r_local >= p.rows_per_group) return;
  const int r = rg * p.rows_per_group + r_local;
  if (r >= p.rows) return;
  const int jq = r / p.S, iq = r % p.S, h = g * p.G + jq;

  const int L = p.ctx_lens[b];
  const bool bad = L < 0 || L > p.max_ctx_len;
  int nact = bad || L == 0 ? 1 : (L + p.chunk - 1) / p.chunk;
  nact = min(nact, p.splits);
  const size_t item0 = (size_t)item_bgr * p.splits;
  float mx = -INFINITY;
  for (int s = 0; s < nact; ++s) mx = fmaxf(mx, p.part_lse[(item0 + s) * p.rows_per_group + r_local]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nact; ++s) {
    const float ls = p.part_lse[(item0 + s) * p.rows_per_group + r_local];
    const float w = __expf(ls - mx);
    wsum += w;
    const f32x4 o = *reinterpret_cast<const f32x4 *>(p.part_o + ((item0 + s) * p.rows_per_group + r_local) * D + d4 * 4);
    acc += w * o;
  }
  const float inv = 1.0f / wsum;
  const float nanv = NAN;
  acc *= inv;
  if (bad) acc = f32x4{nanv, nanv, nanv, nanv};
  const size_t o_off = (((size_t)b * p.S + iq) * p.Hq + h) * D + d4 * 4;
  if (p.out_bf16) {
    uint2 pk;
    pk.x = pack_bf16x2(acc[0], acc[1]);
    pk.y = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o_off) = pk;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.out) + o_off) = acc;
  }
  if (p.lse && d4 == 0) p.lse[((size_t)b * p.Hq + h) * p.S + iq] = bad ? nanv : mx + logf(wsum);
}

// fp32 path: one work-group per (position i, query head h, sequence b); keys in tiles of 256.
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
  __shared__ float qs[D];
  __shared__ float pw[256];
  __shared__ float red[4];
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
    const int j = base + tid;
    float s = -INFINITY;
    if (j < N) {
      const float *key;
      if (j < p.S) {
        key = kb + (size_t)j * D;
      } else {
        const int t = j - p.S;
        const int page = btab[t / p.page_size];
        if (page < 0 || page >= p.num_pages) {
          key = nullptr;
        } else {
          key = kp + (((size_t)page * p.Hkv + g) * p.page_size + t % p.page_size) * D;
        }
      }
      if (key) {
        float acc = 0.f;
        for (int d = 0; d < D; d += 4) {
          const f32x4 kv = *reinterpret_cast<const f32x4 *>(key + d);
          acc = fmaf(qs[d], kv[0], acc);
          acc = fmaf(qs[d + 1], kv[1], acc);
          acc = fmaf(qs[d + 2], kv[2], acc);
          acc = fmaf(qs[d + 3], kv[3], acc);
        }
        s = acc * p.scale;
      } else {
        s = NAN;
      }
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
    if (tid < D) {
      float acc = 0.f;
      const int nt = min(256, N - base);
      for (int t = 0; t < nt; ++t) {
        const int jj = base + t;
        float v;
        if (jj < p.S) {
          v = vb[(size_t)tid * p.S + jj];
        } else {
          const int tt = jj - p.S;
          const int page = btab[tt / p.page_size];
          v = (page >= 0 && page < p.num_pages)
                  ? vp[(((size_t)page * p.Hkv + g) * D + tid) * p.page_size + tt % p.page_size]
                  : 0.f;
        }
        acc = fmaf(pw[t], v, acc);
      }
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
  dim3 grid(p.splits, p.B * p.Hkv * p.row_groups);
  hipError_t e = hipSuccess;
  if (ev_begin && (e = hipEventRecord(ev_begin, stream)) != hipSuccess) return e;
  if (p.D == 128) {
    constexpr int lds = kStages * Geom<128>::STAGE + kMaxPartPages * 4;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&block_attn_bf16_kernel<128>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(block_attn_bf16_kernel<128>, grid, dim3(kThreads), lds, stream, p);
  } else {
    constexpr int lds = kStages * Geom<64>::STAGE + kMaxPartPages * 4;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&block_attn_bf16_kernel<64>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
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
  if (p.D == 128)
    hipLaunchKernelGGL(block_attn_f32_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(block_attn_f32_kernel<64>, grid, dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end, stream);
  return e;
}

hipError_t launch_attn_reduce(const AttnParams &p, hipStream_t stream) {
  const int threads_needed = p.rows_per_group * (p.D / 4);
  dim3 grid(p.B * p.Hkv * p.row_groups, (threads_needed + 255) / 256);
  if (p.D == 128)
    hipLaunchKernelGGL(attn_reduce_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_reduce_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
