// Host-side launchers of the gfx950 kernels (internal to the library; the public ABI is
// include/twotower.h). Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tt {

// Context cache layout. A (page, KV head) block holds page_size tokens x D elements as 64-token
// tiles; a tile is made of 8-element chunks (16 bytes in bf16) in chunk-major order:
//   K tile [D / 8][64 tokens][8 dims]      (the 64 tokens of one 8-dimension chunk together)
//   V tile [8 token chunks][D][8 tokens]   (8 consecutive tokens of one dimension together)
// Element offsets of (token o of the page, dimension d) within the block:
__host__ __device__ inline size_t k_elem(int o, int d, int D) {
  return ((size_t)(o >> 6) * (D >> 3) + (d >> 3)) * 512 + (size_t)(o & 63) * 8 + (d & 7);
}
__host__ __device__ inline size_t v_elem(int o, int d, int D) {
  return (((size_t)(o >> 6) * 8 + ((o & 63) >> 3)) * D + d) * 8 + (o & 7);
}

// ---------------------------------------------------------------------------- block attention
struct AttnParams {
  const void *q, *k_pages, *v_pages, *k_blk, *v_blk;
  const int32_t *block_table, *ctx_lens;
  void *out;
  float *lse;
  void *part_o;     // [items, rows_per_group, D] fp16 normalized partial rows, row r scaled by
                    // 2^k_r (splits > 1)
  float *part_lse;  // [items, rows_per_group, 2]: (log-sum-exp, k_r) of each partial row
  int B, S, Hq, Hkv, G, D;
  int rows;            // G * S query rows per (sequence, KV head)
  int rows_per_group;  // rows handled by one work-group (multiple of 32, <= 256)
  int row_groups;
  int num_pages, page_size, max_pages, max_ctx_len;
  int chunk;   // context tokens per partition (multiple of 64); balanced plan: the largest
               // partition when every sequence has max_ctx_len tokens and is active
  int splits;  // partitions per (sequence, KV head, row group); balanced plan: the same case
  float scale;
  int out_bf16;
  // Balanced plan (automatic partition count): partitions are sized on the device from the
  // actual lengths so that every work-group gets a nearly equal share (see block_attn.hip).
  int balanced;
  int parts;      // target partitions per (KV head, row group) over the whole batch
  int max_parts;  // bound on the partitions of one sequence
  int items;      // work items per (KV head, row group) the grid and the workspace hold
  const uint8_t *active;  // optional [B, S]: a sequence with no nonzero flag has no work
  int *plan_rec;  // balanced plan with a merge: [B, 2] (partitions, partitions before) of every
                  // sequence, written by work-group 0 of the attention kernel for the merge
};

hipError_t launch_block_attn_bf16(const AttnParams &p, hipStream_t stream, hipEvent_t ev_begin,
                                  hipEvent_t ev_end);
hipError_t launch_block_attn_f32(const AttnParams &p, hipStream_t stream, hipEvent_t ev_begin,
                                 hipEvent_t ev_end);
hipError_t launch_attn_reduce(const AttnParams &p, hipStream_t stream);

// Static scratch of the no-allocation attention entry point (32 MiB per device): the device
// address of the current device's copy, looked up on the first call on that device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch_address(void **ptr);

// ------------------------------------------------------------------------------------ unmask
struct UnmaskParams {
  const float *logits;
  int64_t ld;
  uint8_t *masked;
  int32_t *tokens;
  float *confidence;
  int32_t *n_committed;
  float *part;  // [B*S, chunks, 3] (max, index bits, sum)
  int B, S, vocab, chunk, chunks;
  float threshold;
  int min_commit, commit_all;
};

hipError_t launch_unmask(const UnmaskParams &p, hipStream_t stream);
// Masked-diffusion loss: NLL of the targets at the masked rows of p.logits (row triples in
// p.part as for the unmasking), its mean over the masked rows, and the linear-schedule corruption.
struct NllParams {
  const int32_t *targets;  // [B*S]
  float *nll;              // [B*S] out, 0 at rows not masked
  float *loss;             // [1] out (may be null): mean over masked rows, 0 if none
  int32_t *count;          // [1] out (may be null): masked rows
};
hipError_t launch_masked_nll(const UnmaskParams &p, const NllParams &q, hipStream_t stream);

struct CorruptParams {
  const int32_t *clean;
  const float *u_time, *u_mask;
  int32_t *noisy;
  uint8_t *masked;
  float *t;  // may be null
  int B, S, mask_id;
};
hipError_t launch_mask_corrupt(const CorruptParams &p, hipStream_t stream);

// Decisions from per-row tile triples already in p.part ([B*S, chunks, 4]), e.g. written by the
// EPI_UNMASK linear epilogue.
hipError_t launch_unmask_tiles_finalize(const UnmaskParams &p, hipStream_t stream);

// ----------------------------------------------------------------------- context KV append
constexpr int kMaxAppendLayers = 16;
// status flags (the same values as TT_APPEND_* in include/twotower.h)
constexpr int kAppendOutOfPages = 1;
constexpr int kAppendNoRoomInTable = 2;
constexpr int kAppendBadPage = 4;

struct AppendParams {
  void *k_pages[kMaxAppendLayers];      // [num_pages, Hkv, page_size / 64, D / 8, 64, 8]
  void *v_pages[kMaxAppendLayers];      // [num_pages, Hkv, page_size / 64, 8, D, 8]
  const void *k_new[kMaxAppendLayers];  // [B, Hkv, S, D]
  const void *v_new[kMaxAppendLayers];  // [B, Hkv, D, S]
  int32_t *block_table;                 // [B, max_pages]
  int32_t *ctx_lens;                    // [B]
  const int32_t *free_pages;            // free-page stack; entries 0 .. *free_count - 1 valid
  int32_t *free_count;
  int32_t *status;                      // OR-ed flags
  int32_t *old_len;                     // workspace [B]: length before the append, -1 = skipped
  int layers, B, Hkv, D, S, page_size, max_pages, num_pages, elem_bytes;
};

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream);

// ------------------------------------------------------------------------ skinny bf16 linear
// Arrival counters of the in-kernel merge of K partials (group_arrive): one 64-bit word per output
// tile, each in its own 128-byte line.
constexpr int kSyncWords = 16;

enum Epilogue : int {
  EPI_F32 = 0,       // y fp32 [M, ldy]
  EPI_QKV = 1,       // scatter to q [B,S,Hq,D], k_blk [B,Hkv,S,D], v_blk [B,Hkv,D,S] (bf16)
  EPI_RESIDUAL = 2,  // y bf16 [M, N] = residual bf16 [M, N] + x w^T
  EPI_UNMASK = 3,    // per (row, 256-feature tile) triples for the unmasking; y fp32 optional
};

struct LinearParams {
  const void *x;  // bf16 [M, K]
  const void *w;  // bf16 [N, K], packed (twotower_pack_weight)
  int M, N, K;
  int ksplit;     // partitions of K (>= 1); > 1 uses `part` and a reduce pass
  int wide;       // 1: 256-feature work-group tiles (large N), 0: 64-feature tiles
  float *part;    // [ksplit, M, N] fp32 when ksplit > 1
  int epi;
  // EPI_F32
  float *y;
  int64_t ldy;
  // EPI_QKV
  void *q, *k_blk, *v_blk;
  int S, Hq, Hkv, D;
  // EPI_RESIDUAL
  const void *residual;
  void *y_bf16;
  // EPI_UNMASK (256-feature tiles, K not split): rows with masked[m] != 0 get, for every tile t,
  // (max, first argmax, sum of exp(y - max)) of y[m, 256 t .. 256 t + 255] at
  // triples[(m * ceil(N / 256) + t) * 4 + 0..2]; y (fp32 [M, ldy]) is also stored when not null.
  const uint8_t *masked;
  float *triples;
  // ksplit > 1: the arrival counters of an in-kernel merge of the K partials (one per output tile,
  // kSyncWords words each, see group_arrive), the launch's nonzero tag and the polls after which a
  // partition hands its share to the last one to arrive; null, or a grid that cannot be resident
  // at once: linear_reduce_kernel merges them.
  unsigned long long *sync;
  uint32_t sync_tag;
  int sync_polls;
};

hipError_t launch_linear(const LinearParams &p, hipStream_t stream);

// Packed weight layout of the linear kernels (see twotower_pack_weight).
hipError_t launch_pack_weight(const void *w, int N, int K, void *out, hipStream_t stream);

// --------------------------------------------------------------------------- measurement
// Streaming read of `bytes` (a multiple of 16) from src with `workgroups` work-groups of 256.
hipError_t launch_stream_read(const void *src, size_t bytes, int workgroups, uint32_t *sink,
                              hipStream_t stream);
// MFMA issue rate: `workgroups` x 8 waves x `iters` x 16 MFMAs 32x32x16 bf16; mode bit 0: A operand
// read from LDS per MFMA, bit 1: two work-groups per compute unit (else one). sink: workgroups x 512.
hipError_t launch_mfma_rate(int mode, int workgroups, int iters, float *sink, hipStream_t stream);

}  // namespace tt
