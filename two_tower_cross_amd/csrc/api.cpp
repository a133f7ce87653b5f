// C ABI of the denoise-step library: argument validation, workspace sizing, partition planning
// and the composition of one denoise step. No device memory is allocated here; every kernel is
// enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdlib>

#include "../../include/twotower.h"
#include "kernels.hpp"

namespace {

constexpr int kTargetWorkgroups = 256;  // one work-group per compute unit on MI355X
constexpr int kMinChunk = 256;          // context tokens per partition, lower bound
constexpr int kMaxPartitionTiles = 4096;  // 64-token tile indices one attention work-group stages in LDS
constexpr int kMinPartTiles = 1;          // the balanced plan's smallest partition (64 tokens)
constexpr int kPlanMaxB = 256;            // sequences the balanced plan handles
constexpr int kHalfGroupRows = 128;       // query rows per work-group when partitions are short
constexpr int kHalfGroupBelowTiles = 24;  // ... i.e. below this many 64-token tiles at 256 rows
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validated geometry of one block-attention call.
struct AttnPlan {
  tt::AttnParams p{};
  size_t ws_bytes = 0;
  bool use_bf16 = false;
};

// Nonzero tag of one launch that merges its K partials inside the kernel (see group_arrive):
// a process-wide counter, started from the clock so that a workspace left over from another
// process does not hold the first tags.
uint32_t next_sync_tag() {
  static std::atomic<uint32_t> next{
      static_cast<uint32_t>(std::chrono::steady_clock::now().time_since_epoch().count())};
  for (;;) {
    const uint32_t t = next.fetch_add(1, std::memory_order_relaxed);
    if (t != 0) return t;
  }
}

// Balanced plan (see block_attn.hip): the smallest partition size c >= kMinPartTiles (in 64-token
// tiles) for which B sequences of t tiles need at most `parts` partitions, n = max(1, ceil(t / c))
// each; kMaxPartitionTiles when one partition per sequence is already too many. The device
// computes the same from the actual lengths; for equal lengths both agree.
int64_t balanced_tiles(int64_t B, int64_t t, int64_t parts) {
  auto count = [&](int64_t c) { return B * std::max<int64_t>(1, cdiv(t, c)); };
  int64_t lo = std::min<int64_t>(std::max<int64_t>(kMinPartTiles, cdiv(B * t, parts)),
                                 kMaxPartitionTiles);
  if (count(lo) <= parts) return lo;
  if (B >= parts) return kMaxPartitionTiles;
  int64_t hi = std::min<int64_t>(kMaxPartitionTiles,
                                 std::max<int64_t>(lo + 1, cdiv(B * t, parts - B)));
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if (count(mid) <= parts) hi = mid;
    else lo = mid;
  }
  return hi;
}

// Partial slots of a call (per row-group row block) and whether the merge runs.
size_t attn_slots(const tt::AttnParams &p) {
  return p.balanced ? (size_t)p.items * p.Hkv * p.row_groups
                    : (size_t)p.B * p.Hkv * p.row_groups * p.splits;
}
bool attn_needs_merge(const tt::AttnParams &p) { return p.balanced ? p.max_parts > 1 : p.splits > 1; }

tt_status plan_attn(const tt_block_attn_args *a, bool check_pointers, AttnPlan *out) {
  if (!a) return TT_EINVAL;
  if (a->batch < 0 || a->S < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1) return TT_EINVAL;
  if (a->num_q_heads % a->num_kv_heads != 0) return TT_EINVAL;
  if (a->dtype != TT_FP32 && a->dtype != TT_BF16) return TT_EINVAL;
  if (a->out_dtype != TT_FP32 && a->out_dtype != TT_BF16) return TT_EINVAL;
  if (!(a->scale > 0.f) || !std::isfinite(a->scale)) return TT_EINVAL;
  if (a->num_pages < 1 || a->page_size < 1 || a->max_pages_per_seq < 1 || a->max_ctx_len < 0)
    return TT_EINVAL;
  if ((int64_t)a->max_ctx_len > (int64_t)a->max_pages_per_seq * a->page_size) return TT_EINVAL;
  if (a->num_splits < 0) return TT_EINVAL;
  if (a->head_dim != 64 && a->head_dim != 128) return TT_ENOTSUP;
  if (a->S > 256) return TT_ENOTSUP;
  if (a->page_size % 64 != 0) return TT_ENOTSUP;
  // 64-token tiles of either pool are indexed with 32-bit integers
  if ((int64_t)a->num_pages * a->num_kv_heads * (a->page_size / 64) > INT32_MAX) return TT_ENOTSUP;
  if (a->out_dtype != TT_FP32 && a->out_dtype != a->dtype) return TT_ENOTSUP;
  if (check_pointers && a->batch > 0) {  // an empty batch reads and writes nothing
    const void *p16[] = {a->q, a->k_pages, a->v_pages, a->k_blk, a->v_blk, a->out};
    for (const void *p : p16)
      if (!p || !aligned(p, 16)) return TT_EINVAL;
    if (!a->block_table || !aligned(a->block_table, 4)) return TT_EINVAL;
    if (!a->ctx_lens || !aligned(a->ctx_lens, 4)) return TT_EINVAL;
    if (a->lse && !aligned(a->lse, 4)) return TT_EINVAL;
  }
  tt::AttnParams &p = out->p;
  p.q = a->q;
  p.k_pages = a->k_pages;
  p.v_pages = a->v_pages;
  p.k_blk = a->k_blk;
  p.v_blk = a->v_blk;
  p.block_table = a->block_table;
  p.ctx_lens = a->ctx_lens;
  p.out = a->out;
  p.lse = a->lse;
  p.B = a->batch;
  p.S = a->S;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.D = a->head_dim;
  p.num_pages = a->num_pages;
  p.page_size = a->page_size;
  p.max_pages = a->max_pages_per_seq;
  p.max_ctx_len = a->max_ctx_len;
  p.scale = a->scale;
  p.out_bf16 = a->out_dtype == TT_BF16;
  out->use_bf16 = a->dtype == TT_BF16;
  const int64_t rows = (int64_t)p.G * p.S;
  if (rows > (1 << 20)) return TT_ENOTSUP;
  p.rows = (int)rows;
  const int rows_pad = (int)cdiv(rows, 32) * 32;
  p.rows_per_group = std::min(rows_pad, 256);
  p.row_groups = (int)cdiv(rows_pad, p.rows_per_group);
  const int64_t t_max = cdiv(a->max_ctx_len, 64);
  int64_t groups = (int64_t)p.Hkv * p.row_groups;
  if (!out->use_bf16 || a->max_ctx_len == 0) {
    p.splits = 1;
    p.chunk = std::max(64, (int)cdiv(std::max(a->max_ctx_len, 1), 64) * 64);
  } else if (a->num_splits == 0 && p.B <= kPlanMaxB && t_max < (1 << 24) &&
             (int64_t)p.B * t_max < INT32_MAX) {
    // Balanced plan: the kernels size the partitions from the actual lengths; here the case of
    // every sequence at max_ctx_len (the same search as on the device) gives the speculative
    // split, and the bounds give the grid and the workspace.
    int64_t parts = std::max<int64_t>(1, kTargetWorkgroups / groups);
    int64_t c = balanced_tiles(p.B, t_max, parts);
    if (p.row_groups == 1 && rows_pad > kHalfGroupRows && c < kHalfGroupBelowTiles) {
      // Short partitions: the query rows go into groups of 128 (one active wave per SIMD), so
      // each work-group walks twice the tiles for half the rows and the split-KV partials and
      // their merge halve, which outweighs the slower half-height tiles below about 24 tiles
      // per partition (131072-token context, batch 1: 54.5 against 57.7 us per call; 4K
      // context: 21.7 against 23.6 us; the 32K loop at 32 tiles per partition is faster with
      // 256 rows: 80.0 against 84.4 us).
      p.rows_per_group = kHalfGroupRows;
      p.row_groups = (int)cdiv(rows_pad, kHalfGroupRows);
      groups = (int64_t)p.Hkv * p.row_groups;
      parts = std::max<int64_t>(1, kTargetWorkgroups / groups);
      c = balanced_tiles(p.B, t_max, parts);
    }
    p.balanced = 1;
    p.parts = (int)parts;
    p.splits = (int)std::max<int64_t>(1, cdiv(t_max, c));
    p.chunk = (int)(c * 64);
    p.items = (int)std::max<int64_t>(parts, (int64_t)p.B * cdiv(t_max, kMaxPartitionTiles));
    p.max_parts = (int)std::min<int64_t>(p.items, cdiv(t_max, kMinPartTiles));
  } else {
    const int64_t units = std::max<int64_t>(1, (int64_t)p.B * p.Hkv * p.row_groups);
    int64_t want = a->num_splits > 0 ? a->num_splits : cdiv(kTargetWorkgroups, units);
    want = std::max<int64_t>(1, want);
    int64_t chunk = cdiv(cdiv(a->max_ctx_len, want), 64) * 64;
    if (a->num_splits == 0) chunk = std::max<int64_t>(chunk, kMinChunk);
    chunk = std::max<int64_t>(chunk, 64);
    // a partition's tile indices are staged on chip: at most kMaxPartitionTiles of them
    chunk = std::min<int64_t>(chunk, (int64_t)kMaxPartitionTiles * 64);
    p.chunk = (int)chunk;
    p.splits = (int)cdiv(a->max_ctx_len, chunk);
  }
  if (p.splits > 65535 || (int64_t)p.B * p.Hkv * p.row_groups > 65535) return TT_ENOTSUP;
  if (p.balanced && (int64_t)p.items * groups * 8 > INT32_MAX) return TT_ENOTSUP;
  out->ws_bytes = 0;
  if (p.B > 0 && attn_needs_merge(p)) {
    const size_t items = attn_slots(p);
    out->ws_bytes = align_up(items * p.rows_per_group * p.D * sizeof(uint16_t)) +
                    align_up(items * p.rows_per_group * 2 * sizeof(float)) +
                    (p.balanced ? align_up((size_t)p.B * 2 * sizeof(int32_t)) : 0);
  }
  return TT_OK;
}

// e0 / e1: recorded before / after the main kernel, e2 after the merge (each may be null).
hipError_t run_attn(AttnPlan &pl, void *ws, hipStream_t stream, hipEvent_t e0, hipEvent_t e1,
                    hipEvent_t e2) {
  tt::AttnParams &p = pl.p;
  if (p.B == 0) return hipSuccess;
  hipError_t e;
  if (!pl.use_bf16) {
    e = tt::launch_block_attn_f32(p, stream, e0, e1);
    if (e == hipSuccess && e2) e = hipEventRecord(e2, stream);
    return e;
  }
  if (attn_needs_merge(p)) {
    const size_t items = attn_slots(p);
    char *w = static_cast<char *>(ws);
    const size_t o_bytes = align_up(items * p.rows_per_group * p.D * sizeof(uint16_t));
    const size_t l_bytes = align_up(items * p.rows_per_group * 2 * sizeof(float));
    p.part_o = w;
    p.part_lse = reinterpret_cast<float *>(w + o_bytes);
    p.plan_rec = p.balanced ? reinterpret_cast<int32_t *>(w + o_bytes + l_bytes) : nullptr;
  }
  e = tt::launch_block_attn_bf16(p, stream, e0, e1);
  if (e == hipSuccess && attn_needs_merge(p)) e = tt::launch_attn_reduce(p, stream);
  if (e == hipSuccess && e2) e = hipEventRecord(e2, stream);
  return e;
}

tt_status ws_protocol(size_t need, void *ws, size_t *ws_bytes, bool *launch) {
  *launch = false;
  if (!ws_bytes) return TT_EINVAL;
  if (!ws) {
    *ws_bytes = need;
    return TT_OK;
  }
  if (*ws_bytes < need) {
    *ws_bytes = need;
    return TT_ENOSPACE;
  }
  if (need > 0 && !aligned(ws, kAlign)) return TT_EINVAL;
  *launch = true;
  return TT_OK;
}

// ---------------------------------------------------------------------------------- unmask
struct UnmaskPlan {
  tt::UnmaskParams p{};
  size_t ws_bytes = 0;
};

// max_S: the decisions run one work-group of 256 threads per sequence (S <= 256); the loss has no
// such limit.
tt_status plan_unmask(const tt_unmask_args *a, bool check_logits, UnmaskPlan *out, int max_S = 256) {
  if (!a) return TT_EINVAL;
  if (a->batch < 0 || a->S < 1 || a->vocab < 1 || a->ld < a->vocab) return TT_EINVAL;
  if (std::isnan(a->threshold)) return TT_EINVAL;
  if (a->S > max_S) return TT_ENOTSUP;
  if (a->batch > 0) {  // an empty batch reads and writes nothing
    if (check_logits && (!a->logits || !aligned(a->logits, 4))) return TT_EINVAL;
    if (!a->masked || !a->tokens || !aligned(a->tokens, 4)) return TT_EINVAL;
    if (a->confidence && !aligned(a->confidence, 4)) return TT_EINVAL;
    if (a->n_committed && !aligned(a->n_committed, 4)) return TT_EINVAL;
  }
  tt::UnmaskParams &p = out->p;
  p.logits = a->logits;
  p.ld = a->ld;
  p.masked = a->masked;
  p.tokens = a->tokens;
  p.confidence = a->confidence;
  p.n_committed = a->n_committed;
  p.B = a->batch;
  p.S = a->S;
  p.vocab = a->vocab;
  p.chunk = 8192;
  p.chunks = (int)cdiv(a->vocab, p.chunk);
  p.threshold = a->threshold;
  p.min_commit = a->min_commit != 0;
  p.commit_all = a->commit_all != 0;
  if ((int64_t)p.B * p.S > 65535) return TT_ENOTSUP;
  out->ws_bytes = align_up((size_t)p.B * p.S * p.chunks * 4 * sizeof(float));
  return TT_OK;
}

hipError_t run_unmask(UnmaskPlan &pl, void *ws, hipStream_t stream) {
  if (pl.p.B == 0) return hipSuccess;
  pl.p.part = static_cast<float *>(ws);
  return tt::launch_unmask(pl.p, stream);
}

// ---------------------------------------------------------------------------------- linear
// Tile shape and K partitions of a skinny product: 256-feature tiles once N alone yields a full
// wave of work-groups (one per compute unit); otherwise 64-feature tiles with K split so that up
// to one work-group per compute unit runs, each over at least 4 chunks of 64 along K.
// X is addressed through a buffer resource with 32-bit byte offsets, and a group of 8 packed
// weight slabs too.
bool linear_fits(int64_t M, int64_t K) {
  if (M < 0 || K < 1 || M > INT32_MAX || K > INT32_MAX) return false;
  return M * K <= INT32_MAX / 2 && 8 * cdiv(K, 16) * 1024 <= INT32_MAX;
}

void choose_tiling(int M, int N, int K, tt::LinearParams *p) {
  const int64_t mt = cdiv(M, 128);
  if (mt == 0) {  // no rows: nothing is launched
    p->wide = 0;
    p->ksplit = 1;
    return;
  }
  p->wide = cdiv(N, 256) * mt >= kTargetWorkgroups ? 1 : 0;
  if (p->wide) {
    p->ksplit = 1;
    return;
  }
  const int64_t tiles = cdiv(N, 64) * mt;
  int64_t ks = kTargetWorkgroups / tiles;
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, cdiv(K, 64) / 4));
  p->ksplit = (int)std::max<int64_t>(1, ks);
}

// Workspace of a product with K partitions: the fp32 partials, then one arrival counter per output
// tile for the merge inside the kernel.
size_t linear_part_bytes(const tt::LinearParams &p) {
  return p.ksplit > 1 ? align_up((size_t)p.ksplit * p.M * p.N * sizeof(float)) : 0;
}
size_t linear_sync_bytes(const tt::LinearParams &p) {
  if (p.ksplit <= 1) return 0;
  const int64_t tiles = cdiv(p.N, p.wide ? 256 : 64) * cdiv(p.M, 128);
  return align_up((size_t)tiles * tt::kSyncWords * sizeof(unsigned long long));
}
size_t linear_ws(const tt::LinearParams &p) { return linear_part_bytes(p) + linear_sync_bytes(p); }

// Whether K partials may be merged inside the product kernel: yes unless the environment sets
// TWOTOWER_MERGE_IN_KERNEL=0 (read at every call).
bool merge_in_kernel_allowed() {
  const char *v = std::getenv("TWOTOWER_MERGE_IN_KERNEL");
  return !(v && v[0] == '0' && v[1] == '\0');
}

// Polls (about 1.5 us each) after which a partition of the in-kernel merge hands its share to the
// last one to arrive: TWOTOWER_MERGE_WAIT_POLLS (read at every call; 0 hands every share over at
// once), default 256. In a normal launch the partitions of a tile arrive within a few polls.
constexpr int kDefaultMergeWaitPolls = 256;
int merge_wait_polls() {
  const char *v = std::getenv("TWOTOWER_MERGE_WAIT_POLLS");
  if (!v || !*v) return kDefaultMergeWaitPolls;
  char *end = nullptr;
  const long n = std::strtol(v, &end, 10);
  if (*end != '\0' || n < 0) return kDefaultMergeWaitPolls;
  return (int)std::min<long>(n, 1L << 20);
}

// sync: the counters (linear_sync_bytes), or null for the separate merge kernel.
hipError_t run_linear(tt::LinearParams p, void *ws, void *sync, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  p.part = static_cast<float *>(ws);
  p.sync = p.ksplit > 1 && merge_in_kernel_allowed() ? static_cast<unsigned long long *>(sync)
                                                     : nullptr;
  if (p.sync) {
    p.sync_tag = next_sync_tag();
    p.sync_polls = merge_wait_polls();
  }
  return tt::launch_linear(p, stream);
}
hipError_t run_linear(const tt::LinearParams &p, void *ws, hipStream_t stream) {
  return run_linear(p, ws, static_cast<char *>(ws) + linear_part_bytes(p), stream);
}

tt_status plan_qkv(const tt_qkv_args *a, bool check_pointers, tt::LinearParams *p) {
  if (!a) return TT_EINVAL;
  if (a->batch < 0 || a->S < 1 || a->hidden < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1 ||
      a->head_dim < 1)
    return TT_EINVAL;
  if (a->hidden % 8 != 0 || a->head_dim % 4 != 0) return TT_ENOTSUP;
  if (check_pointers && a->batch > 0) {
    if (!a->h || !a->w_qkv || !aligned(a->h, 16) || !aligned(a->w_qkv, 16)) return TT_EINVAL;
    if (!a->q || !a->k_blk || !a->v_blk || !aligned(a->q, 8) || !aligned(a->k_blk, 8) ||
        !aligned(a->v_blk, 2))
      return TT_EINVAL;
  }
  if (!linear_fits((int64_t)a->batch * a->S, a->hidden)) return TT_ENOTSUP;
  const int64_t n = ((int64_t)a->num_q_heads + 2 * (int64_t)a->num_kv_heads) * a->head_dim;
  if (n > INT32_MAX) return TT_ENOTSUP;
  *p = tt::LinearParams{};
  p->x = a->h;
  p->w = a->w_qkv;
  p->M = a->batch * a->S;
  p->N = (int)n;
  p->K = a->hidden;
  p->epi = tt::EPI_QKV;
  p->q = a->q;
  p->k_blk = a->k_blk;
  p->v_blk = a->v_blk;
  p->S = a->S;
  p->Hq = a->num_q_heads;
  p->Hkv = a->num_kv_heads;
  p->D = a->head_dim;
  choose_tiling(p->M, p->N, p->K, p);
  return TT_OK;
}

tt_status plan_out(const tt_out_proj_args *a, bool check_pointers, tt::LinearParams *p) {
  if (!a) return TT_EINVAL;
  if (a->rows < 0 || a->hidden < 1 || a->in_features < 1) return TT_EINVAL;
  if (a->hidden % 4 != 0 || a->in_features % 8 != 0) return TT_ENOTSUP;
  if (check_pointers && a->rows > 0) {
    if (!a->h_in || !a->o || !a->w_o || !a->h_out) return TT_EINVAL;
    if (!aligned(a->o, 16) || !aligned(a->w_o, 16) || !aligned(a->h_in, 8) || !aligned(a->h_out, 8))
      return TT_EINVAL;
  }
  if (!linear_fits(a->rows, a->in_features)) return TT_ENOTSUP;
  *p = tt::LinearParams{};
  p->x = a->o;
  p->w = a->w_o;
  p->M = a->rows;
  p->N = a->hidden;
  p->K = a->in_features;
  p->epi = tt::EPI_RESIDUAL;
  p->residual = a->h_in;
  p->y_bf16 = a->h_out;
  choose_tiling(p->M, p->N, p->K, p);
  return TT_OK;
}

tt_status plan_lm(const tt_lm_head_args *a, bool check_pointers, tt::LinearParams *p) {
  if (!a) return TT_EINVAL;
  if (a->rows < 0 || a->hidden < 1 || a->vocab < 1 || a->ld < a->vocab) return TT_EINVAL;
  if (a->hidden % 8 != 0 || a->vocab % 4 != 0 || a->ld % 4 != 0) return TT_ENOTSUP;
  if (check_pointers && a->rows > 0) {
    if (!a->h || !a->w_lm || !a->logits) return TT_EINVAL;
    if (!aligned(a->h, 16) || !aligned(a->w_lm, 16) || !aligned(a->logits, 16)) return TT_EINVAL;
  }
  if (!linear_fits(a->rows, a->hidden)) return TT_ENOTSUP;
  *p = tt::LinearParams{};
  p->x = a->h;
  p->w = a->w_lm;
  p->M = a->rows;
  p->N = a->vocab;
  p->K = a->hidden;
  p->epi = tt::EPI_F32;
  p->y = a->logits;
  p->ldy = a->ld;
  choose_tiling(p->M, p->N, p->K, p);
  return TT_OK;
}

// lm-head fused with the unmasking: 256-feature tiles over all of K (no split), tile triples in
// the workspace, then the per-sequence decisions.
struct LmUnmaskPlan {
  tt::LinearParams lp{};
  UnmaskPlan up;
  size_t ws_bytes = 0;
};

tt_status plan_lm_unmask(const tt_lm_head_unmask_args *a, bool check_pointers, LmUnmaskPlan *out) {
  if (!a) return TT_EINVAL;
  const tt_lm_head_args &l = a->lm;
  if (l.rows < 0 || l.hidden < 1 || l.vocab < 1) return TT_EINVAL;
  if (l.hidden % 8 != 0 || l.vocab % 4 != 0) return TT_ENOTSUP;
  if (l.logits && (l.ld < l.vocab || l.ld % 4 != 0)) return l.ld < l.vocab ? TT_EINVAL : TT_ENOTSUP;
  if (check_pointers && l.rows > 0) {
    if (!l.h || !l.w_lm || !aligned(l.h, 16) || !aligned(l.w_lm, 16)) return TT_EINVAL;
    if (l.logits && !aligned(l.logits, 16)) return TT_EINVAL;
  }
  if (!linear_fits(l.rows, l.hidden)) return TT_ENOTSUP;
  tt_unmask_args ua = a->unmask;
  ua.vocab = l.vocab;
  ua.ld = l.vocab;
  ua.logits = nullptr;
  tt_status st = plan_unmask(&ua, false, &out->up);
  if (st != TT_OK) return st;
  if ((int64_t)ua.batch * ua.S != l.rows) return TT_EINVAL;
  tt::LinearParams &p = out->lp;
  p = tt::LinearParams{};
  p.x = l.h;
  p.w = l.w_lm;
  p.M = l.rows;
  p.N = l.vocab;
  p.K = l.hidden;
  p.epi = tt::EPI_UNMASK;
  p.y = l.logits;
  p.ldy = l.logits ? l.ld : 0;
  p.wide = 1;
  p.ksplit = 1;
  p.masked = ua.masked;
  const int tiles = (int)cdiv(l.vocab, 256);
  out->up.p.chunks = tiles;
  out->up.p.chunk = 256;
  out->ws_bytes = align_up((size_t)l.rows * tiles * 4 * sizeof(float));
  return TT_OK;
}

hipError_t run_lm_unmask(LmUnmaskPlan &pl, void *ws, hipStream_t stream) {
  if (pl.lp.M == 0) return hipSuccess;
  pl.lp.triples = static_cast<float *>(ws);
  pl.up.p.part = static_cast<float *>(ws);
  hipError_t e = tt::launch_linear(pl.lp, stream);
  if (e != hipSuccess) return e;
  return tt::launch_unmask_tiles_finalize(pl.up.p, stream);
}

tt_status hip_status(hipError_t e) { return e == hipSuccess ? TT_OK : TT_EHIP; }

// ---------------------------------------------------------------------------- KV append
static_assert(TT_APPEND_OUT_OF_PAGES == tt::kAppendOutOfPages &&
                  TT_APPEND_NO_ROOM_IN_TABLE == tt::kAppendNoRoomInTable &&
                  TT_APPEND_BAD_PAGE == tt::kAppendBadPage,
              "append status flags");

tt_status plan_append(const tt_kv_append_args *a, tt::AppendParams *p, size_t *ws_bytes) {
  if (!a) return TT_EINVAL;
  if (a->num_layers < 1 || a->batch < 0 || a->num_kv_heads < 1 || a->head_dim < 1 || a->S < 1)
    return TT_EINVAL;
  if (a->num_pages < 1 || a->page_size < 1 || a->max_pages_per_seq < 1) return TT_EINVAL;
  if (a->dtype != TT_FP32 && a->dtype != TT_BF16) return TT_EINVAL;
  if (a->num_layers > tt::kMaxAppendLayers || a->page_size % 64 != 0) return TT_ENOTSUP;
  if ((int64_t)a->max_pages_per_seq * a->page_size > INT32_MAX ||
      (int64_t)a->batch * a->max_pages_per_seq > INT32_MAX || a->batch > 65535)
    return TT_ENOTSUP;
  if (!a->k_pages || !a->v_pages || !a->k_new || !a->v_new) return TT_EINVAL;  // host arrays
  // an empty batch reads and writes nothing: its device pointers may be null
  const bool work = a->batch > 0;
  if (work && (!a->block_table || !a->ctx_lens || !a->free_pages || !a->free_count || !a->status))
    return TT_EINVAL;
  const uintptr_t es = a->dtype == TT_BF16 ? 2 : 4;
  *p = tt::AppendParams{};
  for (int l = 0; l < a->num_layers; ++l) {
    const void *ptrs[] = {a->k_pages[l], a->v_pages[l], a->k_new[l], a->v_new[l]};
    for (const void *q : ptrs)
      if (work && (!q || !aligned(q, es))) return TT_EINVAL;
    p->k_pages[l] = a->k_pages[l];
    p->v_pages[l] = a->v_pages[l];
    p->k_new[l] = a->k_new[l];
    p->v_new[l] = a->v_new[l];
  }
  p->block_table = a->block_table;
  p->ctx_lens = a->ctx_lens;
  p->free_pages = a->free_pages;
  p->free_count = a->free_count;
  p->status = a->status;
  p->layers = a->num_layers;
  p->B = a->batch;
  p->Hkv = a->num_kv_heads;
  p->D = a->head_dim;
  p->S = a->S;
  p->page_size = a->page_size;
  p->max_pages = a->max_pages_per_seq;
  p->num_pages = a->num_pages;
  p->elem_bytes = (int)es;
  *ws_bytes = align_up((size_t)a->batch * sizeof(int32_t));
  return TT_OK;
}

}  // namespace

extern "C" {

size_t twotower_packed_weight_bytes(int32_t out_features, int32_t in_features) {
  if (out_features < 1 || in_features < 1) return 0;
  return (size_t)cdiv(out_features, 32) * (size_t)cdiv(in_features, 16) * 1024;
}

tt_status twotower_pack_weight(const void *w, int32_t out_features, int32_t in_features,
                               void *packed, void *stream) {
  if (out_features < 1 || in_features < 1) return TT_EINVAL;
  if (in_features % 8 != 0) return TT_ENOTSUP;
  // one packed group of 8 slabs is addressed with 32-bit byte offsets
  if ((int64_t)8 * cdiv(in_features, 16) * 1024 > INT32_MAX) return TT_ENOTSUP;
  if (!w || !packed || !aligned(w, 16) || !aligned(packed, 16)) return TT_EINVAL;
  return hip_status(
      tt::launch_pack_weight(w, out_features, in_features, packed, static_cast<hipStream_t>(stream)));
}

tt_status twotower_block_attn(const tt_block_attn_args *args, void *ws, size_t *ws_bytes,
                              void *stream) {
  AttnPlan pl;
  tt_status st = plan_attn(args, true, &pl);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(pl.ws_bytes, ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  if (args->timing_events)
    for (int i = 0; i < 3; ++i) ev[i] = static_cast<hipEvent_t>(args->timing_events[i]);
  return hip_status(run_attn(pl, ws, static_cast<hipStream_t>(stream), ev[0], ev[1], ev[2]));
}

static_assert(TWOTOWER_STATIC_SCRATCH_BYTES == tt::kStaticScratchBytes, "static scratch size");

tt_status twotower_block_attn_static(const tt_block_attn_args *args, void *stream) {
  AttnPlan pl;
  tt_status st = plan_attn(args, true, &pl);
  if (st != TT_OK) return st;
  if (pl.ws_bytes > tt::kStaticScratchBytes) {
    if (args->num_splits != 0) return TT_ENOSPACE;
    // the library's own partition count, lowered until the partials fit the scratch
    const tt::AttnParams &p = pl.p;
    const size_t per_split = (size_t)p.B * p.Hkv * p.row_groups * p.rows_per_group *
                             (p.D * sizeof(uint16_t) + 2 * sizeof(float));
    tt_block_attn_args a = *args;
    a.num_splits = (int32_t)std::max<size_t>(1, (tt::kStaticScratchBytes - 2 * kAlign) / per_split);
    if ((st = plan_attn(&a, true, &pl)) != TT_OK) return st;
    if (pl.ws_bytes > tt::kStaticScratchBytes) return TT_ENOSPACE;
  }
  void *scratch = nullptr;
  if (pl.ws_bytes > 0 && tt::static_scratch_address(&scratch) != hipSuccess) return TT_EHIP;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  if (args->timing_events)
    for (int i = 0; i < 3; ++i) ev[i] = static_cast<hipEvent_t>(args->timing_events[i]);
  return hip_status(run_attn(pl, scratch, static_cast<hipStream_t>(stream), ev[0], ev[1], ev[2]));
}

tt_status twotower_unmask(const tt_unmask_args *args, void *ws, size_t *ws_bytes, void *stream) {
  UnmaskPlan pl;
  tt_status st = plan_unmask(args, true, &pl);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(pl.ws_bytes, ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  return hip_status(run_unmask(pl, ws, static_cast<hipStream_t>(stream)));
}

tt_status twotower_qkv_projection(const tt_qkv_args *args, void *ws, size_t *ws_bytes,
                                  void *stream) {
  tt::LinearParams p;
  tt_status st = plan_qkv(args, true, &p);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(linear_ws(p), ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  return hip_status(run_linear(p, ws, static_cast<hipStream_t>(stream)));
}

tt_status twotower_out_projection(const tt_out_proj_args *args, void *ws, size_t *ws_bytes,
                                  void *stream) {
  tt::LinearParams p;
  tt_status st = plan_out(args, true, &p);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(linear_ws(p), ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  return hip_status(run_linear(p, ws, static_cast<hipStream_t>(stream)));
}

tt_status twotower_lm_head(const tt_lm_head_args *args, void *ws, size_t *ws_bytes, void *stream) {
  tt::LinearParams p;
  tt_status st = plan_lm(args, true, &p);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(linear_ws(p), ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  return hip_status(run_linear(p, ws, static_cast<hipStream_t>(stream)));
}

tt_status twotower_mask_corrupt(const tt_mask_corrupt_args *a, void *ws, size_t *ws_bytes,
                                void *stream) {
  if (!a) return TT_EINVAL;
  if (a->batch < 0 || a->S < 1) return TT_EINVAL;
  if ((int64_t)a->batch * a->S > INT32_MAX / 2) return TT_ENOTSUP;
  if (a->batch > 0) {  // an empty batch reads and writes nothing
    if (!a->clean || !a->u_time || !a->u_mask || !a->noisy || !a->masked) return TT_EINVAL;
    const void *p4[] = {a->clean, a->u_time, a->u_mask, a->noisy};
    for (const void *q : p4)
      if (!aligned(q, 4)) return TT_EINVAL;
    if (a->t_out && !aligned(a->t_out, 4)) return TT_EINVAL;
  }
  bool launch;
  tt_status st = ws_protocol(0, ws, ws_bytes, &launch);
  if (st != TT_OK || !launch || a->batch == 0) return st;
  tt::CorruptParams p{};
  p.clean = a->clean;
  p.u_time = a->u_time;
  p.u_mask = a->u_mask;
  p.noisy = a->noisy;
  p.masked = a->masked;
  p.t = a->t_out;
  p.B = a->batch;
  p.S = a->S;
  p.mask_id = a->mask_id;
  return hip_status(tt::launch_mask_corrupt(p, static_cast<hipStream_t>(stream)));
}

tt_status twotower_masked_nll(const tt_masked_nll_args *a, void *ws, size_t *ws_bytes,
                              void *stream) {
  if (!a) return TT_EINVAL;
  if (a->batch > 0) {  // an empty batch reads and writes nothing
    if (!a->targets || !a->nll || !aligned(a->targets, 4) || !aligned(a->nll, 4)) return TT_EINVAL;
    if ((a->loss && !aligned(a->loss, 4)) || (a->n_masked && !aligned(a->n_masked, 4)))
      return TT_EINVAL;
  }
  // the row reduction is the unmasking's: reuse its plan (masked rows, chunk triples)
  tt_unmask_args ua{};
  ua.batch = a->batch;
  ua.S = a->S;
  ua.vocab = a->vocab;
  ua.ld = a->ld;
  ua.logits = a->logits;
  ua.masked = const_cast<uint8_t *>(a->masked);
  ua.tokens = const_cast<int32_t *>(a->targets);  // only checked, never written here
  ua.threshold = 0.f;
  if (a->S < 1) return TT_EINVAL;
  UnmaskPlan up;
  tt_status st = plan_unmask(&ua, true, &up, /*max_S=*/65535);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(up.ws_bytes, ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  if (a->batch == 0) return TT_OK;
  up.p.part = static_cast<float *>(ws);
  tt::NllParams q{};
  q.targets = a->targets;
  q.nll = a->nll;
  q.loss = a->loss;
  q.count = a->n_masked;
  return hip_status(tt::launch_masked_nll(up.p, q, static_cast<hipStream_t>(stream)));
}

tt_status twotower_kv_append(const tt_kv_append_args *args, void *ws, size_t *ws_bytes,
                             void *stream) {
  tt::AppendParams p;
  size_t need = 0;
  tt_status st = plan_append(args, &p, &need);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(need, ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  if (p.B == 0) return TT_OK;
  p.old_len = static_cast<int32_t *>(ws);
  return hip_status(tt::launch_kv_append(p, static_cast<hipStream_t>(stream)));
}

tt_status twotower_lm_head_unmask(const tt_lm_head_unmask_args *args, void *ws, size_t *ws_bytes,
                                  void *stream) {
  LmUnmaskPlan pl;
  tt_status st = plan_lm_unmask(args, true, &pl);
  if (st != TT_OK) return st;
  bool launch;
  st = ws_protocol(pl.ws_bytes, ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  return hip_status(run_lm_unmask(pl, ws, static_cast<hipStream_t>(stream)));
}

tt_status twotower_denoise_step(const tt_denoise_step_args *a, void *ws, size_t *ws_bytes,
                                void *stream) {
  if (!a || a->num_layers < 1 || a->hidden < 1 || a->vocab < 1) return TT_EINVAL;
  const tt_block_attn_args &g = a->attn;
  if (g.dtype != TT_BF16) return TT_ENOTSUP;
  if (!a->k_pages || !a->v_pages || !a->w_qkv || !a->w_o || !a->k_blk || !a->v_blk)
    return TT_EINVAL;  // host arrays
  // an empty batch reads and writes nothing: its device pointers may be null
  if (g.batch > 0 && (!a->w_lm || !a->h_in || !a->h_work || !a->q || !a->attn_out))
    return TT_EINVAL;

  // Plan every stage once (layer 0's pointers; the geometry is shared by all layers).
  tt_block_attn_args ga = g;
  ga.q = a->q;
  ga.k_pages = a->k_pages[0];
  ga.v_pages = a->v_pages[0];
  ga.k_blk = a->k_blk[0];
  ga.v_blk = a->v_blk[0];
  ga.out = a->attn_out;
  ga.out_dtype = TT_BF16;
  ga.lse = nullptr;
  AttnPlan ap;
  tt_status st = plan_attn(&ga, true, &ap);
  if (st != TT_OK) return st;
  // sequences with no masked position left get no attention work (balanced plan)
  ap.p.active = a->unmask.masked;

  tt_qkv_args qa{};
  qa.batch = g.batch;
  qa.S = g.S;
  qa.hidden = a->hidden;
  qa.num_q_heads = g.num_q_heads;
  qa.num_kv_heads = g.num_kv_heads;
  qa.head_dim = g.head_dim;
  qa.h = a->h_in;
  qa.w_qkv = a->w_qkv[0];
  qa.q = a->q;
  qa.k_blk = a->k_blk[0];
  qa.v_blk = a->v_blk[0];
  tt::LinearParams qp;
  if ((st = plan_qkv(&qa, true, &qp)) != TT_OK) return st;

  tt_out_proj_args oa{};
  oa.rows = g.batch * g.S;
  oa.hidden = a->hidden;
  oa.in_features = g.num_q_heads * g.head_dim;
  oa.h_in = a->h_in;
  oa.o = a->attn_out;
  oa.w_o = a->w_o[0];
  oa.h_out = a->h_work;
  tt::LinearParams op;
  if ((st = plan_out(&oa, true, &op)) != TT_OK) return st;

  tt_lm_head_unmask_args lu{};
  lu.lm.rows = g.batch * g.S;
  lu.lm.hidden = a->hidden;
  lu.lm.vocab = a->vocab;
  lu.lm.ld = a->logits_ld;
  lu.lm.h = a->h_work;
  lu.lm.w_lm = a->w_lm;
  lu.lm.logits = a->logits;
  lu.unmask = a->unmask;
  lu.unmask.batch = g.batch;
  lu.unmask.S = g.S;
  LmUnmaskPlan lup;
  if ((st = plan_lm_unmask(&lu, true, &lup)) != TT_OK) return st;

  for (int l = 0; l < a->num_layers && g.batch > 0; ++l) {
    const void *p16[] = {a->k_pages[l], a->v_pages[l], a->w_qkv[l], a->w_o[l]};
    for (const void *p : p16)
      if (!p || !aligned(p, 16)) return TT_EINVAL;
    if (!a->k_blk[l] || !a->v_blk[l] || !aligned(a->k_blk[l], 16) || !aligned(a->v_blk[l], 16))
      return TT_EINVAL;
  }

  // The stages share the workspace; the arrival counters of the two products follow everything
  // they share, each in a region of its own, so that only the counting writes them.
  const size_t q_sync =
      std::max({ap.ws_bytes, lup.ws_bytes, linear_part_bytes(qp), linear_part_bytes(op)});
  const size_t o_sync = q_sync + linear_sync_bytes(qp);
  const size_t need = o_sync + linear_sync_bytes(op);
  bool launch;
  st = ws_protocol(need, ws, ws_bytes, &launch);
  if (st != TT_OK || !launch) return st;
  if (g.batch == 0) return TT_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int l = 0; l < a->num_layers; ++l) {
    const void *h_prev = l == 0 ? a->h_in : a->h_work;
    qp.x = h_prev;
    qp.w = a->w_qkv[l];
    qp.k_blk = a->k_blk[l];
    qp.v_blk = a->v_blk[l];
    hipError_t e = run_linear(qp, ws, static_cast<char *>(ws) + q_sync, s);
    if (e != hipSuccess) return TT_EHIP;
    AttnPlan al = ap;
    al.p.k_pages = a->k_pages[l];
    al.p.v_pages = a->v_pages[l];
    al.p.k_blk = a->k_blk[l];
    al.p.v_blk = a->v_blk[l];
    hipEvent_t e0 = nullptr, e1 = nullptr, e2 = nullptr;
    if (a->timing_events) {
      e0 = static_cast<hipEvent_t>(a->timing_events[3 * l]);
      e1 = static_cast<hipEvent_t>(a->timing_events[3 * l + 1]);
      e2 = static_cast<hipEvent_t>(a->timing_events[3 * l + 2]);
    }
    if ((e = run_attn(al, ws, s, e0, e1, e2)) != hipSuccess) return TT_EHIP;
    op.residual = h_prev;
    op.w = a->w_o[l];
    if ((e = run_linear(op, ws, static_cast<char *>(ws) + o_sync, s)) != hipSuccess) return TT_EHIP;
  }
  if (run_lm_unmask(lup, ws, s) != hipSuccess) return TT_EHIP;
  return TT_OK;
}

tt_status twotower_probe_stream_read(const void *src, size_t bytes, int32_t workgroups,
                                     uint32_t *sink, void *stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(src, 16) || !aligned(sink, 4))
    return TT_EINVAL;
  if (workgroups < 1 || workgroups > 65536) return TT_EINVAL;
  return hip_status(
      tt::launch_stream_read(src, bytes, workgroups, sink, static_cast<hipStream_t>(stream)));
}

tt_status twotower_probe_mfma_rate(int32_t mode, int32_t workgroups, int32_t iters, float *sink,
                                   void *stream) {
  if (!sink || !aligned(sink, 4) || mode < 0 || mode > 3) return TT_EINVAL;
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20)) return TT_EINVAL;
  return hip_status(tt::launch_mfma_rate(mode, workgroups, iters, sink,
                                         static_cast<hipStream_t>(stream)));
}

const char *twotower_status_string(int32_t status) {
  switch (status) {
    case TT_OK: return "TT_OK";
    case TT_EINVAL: return "TT_EINVAL";
    case TT_ENOTSUP: return "TT_ENOTSUP";
    case TT_ENOSPACE: return "TT_ENOSPACE";
    case TT_EHIP: return "TT_EHIP";
    default: return "TT_UNKNOWN";
  }
}

int32_t twotower_abi_version(void) { return TWOTOWER_ABI_VERSION; }

int64_t twotower_struct_size(int32_t which) {
  switch (which) {
    case 0: return sizeof(tt_block_attn_args);
    case 1: return sizeof(tt_unmask_args);
    case 2: return sizeof(tt_qkv_args);
    case 3: return sizeof(tt_out_proj_args);
    case 4: return sizeof(tt_lm_head_args);
    case 5: return sizeof(tt_denoise_step_args);
    case 6: return sizeof(tt_lm_head_unmask_args);
    case 7: return sizeof(tt_kv_append_args);
    case 8: return sizeof(tt_mask_corrupt_args);
    case 9: return sizeof(tt_masked_nll_args);
    default: return -1;
  }
}

#define TT_OFF(T, f) (int64_t) offsetof(T, f)
int64_t twotower_struct_offset(int32_t which, int32_t field) {
  static const int64_t attn[] = {
      TT_OFF(tt_block_attn_args, batch), TT_OFF(tt_block_attn_args, S),
      TT_OFF(tt_block_attn_args, num_q_heads), TT_OFF(tt_block_attn_args, num_kv_heads),
      TT_OFF(tt_block_attn_args, head_dim), TT_OFF(tt_block_attn_args, dtype),
      TT_OFF(tt_block_attn_args, out_dtype), TT_OFF(tt_block_attn_args, scale),
      TT_OFF(tt_block_attn_args, q), TT_OFF(tt_block_attn_args, k_pages),
      TT_OFF(tt_block_attn_args, v_pages), TT_OFF(tt_block_attn_args, num_pages),
      TT_OFF(tt_block_attn_args, page_size), TT_OFF(tt_block_attn_args, max_pages_per_seq),
      TT_OFF(tt_block_attn_args, max_ctx_len), TT_OFF(tt_block_attn_args, block_table),
      TT_OFF(tt_block_attn_args, ctx_lens), TT_OFF(tt_block_attn_args, k_blk),
      TT_OFF(tt_block_attn_args, v_blk), TT_OFF(tt_block_attn_args, out),
      TT_OFF(tt_block_attn_args, lse), TT_OFF(tt_block_attn_args, num_splits),
      TT_OFF(tt_block_attn_args, reserved0), TT_OFF(tt_block_attn_args, timing_events)};
  static const int64_t unm[] = {
      TT_OFF(tt_unmask_args, batch), TT_OFF(tt_unmask_args, S), TT_OFF(tt_unmask_args, vocab),
      TT_OFF(tt_unmask_args, reserved0), TT_OFF(tt_unmask_args, ld),
      TT_OFF(tt_unmask_args, logits), TT_OFF(tt_unmask_args, masked),
      TT_OFF(tt_unmask_args, tokens), TT_OFF(tt_unmask_args, confidence),
      TT_OFF(tt_unmask_args, n_committed), TT_OFF(tt_unmask_args, threshold),
      TT_OFF(tt_unmask_args, min_commit), TT_OFF(tt_unmask_args, commit_all),
      TT_OFF(tt_unmask_args, reserved1)};
  static const int64_t qkv[] = {
      TT_OFF(tt_qkv_args, batch), TT_OFF(tt_qkv_args, S), TT_OFF(tt_qkv_args, hidden),
      TT_OFF(tt_qkv_args, num_q_heads), TT_OFF(tt_qkv_args, num_kv_heads),
      TT_OFF(tt_qkv_args, head_dim), TT_OFF(tt_qkv_args, h), TT_OFF(tt_qkv_args, w_qkv),
      TT_OFF(tt_qkv_args, q), TT_OFF(tt_qkv_args, k_blk), TT_OFF(tt_qkv_args, v_blk)};
  static const int64_t outp[] = {
      TT_OFF(tt_out_proj_args, rows), TT_OFF(tt_out_proj_args, hidden),
      TT_OFF(tt_out_proj_args, in_features), TT_OFF(tt_out_proj_args, reserved0),
      TT_OFF(tt_out_proj_args, h_in), TT_OFF(tt_out_proj_args, o), TT_OFF(tt_out_proj_args, w_o),
      TT_OFF(tt_out_proj_args, h_out)};
  static const int64_t lm[] = {
      TT_OFF(tt_lm_head_args, rows), TT_OFF(tt_lm_head_args, hidden),
      TT_OFF(tt_lm_head_args, vocab), TT_OFF(tt_lm_head_args, reserved0),
      TT_OFF(tt_lm_head_args, ld), TT_OFF(tt_lm_head_args, h), TT_OFF(tt_lm_head_args, w_lm),
      TT_OFF(tt_lm_head_args, logits)};
  static const int64_t step[] = {
      TT_OFF(tt_denoise_step_args, num_layers), TT_OFF(tt_denoise_step_args, hidden),
      TT_OFF(tt_denoise_step_args, vocab), TT_OFF(tt_denoise_step_args, reserved0),
      TT_OFF(tt_denoise_step_args, attn), TT_OFF(tt_denoise_step_args, k_pages),
      TT_OFF(tt_denoise_step_args, v_pages), TT_OFF(tt_denoise_step_args, w_qkv),
      TT_OFF(tt_denoise_step_args, w_o), TT_OFF(tt_denoise_step_args, k_blk),
      TT_OFF(tt_denoise_step_args, v_blk), TT_OFF(tt_denoise_step_args, w_lm),
      TT_OFF(tt_denoise_step_args, h_in), TT_OFF(tt_denoise_step_args, h_work),
      TT_OFF(tt_denoise_step_args, q), TT_OFF(tt_denoise_step_args, attn_out),
      TT_OFF(tt_denoise_step_args, logits), TT_OFF(tt_denoise_step_args, logits_ld),
      TT_OFF(tt_denoise_step_args, unmask), TT_OFF(tt_denoise_step_args, timing_events)};
  static const int64_t lmu[] = {TT_OFF(tt_lm_head_unmask_args, lm),
                                TT_OFF(tt_lm_head_unmask_args, unmask)};
  static const int64_t app[] = {
      TT_OFF(tt_kv_append_args, num_layers), TT_OFF(tt_kv_append_args, batch),
      TT_OFF(tt_kv_append_args, num_kv_heads), TT_OFF(tt_kv_append_args, head_dim),
      TT_OFF(tt_kv_append_args, S), TT_OFF(tt_kv_append_args, dtype),
      TT_OFF(tt_kv_append_args, num_pages), TT_OFF(tt_kv_append_args, page_size),
      TT_OFF(tt_kv_append_args, max_pages_per_seq), TT_OFF(tt_kv_append_args, reserved0),
      TT_OFF(tt_kv_append_args, k_pages), TT_OFF(tt_kv_append_args, v_pages),
      TT_OFF(tt_kv_append_args, k_new), TT_OFF(tt_kv_append_args, v_new),
      TT_OFF(tt_kv_append_args, block_table), TT_OFF(tt_kv_append_args, ctx_lens),
      TT_OFF(tt_kv_append_args, free_pages), TT_OFF(tt_kv_append_args, free_count),
      TT_OFF(tt_kv_append_args, status)};
  static const int64_t cor[] = {
      TT_OFF(tt_mask_corrupt_args, batch), TT_OFF(tt_mask_corrupt_args, S),
      TT_OFF(tt_mask_corrupt_args, mask_id), TT_OFF(tt_mask_corrupt_args, reserved0),
      TT_OFF(tt_mask_corrupt_args, clean), TT_OFF(tt_mask_corrupt_args, u_time),
      TT_OFF(tt_mask_corrupt_args, u_mask), TT_OFF(tt_mask_corrupt_args, noisy),
      TT_OFF(tt_mask_corrupt_args, masked), TT_OFF(tt_mask_corrupt_args, t_out)};
  static const int64_t nll[] = {
      TT_OFF(tt_masked_nll_args, batch), TT_OFF(tt_masked_nll_args, S),
      TT_OFF(tt_masked_nll_args, vocab), TT_OFF(tt_masked_nll_args, reserved0),
      TT_OFF(tt_masked_nll_args, ld), TT_OFF(tt_masked_nll_args, logits),
      TT_OFF(tt_masked_nll_args, targets), TT_OFF(tt_masked_nll_args, masked),
      TT_OFF(tt_masked_nll_args, nll), TT_OFF(tt_masked_nll_args, loss),
      TT_OFF(tt_masked_nll_args, n_masked)};
  const int64_t *tab = nullptr;
  int n = 0;
  switch (which) {
    case 0: tab = attn; n = sizeof(attn) / sizeof(attn[0]); break;
    case 1: tab = unm; n = sizeof(unm) / sizeof(unm[0]); break;
    case 2: tab = qkv; n = sizeof(qkv) / sizeof(qkv[0]); break;
    case 3: tab = outp; n = sizeof(outp) / sizeof(outp[0]); break;
    case 4: tab = lm; n = sizeof(lm) / sizeof(lm[0]); break;
    case 5: tab = step; n = sizeof(step) / sizeof(step[0]); break;
    case 6: tab = lmu; n = sizeof(lmu) / sizeof(lmu[0]); break;
    case 7: tab = app; n = sizeof(app) / sizeof(app[0]); break;
    case 8: tab = cor; n = sizeof(cor) / sizeof(cor[0]); break;
    case 9: tab = nll; n = sizeof(nll) / sizeof(nll[0]); break;
    default: return -1;
  }
  if (field < 0 || field >= n) return -1;
  return tab[field];
}
#undef TT_OFF

}  // extern "C"
