/*
 * twotower.h -- C ABI of the block-diffusion denoise-step library for AMD MI355X (gfx950).
 *
 * The library computes the hot path of TwoTower block-wise autoregressive diffusion decoding:
 * one denoise step of the trainable denoiser tower, in which the S positions of the current
 * block attend, under one softmax, to the frozen context tower's KV cache of the same layer and
 * to the block's own bidirectional KV, followed by confidence unmasking of the block logits.
 * Sources: "Nemotron-TwoTower: Diffusion Language Modeling with Pretrained Autoregressive
 * Context" explainer (gist.science), sections "Architektur", "Generierungsprozess" and
 * "Training und Konditionierung"; "NVIDIA loest den zentralen Kompromiss moderner LLMs"
 * (gotburnout.io), section "2. Denoiser Tower"; dgnews.ru report on Nemotron-Labs-TwoTower,
 * architecture and test-results sections.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers unless a field says "host". Arrays of pointers in
 *   tt_denoise_step_args are host arrays holding device pointers.
 * - The caller owns every buffer. The library never allocates or frees device memory and keeps
 *   no pointer after returning. Buffers must stay alive until the stream work completes.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream). No call
 *   synchronizes with the host.
 * - Workspace protocol: a call with ws == NULL is always a size query: it sets *ws_bytes to the
 *   required size, launches nothing and returns TT_OK. To run, call with a non-NULL ws pointing
 *   to at least that many bytes of device memory (256-byte aligned), passing its size in
 *   *ws_bytes; when the required size is 0 any non-NULL ws is accepted and never dereferenced.
 *   A smaller *ws_bytes returns TT_ENOSPACE and sets *ws_bytes to the required size. The
 *   workspace content on entry does not matter.
 * - Errors are return codes only; the library never prints or aborts. Every argument check runs
 *   on the host before anything is launched, so an error leaves all outputs untouched.
 *   TT_EHIP means a HIP launch failed; asynchronous device faults surface at the caller's next
 *   synchronization.
 * - Results are deterministic: fixed reduction order, no floating-point atomics.
 * - An empty batch (batch = 0; rows = 0 for the row-wise products) is a valid call: the sizes are
 *   still checked, no workspace is needed, nothing is launched (timing events included) and the
 *   call returns TT_OK. Its device pointers may then be NULL (as PyTorch gives for empty
 *   tensors); host arrays, such as the step's per-layer pointer arrays, must still be given.
 *   Outputs that do not scale with the batch (twotower_masked_nll's loss and n_masked,
 *   twotower_kv_append's free_count and status) are left as they are.
 * - Calls that share a workspace must be ordered on one stream.
 */
#ifndef TWOTOWER_H
#define TWOTOWER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TWOTOWER_ABI_VERSION 9

typedef enum {
  TT_OK = 0,
  TT_EINVAL = 1,   /* invalid argument: null/misaligned pointer, negative or inconsistent size */
  TT_ENOTSUP = 2,  /* valid but unsupported shape or dtype combination */
  TT_ENOSPACE = 3, /* workspace too small; *ws_bytes holds the required size */
  TT_EHIP = 4      /* a HIP runtime call or kernel launch failed */
} tt_status;

typedef enum { TT_FP32 = 0, TT_BF16 = 1 } tt_dtype;

/*
 * Block attention of the denoiser at one layer (twotower_block_attn).
 *
 * Definition (explainer, "Architektur" / "Generierungsprozess"; gotburnout.io, "2. Denoiser
 * Tower"): for every sequence b, query head h, block position i, with KV head
 * g = h / (num_q_heads / num_kv_heads), the keys are the context rows 0..ctx_lens[b]-1 of KV head
 * g followed by the S block rows of KV head g, and
 *     s_j = scale * <q[b,i,h,:], key_j>,  m = max_j s_j,  w_j = exp(s_j - m),
 *     out[b,i,h,:] = sum_j w_j value_j / sum_j w_j,   lse[b,h,i] = m + ln(sum_j w_j).
 * No mask: the context holds only tokens before the block (causal across blocks); inside the
 * block every query sees every block key, its own position included.
 *
 * Layouts (elements of `dtype`, innermost last, all contiguous):
 *   q        [batch, S, num_q_heads, head_dim]
 *   k_pages  [num_pages, num_kv_heads, page_size/64, head_dim/8, 64, 8]   64-token tiles of
 *            8-element chunks, chunk-major: element (row o of the page, dimension d) is at
 *            [page, g, o / 64, d / 8, o % 64, d % 8]
 *   v_pages  [num_pages, num_kv_heads, page_size/64, 8, head_dim, 8]        64-token tiles of
 *            8-token chunks: element (o, d) is at [page, g, o / 64, (o % 64) / 8, d, o % 8]
 *            (a tile of either is contiguous: head_dim * 64 elements; the 32 lanes of a matrix
 *            operand read 32 consecutive 16-byte chunks of it)
 *   block_table [batch, max_pages_per_seq] int32: context row t of sequence b is in page
 *            block_table[b, t / page_size] at offset t % page_size
 *   ctx_lens [batch] int32, 0 <= ctx_lens[b] <= max_ctx_len
 *   k_blk    [batch, num_kv_heads, S, head_dim]
 *   v_blk    [batch, num_kv_heads, head_dim, S]                 dim-major
 *   out      [batch, S, num_q_heads, head_dim] in `out_dtype`
 *   lse      [batch, num_q_heads, S] fp32, natural log; optional (NULL = not written)
 * A contiguous cache is the case page_size >= max_ctx_len, block_table[b] = {b}.
 *
 * Supported: dtype TT_BF16 (bf16 MFMA, fp32 softmax and accumulation, probabilities rounded to
 * bf16 for the PV product) or TT_FP32 (fp32 throughout); out_dtype TT_FP32, or equal to dtype.
 * head_dim in {64, 128}; 1 <= S <= 256; num_q_heads % num_kv_heads == 0; page_size a positive
 * multiple of 64; max_ctx_len <= max_pages_per_seq * page_size. Pointers 16-byte aligned.
 * Unsupported shapes return TT_ENOTSUP.
 *
 * Device-side checks: a sequence whose ctx_lens[b] lies outside [0, max_ctx_len], or whose
 * needed block_table entries lie outside [0, num_pages), gets NaN in all its outputs (nothing out
 * of bounds is read). Page slots past ctx_lens[b] are never used, so they may hold anything.
 *
 * num_splits: number of context partitions per (sequence, KV head) at max_ctx_len; 0 = chosen
 * by the library: for up to 256 sequences the partitions are sized on the device from the actual
 * lengths, nearly equal across the whole batch and about one per compute unit (sequence b's
 * ceil(ctx_lens[b] / 64) tiles in nearly equal parts of at most c tiles, c the smallest size that
 * keeps the total near the GPU's compute units), so ragged batches keep every compute unit busy.
 * Partitions are merged exactly with their log-sum-exp weights; the result depends on the
 * partitioning only through floating-point rounding.
 *
 * Value range: any finite inputs. With several partitions each partition's normalized output row
 * is kept in the workspace as fp16 scaled by a power of two chosen per row (its largest magnitude
 * in [2^14, 2^15)), so no bf16 value overflows and rows of small values keep fp16's relative
 * precision (2^-11); the bf16 path's error is relative to max|V| (P is rounded to bf16 once,
 * relative 2^-8; the fp16 partial adds 2^-12 of the row's largest magnitude).
 *
 * timing_events: optional host array of 3 hipEvent_t (NULL in normal use): events[0] and
 * events[1] are recorded on `stream` immediately before and after the main attention kernel,
 * events[2] after the partition merge (equal in time to events[1] when there is one partition).
 * A NULL entry is not recorded. A profiling hook; the events must have been created by the
 * caller, preferably with hipEventDisableSystemFence (a default event's record writes back and
 * invalidates the caches between the kernels it separates, which lengthens the timed interval).
 */
typedef struct {
  int32_t batch, S, num_q_heads, num_kv_heads, head_dim;
  int32_t dtype;       /* tt_dtype of q, k_pages, v_pages, k_blk, v_blk */
  int32_t out_dtype;   /* tt_dtype of out */
  float scale;         /* softmax scale, e.g. 1/sqrt(head_dim) */
  const void *q;
  const void *k_pages;
  const void *v_pages;
  int32_t num_pages, page_size, max_pages_per_seq, max_ctx_len;
  const int32_t *block_table;
  const int32_t *ctx_lens;
  const void *k_blk;
  const void *v_blk;
  void *out;
  float *lse;
  int32_t num_splits;
  int32_t reserved0;
  void *const *timing_events;  /* host array [3] of hipEvent_t, optional */
} tt_block_attn_args;

/*
 * Confidence unmasking of one step (twotower_unmask).
 *
 * Definition (explainer, "Training und Konditionierung", sampling paragraph; dgnews.ru,
 * test-results section): every still-masked position is predicted in parallel; positions whose
 * confidence is above `threshold` are committed, the others stay masked. For each b and each i
 * with masked[b,i] != 0: token = the lowest index of the row maximum of logits[b,i,:],
 * confidence = 1 / sum_j exp(logits[b,i,j] - max) (the largest softmax probability), computed in
 * fp32. Position i is committed iff confidence > threshold (strict). If min_commit != 0 and no
 * masked position of sequence b is committed, the masked position with the largest confidence is
 * committed (lowest i on ties). If commit_all != 0 every masked position is committed.
 * Committing sets tokens[b,i] = token and masked[b,i] = 0. Positions with masked[b,i] == 0 are
 * neither read nor written (their logits rows are never loaded).
 *
 * Layouts: logits fp32, row (b, i) starts at element (b*S + i) * ld, vocab contiguous elements;
 *   masked uint8 [batch, S] (in/out); tokens int32 [batch, S] (in/out);
 *   confidence fp32 [batch, S] (optional out, written for positions masked on entry);
 *   n_committed int32 [batch] (optional out).
 * Supported: 1 <= S <= 256, 1 <= vocab < 2^31, ld >= vocab. Logits must be finite.
 */
typedef struct {
  int32_t batch, S, vocab;
  int32_t reserved0;
  int64_t ld;
  const float *logits;
  uint8_t *masked;
  int32_t *tokens;
  float *confidence;
  int32_t *n_committed;
  float threshold;
  int32_t min_commit;
  int32_t commit_all;
  int32_t reserved1;
} tt_unmask_args;

/*
 * Masked-diffusion training objective (twotower_mask_corrupt, twotower_masked_nll). The denoiser
 * is trained on clean blocks corrupted by replacing tokens with [MASK] on a linear schedule and
 * minimizes the negative log-likelihood of the original tokens at the masked positions
 * (explainer, "Training und Konditionierung", masked-diffusion paragraph). Training itself is not
 * part of this library; these are its two per-block kernels.
 *
 * twotower_mask_corrupt: sequence b takes the diffusion time t = u_time[b] (uniform draws in
 *   [0, 1), supplied by the caller) and masks position i iff u_mask[b, i] < t (probability t:
 *   the linear schedule); noisy[b, i] = masked ? mask_id : clean[b, i]; masked[b, i] = 0 / 1;
 *   t_out[b] = t (optional, NULL to skip). Needs no workspace (the size query returns 0).
 * twotower_masked_nll: for each row (b, i) with masked[b, i] != 0,
 *     nll[b, i] = ln(sum_j exp(logits[b, i, j])) - logits[b, i, targets[b, i]]
 *   computed in fp32 (NaN if the target is outside 0 .. vocab-1); nll = 0 at the other rows.
 *   loss[0] = mean of nll over the masked rows of the whole batch (0 if there are none) and
 *   n_masked[0] = their number, both optional. Logits layout as for twotower_unmask (fp32, row
 *   (b*S + i) at element (b*S + i) * ld); batch * S <= 65535.
 */
typedef struct {
  int32_t batch, S, mask_id;
  int32_t reserved0;
  const int32_t *clean;      /* [batch, S] */
  const float *u_time;       /* [batch] */
  const float *u_mask;       /* [batch, S] */
  int32_t *noisy;            /* [batch, S] out */
  uint8_t *masked;           /* [batch, S] out */
  float *t_out;              /* [batch] out, optional */
} tt_mask_corrupt_args;

typedef struct {
  int32_t batch, S, vocab;
  int32_t reserved0;
  int64_t ld;
  const float *logits;
  const int32_t *targets;    /* [batch, S] clean tokens */
  const uint8_t *masked;     /* [batch, S] */
  float *nll;                /* [batch, S] out */
  float *loss;               /* [1] out, optional */
  int32_t *n_masked;         /* [1] out, optional */
} tt_masked_nll_args;

/*
 * Dense projections of the synthetic attention-only denoiser (twotower_qkv_projection,
 * twotower_out_projection, twotower_lm_head). The pages give no layer shapes; the model is a
 * residual stream H [rows = batch*S, hidden] (bf16) with, per attention layer,
 *   [Q | K_blk | V_blk] = H W_qkv^T,  W_qkv bf16 [(Hq + 2*Hkv)*head_dim, hidden]
 *   H <- H + O W_o^T,                  W_o   bf16 [hidden, Hq*head_dim]
 * and logits = H W_lm^T,               W_lm  bf16 [vocab, hidden], fp32 logits [rows, vocab].
 * Weights W [out_features, in_features] (row-major bf16) are passed in the packed form written by
 * twotower_pack_weight (once, when the weights are loaded). The block's own KV is rewritten every
 * step because the block changes (explainer, "Generierungsprozess").
 * Products accumulate in fp32 and are rounded once to the output type. When the output features
 * alone give too few work-groups to fill the GPU, the input features are split into partitions
 * whose fp32 partial products are summed in partition order (a fixed order: deterministic). The
 * sum runs inside the product's kernel when all of its work-groups can be resident on the GPU at
 * once and K has at most 16 partitions: the partitions of an output tile meet at an arrival
 * counter in the workspace (a 64-bit word tagged with the launch, so any prior workspace content is
 * accepted and nothing needs clearing; graph replays of one captured call find and restart the
 * previous replay's count), and each then sums an equal share of the tile's rows. A partition that
 * has waited about 0.4 ms for the others (they cannot all be resident, e.g. while another kernel
 * holds compute units) hands its share to the last one to arrive and leaves, so no partition
 * waits for one that cannot run; the environment variable TWOTOWER_MERGE_WAIT_POLLS (read at every
 * call, default 256 polls of about 1.5 us) sets that wait. Otherwise, or with
 * TWOTOWER_MERGE_IN_KERNEL=0 in the environment (read at every call), a second kernel sums the
 * partials. Every way gives the same result, bit for bit.
 *
 * Packed weight layout (the A-operand order of the 32x32x16 bf16 matrix instruction): W is cut
 * into slabs of 32 output features (nb < NS = ceil(out_features / 32)) and K steps of 16 inputs
 * (s < Ks = ceil(in_features / 16)); a (slab, step) block is one 1 KB unit, and the slabs are
 * grouped by 8 (group gi = nb / 8 holds gsize = min(8, NS - 8 gi) slabs) with the units of a group
 * ordered step-major, so that the 64 inputs of 8 slabs are one contiguous 32 KB run:
 *   unit U = 8 * gi * Ks + s * gsize + nb % 8,
 * and the bf16 element at (U * 64 + lane) * 8 + e (lane < 64, e < 8) is
 * W[nb * 32 + lane % 32][s * 16 + (lane / 32) * 8 + e], 0 where that is outside W.
 * Size: twotower_packed_weight_bytes(out_features, in_features) bytes (NS * Ks KB).
 */
typedef struct {
  int32_t batch, S, hidden, num_q_heads, num_kv_heads, head_dim;
  const void *h;        /* bf16 [batch, S, hidden] */
  const void *w_qkv;    /* packed bf16 [(Hq + 2*Hkv)*head_dim, hidden] */
  void *q;              /* bf16 [batch, S, Hq, head_dim] */
  void *k_blk;          /* bf16 [batch, Hkv, S, head_dim] */
  void *v_blk;          /* bf16 [batch, Hkv, head_dim, S] */
} tt_qkv_args;

typedef struct {
  int32_t rows, hidden, in_features;
  int32_t reserved0;
  const void *h_in;     /* bf16 [rows, hidden] residual input (may equal h_out) */
  const void *o;        /* bf16 [rows, in_features] attention output */
  const void *w_o;      /* packed bf16 [hidden, in_features] */
  void *h_out;          /* bf16 [rows, hidden] = h_in + o W_o^T */
} tt_out_proj_args;

typedef struct {
  int32_t rows, hidden, vocab;
  int32_t reserved0;
  int64_t ld;           /* row stride of logits in elements, >= vocab, multiple of 4 */
  const void *h;        /* bf16 [rows, hidden] */
  const void *w_lm;     /* packed bf16 [vocab, hidden] */
  float *logits;        /* fp32 [rows, ld] */
} tt_lm_head_args;

/*
 * lm-head fused with the unmasking (twotower_lm_head_unmask). The operation is the one of the
 * two calls it replaces (explainer, "Training und Konditionierung", sampling paragraph: all masked
 * positions are predicted at once and the confident ones committed): the same results as
 * twotower_lm_head followed by twotower_unmask on its logits, without the logits round trip
 * through memory. Every 256-logit tile of a row is reduced to (max, first argmax, sum of
 * exp(logit - max)) inside the product and the unmasking merges those partials, so the
 * confidences agree with the two-call path up to fp32 rounding of the sum (its order differs) and
 * the committed tokens are the same wherever no confidence ties with the threshold or with
 * another position within that rounding.
 *   lm:     rows must equal unmask.batch * unmask.S. lm.logits may be NULL: the logits are then
 *           not stored and lm.ld is ignored; otherwise they are stored as by twotower_lm_head.
 *   unmask: masked, tokens, confidence, n_committed, threshold, min_commit, commit_all as for
 *           twotower_unmask; its vocab, ld and logits fields are ignored (taken from lm).
 * Rows with masked == 0 still go through the product (their tiles share the weight stream) but
 * produce no partials and are not touched by the unmasking.
 */
typedef struct {
  tt_lm_head_args lm;
  tt_unmask_args unmask;
} tt_lm_head_unmask_args;

/*
 * One denoise step of the synthetic denoiser (twotower_denoise_step): for each layer l,
 * twotower_qkv_projection (rewrites k_blk[l], v_blk[l]) -> twotower_block_attn over
 * (k_pages[l], v_pages[l]) and the block KV of layer l (layer-aligned: denoiser layer l reads the
 * context tower's layer l, gotburnout.io "2. Denoiser Tower") -> twotower_out_projection; then
 * twotower_lm_head_unmask. Layer 0 reads h_in; the residual stream is kept in h_work.
 * All layers share batch, S, heads, head_dim, block_table, ctx_lens and page geometry (taken from
 * `attn`; attn.q/k_pages/v_pages/k_blk/v_blk/out/lse/timing_events are ignored). The context
 * caches are only read. A sequence with no masked position left gets no attention work (with the
 * automatic partition count its context is left out of the partition plan, so the live
 * sequences' contexts spread over the whole GPU, and its attn_out rows are not written); the
 * row-wise projections still run over its rows (their weights are streamed for the live rows
 * anyway) and their results are discarded by the unmasking, which reads no committed row.
 *
 * timing_events: optional host array of 3*num_layers hipEvent_t; if not NULL, events[3l] and
 * events[3l+1] are recorded on `stream` immediately before and after the main attention kernel
 * of layer l and events[3l+2] after its partition merge; NULL entries are skipped (profiling
 * hook, NULL in normal use; see tt_block_attn_args for the event flags).
 */
typedef struct {
  int32_t num_layers, hidden, vocab;
  int32_t reserved0;
  tt_block_attn_args attn;
  const void *const *k_pages;   /* host array [num_layers] of device pointers */
  const void *const *v_pages;
  const void *const *w_qkv;     /* packed weights (see the projections) */
  const void *const *w_o;
  void *const *k_blk;           /* host array [num_layers]: block KV, rewritten every step */
  void *const *v_blk;
  const void *w_lm;             /* packed */
  const void *h_in;             /* bf16 [batch, S, hidden], read only */
  void *h_work;                 /* bf16 [batch, S, hidden], residual stream after the step */
  void *q;                      /* bf16 [batch, S, Hq, head_dim] scratch */
  void *attn_out;               /* bf16 [batch, S, Hq, head_dim] scratch */
  float *logits;                /* fp32 [batch, S, logits_ld], optional (NULL: not stored) */
  int64_t logits_ld;
  tt_unmask_args unmask;        /* masked/tokens/confidence/n_committed/threshold/flags used;
                                   batch/S/vocab/ld/logits are taken from the step */
  void *const *timing_events;
} tt_denoise_step_args;

/*
 * Context KV append after a block is committed (twotower_kv_append). Once every position of the
 * block is committed, the frozen context tower encodes it and its keys and values join the cache
 * that the next block attends to (explainer, "Generierungsprozess"); this call does the cache side
 * of that: it writes, for every layer, the block's S rows at context positions ctx_lens[b] ..
 * ctx_lens[b] + S - 1 of sequence b and advances ctx_lens[b] by S. (The rows themselves come from
 * the context tower, which this library does not include: any [batch, Hkv, S, head_dim] keys and
 * [batch, Hkv, head_dim, S] values are accepted, e.g. the block KV of the last denoise step.)
 *
 * Pages: the rows go to the pages already in the sequence's block table while they have room;
 * each further page is popped from the top of a device-resident free-page stack
 * (free_pages[*free_count - 1], then free_pages[*free_count - 2], ...) and written into the next
 * block-table entry. Sequences are served in order b = 0, 1, ..., so the assignment is
 * deterministic. A sequence whose rows do not fit (ctx_lens[b] outside 0 .. max_pages_per_seq *
 * page_size - S, too few free pages left, or a page id it would write outside 0 .. num_pages-1)
 * is skipped: its table, length and cache rows stay untouched and *status gets
 * TT_APPEND_NO_ROOM_IN_TABLE, TT_APPEND_OUT_OF_PAGES or TT_APPEND_BAD_PAGE OR-ed in (*status
 * is never cleared by the library). Everything happens on the device; the host is not
 * synchronized.
 *
 * Layouts: k_pages / v_pages per layer as in tt_block_attn_args (page_size a multiple of 64);
 *   k_new[l] [batch, num_kv_heads, S, head_dim], v_new[l] [batch, num_kv_heads, head_dim, S]
 *   (elements of `dtype`); block_table int32 [batch, max_pages_per_seq] (in/out);
 *   ctx_lens int32 [batch] (in/out); free_pages int32 [any], free_count int32 [1] (in/out),
 *   status int32 [1] (in/out). Supported: 1 <= num_layers <= 16.
 */
#define TT_APPEND_OUT_OF_PAGES 1
#define TT_APPEND_NO_ROOM_IN_TABLE 2
#define TT_APPEND_BAD_PAGE 4
typedef struct {
  int32_t num_layers, batch, num_kv_heads, head_dim, S;
  int32_t dtype;                 /* tt_dtype of the caches and the new rows */
  int32_t num_pages, page_size, max_pages_per_seq;
  int32_t reserved0;
  void *const *k_pages;          /* host array [num_layers] of device pointers */
  void *const *v_pages;
  const void *const *k_new;      /* host array [num_layers] */
  const void *const *v_new;
  int32_t *block_table;
  int32_t *ctx_lens;
  const int32_t *free_pages;
  int32_t *free_count;
  int32_t *status;
} tt_kv_append_args;

tt_status twotower_block_attn(const tt_block_attn_args *args, void *ws, size_t *ws_bytes,
                              void *stream);

/*
 * twotower_block_attn without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, kernels and arguments as twotower_block_attn, with the split-KV partials kept in a
 * scratch array of TWOTOWER_STATIC_SCRATCH_BYTES that the library holds per device (in its code
 * object, from the first call on a device until the process ends). Nothing is allocated or freed.
 * num_splits == 0: the library's partition count, lowered if needed until the partials fit the
 * scratch; an explicit num_splits whose partials do not fit returns TT_ENOSPACE (nothing is
 * launched). Every call on one device shares that device's scratch: calls that may overlap on one
 * device (different streams, or host threads without ordering) race and give wrong results;
 * order them on one stream. The scratch needs no initial content (every value read is written
 * first by the same call). TT_EHIP if the scratch's device address cannot be obtained.
 */
#define TWOTOWER_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
tt_status twotower_block_attn_static(const tt_block_attn_args *args, void *stream);
tt_status twotower_kv_append(const tt_kv_append_args *args, void *ws, size_t *ws_bytes,
                             void *stream);
tt_status twotower_mask_corrupt(const tt_mask_corrupt_args *args, void *ws, size_t *ws_bytes,
                                void *stream);
tt_status twotower_masked_nll(const tt_masked_nll_args *args, void *ws, size_t *ws_bytes,
                              void *stream);
tt_status twotower_unmask(const tt_unmask_args *args, void *ws, size_t *ws_bytes, void *stream);
tt_status twotower_qkv_projection(const tt_qkv_args *args, void *ws, size_t *ws_bytes,
                                  void *stream);
tt_status twotower_out_projection(const tt_out_proj_args *args, void *ws, size_t *ws_bytes,
                                  void *stream);
tt_status twotower_lm_head(const tt_lm_head_args *args, void *ws, size_t *ws_bytes, void *stream);
tt_status twotower_lm_head_unmask(const tt_lm_head_unmask_args *args, void *ws, size_t *ws_bytes,
                                  void *stream);
tt_status twotower_denoise_step(const tt_denoise_step_args *args, void *ws, size_t *ws_bytes,
                                void *stream);

/* Bytes of the packed form of a weight [out_features, in_features] (layout above):
 * ceil(out_features / 32) * ceil(in_features / 16) * 1024; 0 for a non-positive size. */
size_t twotower_packed_weight_bytes(int32_t out_features, int32_t in_features);
/* Writes the packed form of the row-major bf16 weight w into `packed` (device memory of
 * twotower_packed_weight_bytes bytes, owned by the caller), enqueued on `stream`. Both pointers
 * 16-byte aligned and in_features % 8 == 0 (else TT_EINVAL / TT_ENOTSUP); no workspace. */
tt_status twotower_pack_weight(const void *w, int32_t out_features, int32_t in_features,
                               void *packed, void *stream);

/*
 * Measurement probe (not part of the method): reads `bytes` of device memory at `src` with
 * 16-byte non-temporal loads, `workgroups` work-groups of 256 threads in a grid-stride loop, the
 * practical streaming-read ceiling that the bandwidth-bound kernels are reported against next to
 * the nominal HBM peak. `sink` (device, `workgroups` uint32 words) is written only in the
 * practically never taken case that a work-group's XOR of the data equals 0x9E3779B9, so the
 * probe normally writes nothing. bytes a positive multiple of 16, src 16-byte aligned,
 * 1 <= workgroups <= 65536 (else TT_EINVAL).
 */
tt_status twotower_probe_stream_read(const void *src, size_t bytes, int32_t workgroups,
                                     uint32_t *sink, void *stream);

/*
 * Measurement probe: the issue rate of 32x32x16 bf16 MFMAs (v_mfma_f32_32x32x16_bf16, 32768 flops
 * each) on gfx950, the compute-side ceiling next to the nominal dense bf16 peak. `workgroups`
 * work-groups of 8 waves each run `iters` iterations of 16 MFMAs on four independent accumulators
 * (flops per call = workgroups * 8 * iters * 16 * 32768). mode bit 0: the A operand of every MFMA
 * is a 1 KB LDS read issued one iteration ahead (the attention's operand traffic); bit 1: two
 * work-groups share a compute unit (4 waves per SIMD) instead of one (2 waves per SIMD), so
 * workgroups = 2 * (or 1 *) the compute-unit count fills the GPU. sink: device float array of
 * workgroups * 512 entries, overwritten (values have no meaning). 0 <= mode <= 3,
 * 1 <= workgroups <= 65536, 1 <= iters <= 2^20, else TT_EINVAL.
 */
tt_status twotower_probe_mfma_rate(int32_t mode, int32_t workgroups, int32_t iters, float *sink,
                                   void *stream);

/* Static string for a status code ("TT_OK", ...); never NULL. */
const char *twotower_status_string(int32_t status);
/* TWOTOWER_ABI_VERSION of the built library. */
int32_t twotower_abi_version(void);
/* sizeof of the argument structs, for bindings to check their mirrors:
 * 0 tt_block_attn_args, 1 tt_unmask_args, 2 tt_qkv_args, 3 tt_out_proj_args,
 * 4 tt_lm_head_args, 5 tt_denoise_step_args, 6 tt_lm_head_unmask_args,
 * 7 tt_kv_append_args, 8 tt_mask_corrupt_args, 9 tt_masked_nll_args; -1 for an unknown
 * index. */
int64_t twotower_struct_size(int32_t which);
/* Byte offset of field `field` (0-based declaration order) in struct `which`; -1 if unknown. */
int64_t twotower_struct_offset(int32_t which, int32_t field);

#ifdef __cplusplus
}
#endif
#endif /* TWOTOWER_H */
