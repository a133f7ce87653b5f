// Confidence unmasking for gfx950 ("Nemotron-TwoTower" explainer, section "Training und
// Konditionierung", sampling paragraph: every masked position is predicted in parallel, the ones
// whose confidence is above the threshold are committed, the rest stay masked).
//
// unmask_partial_kernel: one work-group per (masked row, 8192-element vocabulary chunk). Each
//   thread reads 32 logits with coalesced 16-byte loads, keeps (max, first argmax, sum of
//   exp(x - max)) and the triples are merged across the wavefront with lane shuffles and across
//   the four wavefronts through LDS. Committed rows exit before reading anything.
// unmask_finalize_kernel: one wavefront per sequence, lane i = block position i. Merges the
//   chunk triples of its row, confidence = 1 / sum, threshold / fallback / commit-all decisions
//   with wavefront ballots, then updates tokens, masked, confidence and n_committed.
// unmask_tiles_finalize_kernel: the same decisions from the per-256-logit triples that the fused
//   lm-head epilogue writes (hundreds per row), merged by one wavefront per row.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "triple.hpp"

namespace tt {

constexpr int kUThreads = 256;
constexpr int kUPerThread = 32;
constexpr int kUChunk = kUThreads * kUPerThread;  // 8192 logits per work-group

template <bool VEC>
__global__ __launch_bounds__(kUThreads) void unmask_partial_kernel(UnmaskParams p) {
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  if (!p.masked[row]) return;
  const int tid = threadIdx.x;
  const int base = chunk * kUChunk;
  const int n = min(kUChunk, p.vocab - base);
  const float *x = p.logits + (size_t)row * p.ld + base;
  float v[kUPerThread];
  int first[kUPerThread / 4];
  if (VEC) {
#pragma unroll
    for (int k = 0; k < kUPerThread / 4; ++k) {
      const int e = (k * kUThreads + tid) * 4;
      first[k] = e;
      if (e + 3 < n) {
        const f32x4 q = *reinterpret_cast<const f32x4 *>(x + e);
        v[4 * k] = q[0]; v[4 * k + 1] = q[1]; v[4 * k + 2] = q[2]; v[4 * k + 3] = q[3];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * k + j] = e + j < n ? x[e + j] : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kUPerThread / 4; ++k) {
      const int e = (k * kUThreads + tid) * 4;
      first[k] = e;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * k + j] = e + j < n ? x[e + j] : -INFINITY;
    }
  }
  // Elements are visited in increasing index order, so a strict '>' keeps the first maximum.
  Triple t = empty_triple();
#pragma unroll
  for (int k = 0; k < kUPerThread / 4; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (v[4 * k + j] > t.m) {
        t.m = v[4 * k + j];
        t.idx = base + first[k] + j;
      }
  float z = 0.f;
  if (t.m > -INFINITY) {
#pragma unroll
    for (int k = 0; k < kUPerThread; ++k) z += __expf(v[k] - t.m);
  }
  t.z = z;
  for (int o = 1; o < 64; o <<= 1) t = merge(t, shfl_xor_triple(t, o));
  __shared__ Triple red[kUThreads / 64];
  if ((tid & 63) == 0) red[tid >> 6] = t;
  __syncthreads();
  if (tid == 0) {
    Triple r = red[0];
    for (int w = 1; w < kUThreads / 64; ++w) r = merge(r, red[w]);
    float *o = p.part + ((size_t)row * p.chunks + chunk) * 4;
    o[0] = r.m;
    o[1] = __int_as_float(r.idx);
    o[2] = r.z;
  }
}

// Decisions of sequence b from the row triples, thread i of the work-group = block position i
// (every thread of the work-group calls it; positions are i < S <= kDecThreads): confidence = 1 / z,
// commit iff confidence > threshold (or commit-all), the one-commit fallback (largest
// confidence, lowest position on ties) through per-wave reductions in LDS, then the state update.
constexpr int kDecThreads = 256;  // largest block size S

// `flag` is masked[b, i] as read at kernel start (0 for i >= S).
__device__ __forceinline__ void commit_decisions(const UnmaskParams &p, int b, int i, Triple t,
                                                 uint32_t flag) {
  __shared__ int any_commit_w[kDecThreads / 64], any_masked_w[kDecThreads / 64];
  __shared__ float best_c[kDecThreads / 64];
  __shared__ int best_i[kDecThreads / 64], n_w[kDecThreads / 64];
  const int lane = i & 63, w = i >> 6;
  const size_t row = (size_t)b * p.S + i;
  const bool was_masked = flag != 0;
  const float conf = was_masked ? 1.0f / t.z : -1.0f;
  bool commit = was_masked && (p.commit_all || conf > p.threshold);
  // the wave's best candidate for the fallback: largest confidence, lowest position on ties
  float bc = conf;
  int bi = was_masked ? i : 0x7fffffff;
  for (int o = 1; o < 64; o <<= 1) {
    const float oc = __shfl_xor(bc, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (oc > bc || (oc == bc && oi < bi)) {
      bc = oc;
      bi = oi;
    }
  }
  const bool wc = __ballot(commit) != 0, wm = __ballot(was_masked) != 0;  // whole wave
  if (lane == 0 && w < kDecThreads / 64) {
    any_commit_w[w] = wc;
    any_masked_w[w] = wm;
    best_c[w] = bc;
    best_i[w] = bi;
  }
  __syncthreads();
  bool any_commit = false, any_masked = false;
  float gc = -1.0f;
  int gi = 0x7fffffff;
  for (int k = 0; k < kDecThreads / 64; ++k) {  // in wave order: ties keep the lower position
    any_commit = any_commit || any_commit_w[k];
    any_masked = any_masked || any_masked_w[k];
    if (best_c[k] > gc || (best_c[k] == gc && best_i[k] < gi)) {
      gc = best_c[k];
      gi = best_i[k];
    }
  }
  if (!any_commit && p.min_commit && any_masked) commit = was_masked && i == gi;
  if (was_masked) {
    if (p.confidence) p.confidence[row] = conf;
    if (commit) {
      p.tokens[row] = t.idx;
      p.masked[row] = 0;
    }
  }
  const unsigned long long committed = __ballot(commit);
  if (lane == 0 && w < kDecThreads / 64) n_w[w] = __popcll(committed);
  __syncthreads();
  if (i == 0 && p.n_committed) {
    int n = 0;
    for (int k = 0; k < kDecThreads / 64; ++k) n += n_w[k];
    p.n_committed[b] = n;
  }
}

__device__ __forceinline__ Triple load_triple(const float *o) {
  Triple u;
  u.m = o[0];
  u.idx = __float_as_int(o[1]);
  u.z = o[2];
  return u;
}

// A few chunk triples per row (8192-logit chunks): thread i merges the triples of position i.
__global__ __launch_bounds__(kDecThreads) void unmask_finalize_kernel(UnmaskParams p) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const size_t row = (size_t)b * p.S + i;
  const uint32_t flag = i < p.S ? p.masked[row] : 0u;
  Triple t = empty_triple();
  if (flag != 0)
    for (int c = 0; c < p.chunks; ++c) t = merge(t, load_triple(p.part + (row * p.chunks + c) * 4));
  commit_decisions(p, b, i, t, flag);
}

// Many tile triples per row (one per 256-logit lm-head tile): wave w merges rows w, w + 16, ...
// with its 64 lanes (strided, then a butterfly), then threads 0 .. 255 take the decisions.
__global__ __launch_bounds__(1024) void unmask_tiles_finalize_kernel(UnmaskParams p) {
  __shared__ Triple rows[kDecThreads];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Thread i's flag for the decisions, requested together with the triples: a row that is no
  // longer masked has no triples of this step (what its slots hold is merged but never used), so
  // nothing waits for a flag before the triples are requested (one memory round trip).
  const uint32_t flag = threadIdx.x < (unsigned)p.S ? p.masked[(size_t)b * p.S + threadIdx.x] : 0u;
  for (int i = wave; i < p.S; i += 16) {
    const size_t row = (size_t)b * p.S + i;
    Triple t = empty_triple();
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.part) + row * p.chunks;
    for (int c0 = 0; c0 < p.chunks; c0 += 8 * 64) {  // 8 triples per lane in flight at once
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = c0 + j * 64 + lane;
        v[j] = c < p.chunks ? src[c] : f32x4{-INFINITY, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        Triple u;
        u.m = v[j][0];
        u.idx = __float_as_int(v[j][1]);
        u.z = v[j][2];
        t = merge(t, u);
      }
    }
    for (int o = 1; o < 64; o <<= 1) t = merge(t, shfl_xor_triple(t, o));
    if (lane == 0) rows[i] = t;
  }
  __syncthreads();
  const int i = threadIdx.x;
  commit_decisions(p, b, i, i < p.S ? rows[i] : empty_triple(), defer_use(flag));
}

// ------------------------------------------------------------------ masked-diffusion loss
// (explainer, "Training und Konditionierung", masked-diffusion paragraph: clean blocks are
// corrupted by replacing tokens with [MASK] on a linear schedule and the denoiser minimizes the
// negative log-likelihood of the original tokens at the masked positions.)

// Linear schedule: sequence b draws its time t = u_time[b] in [0, 1) and each position is masked
// independently with probability t, i.e. iff u_mask[b, i] < t (the uniform draws are inputs).
__global__ __launch_bounds__(256) void mask_corrupt_kernel(CorruptParams p) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= p.B * p.S) return;
  const int b = e / p.S;
  const float t = p.u_time[b];
  const bool m = p.u_mask[e] < t;
  p.noisy[e] = m ? p.mask_id : p.clean[e];
  p.masked[e] = m ? 1 : 0;
  if (p.t && e % p.S == 0) p.t[b] = t;
}

// NLL of the target token at every masked row, nll = ln(sum_j exp(x_j)) - x_target, from the
// rows' chunk triples (one thread per row, chunks merged in order), then the mean over the masked
// rows of the whole batch with a fixed-order reduction (wave butterflies, then the waves in order).
// A target outside the vocabulary gives NaN.
__global__ __launch_bounds__(1024) void nll_finalize_kernel(UnmaskParams p, NllParams q) {
  __shared__ float wsum[16];
  __shared__ int wcnt[16];
  const int rows = p.B * p.S;
  const int tid = threadIdx.x;
  float s = 0.f;
  int cnt = 0;
  for (int row = tid; row < rows; row += 1024) {
    float nll = 0.f;
    if (p.masked[row] != 0) {
      Triple t = empty_triple();
      for (int c = 0; c < p.chunks; ++c)
        t = merge(t, load_triple(p.part + ((size_t)row * p.chunks + c) * 4));
      const int tg = q.targets[row];
      const float x = (unsigned)tg < (unsigned)p.vocab ? p.logits[(size_t)row * p.ld + tg] : NAN;
      nll = (t.m - x) + logf(t.z);
      s += nll;
      cnt += 1;
    }
    q.nll[row] = nll;
  }
  s = wave_sum(s);
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if ((tid & 63) == 0) {
    wsum[tid >> 6] = s;
    wcnt[tid >> 6] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    int n = 0;
    for (int w = 0; w < 16; ++w) {
      tot += wsum[w];
      n += wcnt[w];
    }
    if (q.loss) *q.loss = n > 0 ? tot / (float)n : 0.f;
    if (q.count) *q.count = n;
  }
}

static hipError_t launch_row_triples(const UnmaskParams &p, hipStream_t stream) {
  const bool vec = (p.ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.logits) & 15) == 0);
  dim3 grid(p.chunks, p.B * p.S);
  if (vec)
    hipLaunchKernelGGL(unmask_partial_kernel<true>, grid, dim3(kUThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(unmask_partial_kernel<false>, grid, dim3(kUThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_unmask(const UnmaskParams &p, hipStream_t stream) {
  hipError_t e = launch_row_triples(p, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(unmask_finalize_kernel, dim3(p.B), dim3(kDecThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_masked_nll(const UnmaskParams &p, const NllParams &q, hipStream_t stream) {
  hipError_t e = launch_row_triples(p, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nll_finalize_kernel, dim3(1), dim3(1024), 0, stream, p, q);
  return hipGetLastError();
}

hipError_t launch_mask_corrupt(const CorruptParams &p, hipStream_t stream) {
  const int n = p.B * p.S;
  hipLaunchKernelGGL(mask_corrupt_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_unmask_tiles_finalize(const UnmaskParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(unmask_tiles_finalize_kernel, dim3(p.B), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
