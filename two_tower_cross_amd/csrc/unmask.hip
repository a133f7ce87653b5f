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
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace tt {

constexpr int kUThreads = 256;
constexpr int kUPerThread = 32;
constexpr int kUChunk = kUThreads * kUPerThread;  // 8192 logits per work-group

struct Triple {
  float m;  // running maximum
  int idx;  // lowest index attaining m
  float z;  // sum of exp(x - m)
};

__device__ __forceinline__ Triple merge(Triple a, Triple b) {
  if (b.z == 0.f) return a;
  if (a.z == 0.f) return b;
  Triple r;
  if (b.m > a.m || (b.m == a.m && b.idx < a.idx)) {
    r.m = b.m;
    r.idx = b.idx;
  } else {
    r.m = a.m;
    r.idx = a.idx;
  }
  r.z = a.z * __expf(a.m - r.m) + b.z * __expf(b.m - r.m);
  return r;
}

__device__ __forceinline__ Triple shfl_xor_triple(Triple t, int o) {
  Triple r;
  r.m = __shfl_xor(t.m, o, 64);
  r.idx = __shfl_xor(t.idx, o, 64);
  r.z = __shfl_xor(t.z, o, 64);
  return r;
}

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
  Triple t;
  t.m = -INFINITY;
  t.idx = 0x7fffffff;
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

__global__ __launch_bounds__(64) void unmask_finalize_kernel(UnmaskParams p) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool in = i < p.S;
  const size_t row = (size_t)b * p.S + i;
  const bool was_masked = in && p.masked[row] != 0;
  Triple t;
  t.m = -INFINITY;
  t.idx = 0x7fffffff;
  t.z = 0.f;
  if (was_masked) {
    for (int c = 0; c < p.chunks; ++c) {
      const float *o = p.part + (row * p.chunks + c) * 4;
      Triple u;
      u.m = o[0];
      u.idx = __float_as_int(o[1]);
      u.z = o[2];
      t = merge(t, u);
    }
  }
  const float conf = was_masked ? 1.0f / t.z : -1.0f;
  bool commit = was_masked && (p.commit_all || conf > p.threshold);
  const unsigned long long any_commit = __ballot(commit);
  const unsigned long long any_masked = __ballot(was_masked);
  if (!any_commit && p.min_commit && any_masked) {
    // largest confidence, lowest position on ties
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
    commit = was_masked && i == bi;
  }
  if (was_masked) {
    if (p.confidence) p.confidence[row] = conf;
    if (commit) {
      p.tokens[row] = t.idx;
      p.masked[row] = 0;
    }
  }
  const unsigned long long committed = __ballot(commit);
  if (i == 0 && p.n_committed) p.n_committed[b] = __popcll(committed);
}

hipError_t launch_unmask(const UnmaskParams &p, hipStream_t stream) {
  const bool vec = (p.ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.logits) & 15) == 0);
  dim3 grid(p.chunks, p.B * p.S);
  if (vec)
    hipLaunchKernelGGL(unmask_partial_kernel<true>, grid, dim3(kUThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(unmask_partial_kernel<false>, grid, dim3(kUThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(unmask_finalize_kernel, dim3(p.B), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
