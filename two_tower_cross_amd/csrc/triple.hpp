// Partial (max, first argmax, sum of exp(x - max)) of a slice of a logits row, and its exact
// merge. Used by the unmasking kernels and by the lm-head epilogue that feeds them.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace tt {

struct Triple {
  float m;  // running maximum
  int idx;  // lowest index attaining m
  float z;  // sum of exp(x - m); 0 for an empty slice
};

__device__ __forceinline__ Triple empty_triple() {
  Triple t;
  t.m = -INFINITY;
  t.idx = 0x7fffffff;
  t.z = 0.f;
  return t;
}

// Exact up to rounding; the index rule (larger m, or equal m and lower index) does not depend on
// the order of the operands.
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

}  // namespace tt
