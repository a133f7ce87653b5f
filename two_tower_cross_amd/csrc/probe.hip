// Measurement probe for gfx950: a plain streaming read of device memory, the practical ceiling
// that the bandwidth-bound kernels of this library are compared with next to the nominal HBM peak.
//
// stream_read_kernel: every thread reads 16-byte words with non-temporal loads (the policy the
// library's streaming kernels use), four independent loads in flight per iteration of a
// grid-stride loop, and folds them with XOR. The result is stored only in the (practically never
// taken) case that it equals a fixed constant, so the loads cannot be removed and the probe writes
// nothing.
#include "common.hpp"
#include "kernels.hpp"

namespace tt {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *src, size_t n16,
                                                          uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    const u32x4 x = (a ^ b) ^ (c ^ d);
    acc ^= (x[0] ^ x[1]) ^ (x[2] ^ x[3]);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= (a[0] ^ a[1]) ^ (a[2] ^ a[3]);
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

hipError_t launch_stream_read(const void *src, size_t bytes, int workgroups, uint32_t *sink,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4 *>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace tt
