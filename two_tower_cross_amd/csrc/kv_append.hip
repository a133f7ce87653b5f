// Context KV append after a block is committed, for gfx950 (Nemotron-TwoTower explainer,
// "Generierungsprozess": once a block is fully committed, the frozen context tower encodes it and
// its keys and values join the cache that the next block attends to).
//
// kv_alloc_kernel: one wavefront; lane 0 walks the sequences in order, pops the pages each one
//   needs from the top of the free-page stack into its block table, records the length before the
//   append in the workspace and sets the new length. A sequence that does not fit (free stack or
//   block table too short, a length outside the cache, or a page id outside the pools) is skipped
//   and flagged in *status, so the copy below never writes outside the pools.
// kv_write_kernel: one work-group per (sequence, KV head, layer) copies the block's S key rows
//   and value rows to their cache slots (the chunk-major 64-token tiles of k_elem / v_elem).
#include "common.hpp"
#include "kernels.hpp"

namespace tt {

__global__ __launch_bounds__(64) void kv_alloc_kernel(AppendParams p) {
  if (threadIdx.x != 0) return;
  int top = *p.free_count;
  int flags = 0;
  const int P = p.page_size;
  for (int b = 0; b < p.B; ++b) {
    const int L = p.ctx_lens[b];
    if (L < 0 || (int64_t)L + p.S > (int64_t)p.max_pages * P) {
      p.old_len[b] = -1;
      flags |= kAppendNoRoomInTable;
      continue;
    }
    const int have = (L + P - 1) / P;            // pages holding rows 0 .. L-1
    const int need = (L + p.S + P - 1) / P - have;
    if (need > top) {
      p.old_len[b] = -1;
      flags |= kAppendOutOfPages;
      continue;
    }
    // every page the rows will land in must be inside the pools (the partly filled last page of
    // the table, if any, and the popped ones); otherwise nothing of this sequence is written
    bool ok = L % P == 0 || (unsigned)p.block_table[(size_t)b * p.max_pages + L / P] < (unsigned)p.num_pages;
    for (int j = 0; j < need; ++j) ok = ok && (unsigned)p.free_pages[top - 1 - j] < (unsigned)p.num_pages;
    if (!ok) {
      p.old_len[b] = -1;
      flags |= kAppendBadPage;
      continue;
    }
    for (int j = 0; j < need; ++j) p.block_table[(size_t)b * p.max_pages + have + j] = p.free_pages[top - 1 - j];
    top -= need;
    p.old_len[b] = L;
    p.ctx_lens[b] = L + p.S;
  }
  *p.free_count = top;
  if (flags) *p.status |= flags;
}

// E: the element type's storage (uint16_t for bf16, uint32_t for fp32); a copy, no arithmetic.
template <typename E>
__global__ __launch_bounds__(256) void kv_write_kernel(AppendParams p) {
  const int b = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int L = p.old_len[b];
  if (L < 0) return;
  const int P = p.page_size, D = p.D, S = p.S, Hkv = p.Hkv;
  const int32_t *table = p.block_table + (size_t)b * p.max_pages;
  E *kp = static_cast<E *>(p.k_pages[l]);
  E *vp = static_cast<E *>(p.v_pages[l]);
  const E *kn = static_cast<const E *>(p.k_new[l]) + ((size_t)b * Hkv + g) * S * D;
  const E *vn = static_cast<const E *>(p.v_new[l]) + ((size_t)b * Hkv + g) * D * S;
  for (int e = threadIdx.x; e < S * D; e += 256) {
    const int i = e / D, d = e % D;               // key row i, dimension d (rows contiguous)
    const int t = L + i, page = table[t / P], off = t % P;
    kp[((size_t)page * Hkv + g) * P * D + k_elem(off, d, D)] = kn[e];
  }
  for (int e = threadIdx.x; e < S * D; e += 256) {
    const int d = e / S, i = e % S;               // value dimension d, row i (rows contiguous)
    const int t = L + i, page = table[t / P], off = t % P;
    vp[((size_t)page * Hkv + g) * P * D + v_elem(off, d, D)] = vn[e];
  }
}

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(kv_alloc_kernel, dim3(1), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(p.B, p.Hkv, p.layers);
  if (p.elem_bytes == 2)
    hipLaunchKernelGGL(kv_write_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_write_kernel<uint32_t>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
