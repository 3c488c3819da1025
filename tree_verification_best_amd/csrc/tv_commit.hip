// tv_commit.hip -- KV commit of the accepted path after a verification round.
//
// Primer, "KV cache handling": only the accepted tokens stay in the target
// cache; the rejected candidates' entries are dropped.  Tree row L + i holds
// node i; the committed sequence is the root and the accepted drafts,
// accepted_nodes[0..accept_len], and row L + accepted_nodes[j] moves to row
// L + j.  The path starts at node 0 and increases strictly, so no source row
// lies below its destination.  Each thread owns one 16-byte column slice of
// one head's rows and moves batches of rows: it reads a whole batch before
// writing it, and a later batch reads only rows at or past its own first
// destination, which no earlier batch wrote.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_internal.h"

namespace tvk {

constexpr int kCommitNT = 256;
constexpr int kCommitBatch = 8;
constexpr int kCommitMaxPath = 1024;

__global__ __launch_bounds__(kCommitNT) void k_kv_commit(
    uint4* __restrict__ k, uint4* __restrict__ v, int Hkv, int cap, int row16,
    const int* __restrict__ ctx_len, const int* __restrict__ accept_len,
    const int* __restrict__ accepted_nodes, int width, int* new_ctx_len) {
  __shared__ int path[kCommitMaxPath];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = ctx_len[b], a = accept_len[b];
  const int np = min(a + 1, width);
  for (int j = tid; j < np; j += kCommitNT) path[j] = accepted_nodes[(int64_t)b * width + j];
  __syncthreads();
  // a path starting at the root, strictly increasing, inside the cache
  int bad = a + 1 > width ? 1 : 0;
  for (int j = tid; j < np; j += kCommitNT)
    bad |= j == 0 ? (path[0] != 0) : (path[j] <= path[j - 1]);
  if (np > 0 && tid == 0) bad |= (int64_t)L + path[np - 1] >= cap ? 1 : 0;
  bad = __syncthreads_or(bad);
  if (tid == 0) new_ctx_len[b] = a < 0 ? L : (bad ? -1 : L + a + 1);
  if (a <= 0 || bad) return;
  const int items = Hkv * 2 * row16;
  for (int it = tid; it < items; it += kCommitNT) {
    const int col = it % row16;
    const int kv = (it / row16) & 1;
    const int h = it / (2 * row16);
    uint4* base = (kv ? v : k) + (((int64_t)b * Hkv + h) * cap + L) * row16 + col;
    for (int j0 = 1; j0 <= a; j0 += kCommitBatch) {
      uint4 x[kCommitBatch];
#pragma unroll
      for (int q = 0; q < kCommitBatch; ++q)
        if (j0 + q <= a) x[q] = base[(int64_t)path[j0 + q] * row16];
#pragma unroll
      for (int q = 0; q < kCommitBatch; ++q)
        if (j0 + q <= a && path[j0 + q] != j0 + q) base[(int64_t)(j0 + q) * row16] = x[q];
    }
  }
}

hipError_t launch_kv_commit(void* k_cache, void* v_cache, int elem_bytes, int batch, int Hkv,
                            int cap, int D, const int* ctx_len, const int* accept_len,
                            const int* accepted_nodes, int width, int* new_ctx_len,
                            hipStream_t stream) {
  const int row16 = D * elem_bytes / 16;
  hipLaunchKernelGGL(k_kv_commit, dim3(batch), dim3(kCommitNT), 0, stream,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), Hkv, cap, row16,
                     ctx_len, accept_len, accepted_nodes, width, new_ctx_len);
  return hipGetLastError();
}

}  // namespace tvk
