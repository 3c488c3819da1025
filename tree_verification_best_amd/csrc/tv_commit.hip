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
//
// With the rotary embedding fused into verification, tree rows hold keys not
// yet rotated; the rotary commit turns each kept key at the position of the
// row it lands on, L + j (the node's position id L + depth, as the path's
// j-th node has depth j), the root included.  Its K threads own a pair of
// column slices (d, d + D/2) so that both members of each rotation pair are
// in one thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

constexpr int kCommitNT = 256;
constexpr int kCommitBatch = 8;
constexpr int kCommitMaxPath = 1024;

// Loads sequence b's path into LDS and checks it: it starts at the root,
// increases strictly and stays inside the cache (a negative context length
// fails the check).  Writes new_ctx_len[b] and
// returns whether the rows are to be moved.
__device__ bool commit_path(int b, int cap, const int* ctx_len, const int* accept_len,
                            const int* accepted_nodes, int width, int* new_ctx_len, int* path,
                            int& L, int& a) {
  const int tid = threadIdx.x;
  L = ctx_len[b];
  a = accept_len[b];
  // (no a + 1: accept_len may hold any value)
  const int np = a < 0 ? 0 : (a < width ? a + 1 : width);
  for (int j = tid; j < np; j += kCommitNT) path[j] = accepted_nodes[(int64_t)b * width + j];
  __syncthreads();
  int bad = a >= width ? 1 : 0;
  for (int j = tid; j < np; j += kCommitNT)
    bad |= j == 0 ? (path[0] != 0) : (path[j] <= path[j - 1]);
  if (np > 0 && tid == 0) bad |= (L < 0 || (int64_t)L + path[np - 1] >= cap) ? 1 : 0;
  bad = __syncthreads_or(bad);
  if (tid == 0) new_ctx_len[b] = a < 0 ? L : (bad ? -1 : L + a + 1);
  return a >= 0 && !bad;
}

__global__ __launch_bounds__(kCommitNT) void k_kv_commit(
    uint4* __restrict__ k, uint4* __restrict__ v, int Hkv, int cap, int row16,
    const int* __restrict__ ctx_len, const int* __restrict__ accept_len,
    const int* __restrict__ accepted_nodes, int width, int* new_ctx_len) {
  __shared__ int path[kCommitMaxPath];
  const int b = blockIdx.x, tid = threadIdx.x;
  int L, a;
  if (!commit_path(b, cap, ctx_len, accept_len, accepted_nodes, width, new_ctx_len, path, L, a) ||
      a == 0)
    return;
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

// Rotary commit: V rows move as above; each K thread owns the column
// slices (c, c + row16/2) of one head, i.e. the E elements d = E c + e and
// d + D/2, and turns every kept row j (the root included) at position L + j
// before writing it to row L + j.
template <typename T>
__global__ __launch_bounds__(kCommitNT) void k_kv_commit_rope(
    uint4* __restrict__ k, uint4* __restrict__ v, int Hkv, int cap, int row16,
    const int* __restrict__ ctx_len, const int* __restrict__ accept_len,
    const int* __restrict__ accepted_nodes, int width, int* new_ctx_len, int D,
    double log2_base) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte slice
  __shared__ int path[kCommitMaxPath];
  __shared__ double rate[64];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid < D / 2) rate[tid] = rope_rate(tid, D, log2_base);
  int L, a;
  if (!commit_path(b, cap, ctx_len, accept_len, accepted_nodes, width, new_ctx_len, path, L, a))
    return;  // commit_path's barriers also publish `rate`
  const int half16 = row16 / 2;
  const int vitems = Hkv * row16, kitems = Hkv * half16;
  for (int it = tid; it < vitems + kitems; it += kCommitNT) {
    if (it < vitems) {
      const int col = it % row16, h = it / row16;
      uint4* base = v + (((int64_t)b * Hkv + h) * cap + L) * row16 + col;
      for (int j0 = 1; j0 <= a; j0 += kCommitBatch) {
        uint4 x[kCommitBatch];
#pragma unroll
        for (int q = 0; q < kCommitBatch; ++q)
          if (j0 + q <= a) x[q] = base[(int64_t)path[j0 + q] * row16];
#pragma unroll
        for (int q = 0; q < kCommitBatch; ++q)
          if (j0 + q <= a && path[j0 + q] != j0 + q) base[(int64_t)(j0 + q) * row16] = x[q];
      }
    } else {
      const int c = (it - vitems) % half16, h = (it - vitems) / half16;
      uint4* base = k + (((int64_t)b * Hkv + h) * cap + L) * row16 + c;
      for (int j0 = 0; j0 <= a; j0 += kCommitBatch) {
        uint4 lo[kCommitBatch], hi[kCommitBatch];
#pragma unroll
        for (int q = 0; q < kCommitBatch; ++q)
          if (j0 + q <= a) {
            lo[q] = base[(int64_t)path[j0 + q] * row16];
            hi[q] = base[(int64_t)path[j0 + q] * row16 + half16];
          }
#pragma unroll
        for (int q = 0; q < kCommitBatch; ++q)
          if (j0 + q <= a) {
            T* xl = reinterpret_cast<T*>(&lo[q]);
            T* xh = reinterpret_cast<T*>(&hi[q]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              float sn, cs;
              rope_sincos(L + j0 + q, rate[E * c + e], sn, cs);
              const float fl = to_f32(xl[e]), fh = to_f32(xh[e]);
              xl[e] = from_f32<T>(fl * cs - fh * sn);
              xh[e] = from_f32<T>(fh * cs + fl * sn);
            }
            base[(int64_t)(j0 + q) * row16] = lo[q];
            base[(int64_t)(j0 + q) * row16 + half16] = hi[q];
          }
      }
    }
  }
}

hipError_t launch_kv_commit(void* k_cache, void* v_cache, int elem_bytes, int batch, int Hkv,
                            int cap, int D, const int* ctx_len, const int* accept_len,
                            const int* accepted_nodes, int width, int* new_ctx_len,
                            bool rope, double log2_base, hipStream_t stream) {
  const int row16 = D * elem_bytes / 16;
  uint4* k = static_cast<uint4*>(k_cache);
  uint4* v = static_cast<uint4*>(v_cache);
  if (!rope)
    hipLaunchKernelGGL(k_kv_commit, dim3(batch), dim3(kCommitNT), 0, stream, k, v, Hkv, cap,
                       row16, ctx_len, accept_len, accepted_nodes, width, new_ctx_len);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(k_kv_commit_rope<uint16_t>, dim3(batch), dim3(kCommitNT), 0, stream, k, v,
                       Hkv, cap, row16, ctx_len, accept_len, accepted_nodes, width, new_ctx_len, D,
                       log2_base);
  else
    hipLaunchKernelGGL(k_kv_commit_rope<float>, dim3(batch), dim3(kCommitNT), 0, stream, k, v,
                       Hkv, cap, row16, ctx_len, accept_len, accepted_nodes, width, new_ctx_len, D,
                       log2_base);
  return hipGetLastError();
}

}  // namespace tvk
