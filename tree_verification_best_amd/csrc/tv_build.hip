// tv_build.hip -- draft tree construction on gfx950.
//
// TAPS sec. 4.1 / 4.2 and TreeGraft sec. 3.1: per-position top-k candidates
// of the drafter's marginals, each edge scored by the drafter's probability
// of the child token, path score = product of edge scores from the root,
// and the `budget` best paths form a prefix-closed subtree.
//
// Kernels (one stream, in order):
//   k_chunk_topk   grid (chunks, b*K)  top-k of each 8192-token chunk of a draft row
//   k_chunk_z      grid (chunks, b*K)  fixed-point softmax mass of each chunk
//   k_finalize     grid (b*K)          row top-k, q = W / Z, rank by (q desc, id asc)
//   k_select       grid (b)            exact best-B selection + rows + ancestors
//
// Selection (k_select).  Nodes are ordered by (score desc, depth asc,
// parent earlier, rank asc).  Within one depth this is the order of
// (score desc, parent's position in its own depth's order, rank) -- the
// "level order".  The kernel builds, depth by depth, the level-d nodes that
// can still be among the B best:
//   * parents: the depth d-1 nodes currently among the B best, a prefix of
//     their level order with positions 0..m-1;
//   * candidate (i, r) = parent i, child rank r, score fl64(s_i * q_d(r)).
//     Scores fall (weakly) in both i and r, and ties go to smaller i then r,
//     so (i', r') with i' <= i, r' <= r all come first: (i, r) can only be
//     among the B best if (i+1)(r+1) <= B.  Once B nodes are known, a
//     candidate also needs a score above the B-th best (it is deeper than
//     everything chosen so far, so a tie loses);
//   * candidates are bitonic-sorted in LDS into level order, and merged with
//     the running best-B list (bitonic merge); the first B are kept.
// When a depth adds nothing, no deeper node can enter.  The result is the
// exact B-best set in order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

constexpr int kBuildNT = 256;

// ---------------------------------------------------------------------------
template <typename T, int E>
__global__ __launch_bounds__(kBuildNT) void k_chunk_topk(const T* __restrict__ logits, int V,
                                                        int C, int chunk, int k,
                                                        float* __restrict__ cval,
                                                        int* __restrict__ cid) {
  __shared__ TopkScratch<kBuildNT> sc;
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
  const T* p = logits + row * (int64_t)V;
  const int base = c * chunk;
  // A full chunk: thread t holds the E consecutive tokens [base + t*E, ...)
  // (16-byte loads).  The partial last chunk is spread across all threads
  // (token base + e*NT + t), so that every lane holds real tokens when the
  // chunk has at least NT of them.  Ids >= V are padding.
  float val[E];
  int id[E];
  if (base + chunk <= V) {
    const int i0 = base + (int)threadIdx.x * E;
    load_run<E>(p, i0, V, val);
#pragma unroll
    for (int e = 0; e < E; ++e) id[e] = i0 + e;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = base + e * kBuildNT + (int)threadIdx.x;
      val[e] = idx < V ? Elem<T>::load(p, idx) : -__builtin_inff();
      id[e] = idx;
    }
  }
  float* ov = cval + (row * C + c) * (int64_t)k;
  int* oi = cid + (row * C + c) * (int64_t)k;
  // padding slots of a chunk with fewer than k tokens get ids unique per chunk
  block_topk<kBuildNT, E>(val, id, k, sc, ov, oi, V, V + c * k);
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBuildNT) void k_chunk_z(const T* __restrict__ logits, int V,
                                                     int C, int chunk, int k, float inv_t,
                                                     const float* __restrict__ cval,
                                                     uint64_t* __restrict__ cz) {
  __shared__ uint64_t wsum[kBuildNT / WAVE];
  __shared__ float s_m;
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
  // the chunk's logits first; the row maximum (over the chunk maxima, the
  // first candidate of every chunk) arrives while they are in flight
  const T* p = logits + row * (int64_t)V;
  const int base = c * chunk;
  float x[kBuildChunk / kBuildNT];
  load_run<kBuildChunk / kBuildNT>(p, base + (int)threadIdx.x * (kBuildChunk / kBuildNT), V, x);
  if (threadIdx.x < WAVE) {
    float m = -__builtin_inff();
    for (int j = threadIdx.x; j < C; j += WAVE) m = fmaxf(m, cval[(row * C + j) * (int64_t)k]);
    m = wave_max_f(m);
    if (threadIdx.x == 0) s_m = m;
  }
  __syncthreads();
  const float m = s_m;
  uint64_t acc = 0;
#pragma unroll
  for (int j = 0; j < kBuildChunk / kBuildNT; ++j) acc += weight(x[j], m, inv_t);
  acc = wave_sum_u64(acc);
  if (lane_id() == 0) wsum[threadIdx.x / WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t z = 0;
    for (int w = 0; w < kBuildNT / WAVE; ++w) z += wsum[w];
    cz[row * C + c] = z;
  }
}

// ---------------------------------------------------------------------------
template <int E>
__global__ __launch_bounds__(kBuildNT) void k_finalize(int V, int C, int chunk, int k,
                                                      float inv_t,
                                                      const float* __restrict__ cval,
                                                      const int* __restrict__ cid,
                                                      const uint64_t* __restrict__ cz,
                                                      int* __restrict__ ftok,
                                                      double* __restrict__ fq) {
  __shared__ TopkScratch<kBuildNT> sc;
  __shared__ float tv[TV_MAX_TOPK_];
  __shared__ int ti[TV_MAX_TOPK_];
  __shared__ double tq[TV_MAX_TOPK_];
  __shared__ uint64_t s_z;
  const int64_t row = blockIdx.x;
  const int n = C * k;
  float val[E];
  int id[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int j = e * kBuildNT + (int)threadIdx.x;
    bool ok = j < n;
    val[e] = ok ? cval[row * n + j] : -__builtin_inff();
    id[e] = ok ? cid[row * n + j] : V + C * chunk + j;
  }
  if (threadIdx.x < WAVE) {
    uint64_t z = 0;
    for (int j = threadIdx.x; j < C; j += WAVE) z += cz[row * C + j];
    z = wave_sum_u64(z);
    if (threadIdx.x == 0) s_z = z;
  }
  block_topk<kBuildNT, E>(val, id, k, sc, tv, ti, V, V);  // ends with a barrier
  const float m = tv[0];                             // the row maximum
  const uint64_t Z = s_z;
  if ((int)threadIdx.x < k) {
    uint64_t w = weight(tv[threadIdx.x], m, inv_t);
    tq[threadIdx.x] = (double)w / (double)Z;
  }
  __syncthreads();
  if ((int)threadIdx.x < k) {
    const int t = threadIdx.x;
    const double q = tq[t];
    const int me = ti[t];
    int r = 0;
    for (int j = 0; j < k; ++j) r += (tq[j] > q || (tq[j] == q && ti[j] < me)) ? 1 : 0;
    ftok[row * k + r] = me;
    fq[row * k + r] = q;
  }
}

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------
// Workgroup-wide LDS hand-off.  A one-wave workgroup needs no s_barrier:
// its LDS operations complete in issue order, so waiting for its own
// outstanding ones is enough.
template <int NT>
__device__ __forceinline__ void block_sync() {
  if constexpr (NT == WAVE)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  else
    __syncthreads();
}

__device__ __forceinline__ bool sm_better(double as, uint64_t am, double bs, uint64_t bm) {
  return as > bs || (as == bs && am < bm);
}

template <int NT, typename KT>
__device__ void bitonic_sort(double* s, KT* m, int n) {
  for (int size = 2; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += NT) {
        int i = 2 * t - (t & (stride - 1));
        int j = i + stride;
        bool up = (i & size) == 0;
        double si = s[i], sj = s[j];
        KT mi = m[i], mj = m[j];
        bool sw = up ? sm_better(sj, mj, si, mi) : sm_better(si, mi, sj, mj);
        if (sw) {
          s[i] = sj;
          s[j] = si;
          m[i] = mj;
          m[j] = mi;
        }
      }
      block_sync<NT>();
    }
}

// n elements holding a best-first half followed by a worst-first half
template <int NT>
__device__ void bitonic_merge(double* s, uint64_t* m, int n) {
  for (int stride = n >> 1; stride > 0; stride >>= 1) {
    for (int t = threadIdx.x; t < (n >> 1); t += NT) {
      int i = 2 * t - (t & (stride - 1));
      int j = i + stride;
      double si = s[i], sj = s[j];
      uint64_t mi = m[i], mj = m[j];
      if (sm_better(sj, mj, si, mi)) {
        s[i] = sj;
        s[j] = si;
        m[i] = mj;
        m[j] = mi;
      }
    }
    block_sync<NT>();
  }
}

template <int NT>
__device__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = lane_id(), wave = threadIdx.x / WAVE;
  int incl = wave_incl_scan_i(v);
  if (lane == WAVE - 1) wsum[wave] = incl;
  block_sync<NT>();
  int woff = 0, tot = 0;
  for (int w = 0; w < NT / WAVE; ++w) {
    int x = wsum[w];
    if (w < wave) woff += x;
    tot += x;
  }
  total = tot;
  block_sync<NT>();
  return woff + incl - v;
}

__host__ __device__ inline int pow2ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// meta of a chosen node: depth << 48 | level position << 32 | parent << 16 | rank
__device__ __forceinline__ int meta_depth(uint64_t m) { return (int)(m >> 48); }
__device__ __forceinline__ int meta_pos(uint64_t m) { return (int)((m >> 32) & 0xFFFF); }
__device__ __forceinline__ int meta_parent(uint64_t m) { return (int)((m >> 16) & 0xFFFF); }
__device__ __forceinline__ int meta_rank(uint64_t m) { return (int)(m & 0xFFFF); }

// Ancestor bit rows from a parent array held in LDS: each row walks its
// chain to the root (parents strictly decrease, so the walk ends).
template <int NT>
__device__ void write_ancestors(const int* par, int n, int N, int W, uint64_t* anc) {
  for (int j = threadIdx.x; j < N; j += NT) {
    uint64_t acc[16];
#pragma unroll
    for (int w = 0; w < 16; ++w) acc[w] = 0;
    if (j < n) {
      int node = j;
      for (int step = 0; step <= N; ++step) {
        const int w = node >> 6;
        const uint64_t bit = 1ull << (node & 63);
#pragma unroll
        for (int ww = 0; ww < 16; ++ww) acc[ww] |= (ww == w) ? bit : 0ull;
        const int p = par[node];
        if (p < 0 || p >= node) break;
        node = p;
      }
    }
#pragma unroll
    for (int w = 0; w < 16; ++w)
      if (w < W) anc[(int64_t)j * W + w] = acc[w];
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void k_select(const int* __restrict__ ftok,
                                              const double* __restrict__ fq, int K, int k,
                                              int B, int P, int Q2,
                                              const int* __restrict__ root_token,
                                              const int* __restrict__ ctx_len,
                                              int* __restrict__ parent, int* __restrict__ token,
                                              int* __restrict__ depth, int* __restrict__ pos,
                                              double* __restrict__ score,
                                              uint64_t* __restrict__ anc,
                                              int* __restrict__ n_nodes) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x;
  const int N = B + 1;
  const int W = (N + 63) / 64;
  const int Kk = K * k;
  double* qtab = reinterpret_cast<double*>(smem);
  double* Ms = qtab + Kk;
  double* Cs = Ms + Q2;
  double* par_s = Cs + P;
  uint64_t* Mm = reinterpret_cast<uint64_t*>(par_s + N);
  uint32_t* Ck = reinterpret_cast<uint32_t*>(Mm + Q2);
  int* ttab = reinterpret_cast<int*>(Ck + P);
  int* rowpar = ttab + Kk;            // [N] parent rows (epilogue)
  int* flat = rowpar + N;             // [N] row of (depth, position)
  int* dcnt = flat + N;               // [K + 2] per-depth counts / offsets
  __shared__ int wsum[NT / WAVE];

  for (int i = threadIdx.x; i < Kk; i += NT) {
    qtab[i] = fq[(int64_t)b * Kk + i];
    ttab[i] = ftok[(int64_t)b * Kk + i];
  }
  if (threadIdx.x == 0) par_s[0] = 1.0;
  block_sync<NT>();

  int g = 0, m_par = 1;
  bool have_kappa = false;
  double kappa = 0.0;
  for (int d = 1; d <= K && B > 0; ++d) {
    const double* qd = qtab + (d - 1) * k;
    const int ppt = (m_par + NT - 1) / NT;
    // children of each parent that can still be among the B best
    int my = 0;
    for (int j = 0; j < ppt; ++j) {
      const int i = threadIdx.x * ppt + j;
      if (i < m_par) {
        const int lim = min(k, B / (i + 1));
        const double si = par_s[i];
        int c = 0;
        while (c < lim) {
          const double s = si * qd[c];
          if (have_kappa && !(s > kappa)) break;
          ++c;
        }
        my += c;
      }
    }
    int total;
    int off = block_excl_scan<NT>(my, wsum, total);
    if (total == 0) break;
    for (int j = 0; j < ppt; ++j) {
      const int i = threadIdx.x * ppt + j;
      if (i < m_par) {
        const int lim = min(k, B / (i + 1));
        const double si = par_s[i];
        for (int c = 0; c < lim; ++c) {
          const double s = si * qd[c];
          if (have_kappa && !(s > kappa)) break;
          Cs[off] = s;
          Ck[off] = ((uint32_t)i << 16) | (uint32_t)c;
          ++off;
        }
      }
    }
    const int Pn = pow2ceil(total);
    for (int t = total + threadIdx.x; t < Pn; t += NT) {
      Cs[t] = -1.0;
      Ck[t] = 0xFFFFFFFFu;
    }
    block_sync<NT>();
    bitonic_sort<NT, uint32_t>(Cs, Ck, Pn);
    const int l = min(total, B);
    const int Q = pow2ceil(max(g, l));
    for (int p = threadIdx.x; p < Q; p += NT) {
      if (p >= g) {
        Ms[p] = -1.0;
        Mm[p] = ~0ull;
      }
      if (p < l) {
        Ms[2 * Q - 1 - p] = Cs[p];
        Mm[2 * Q - 1 - p] = ((uint64_t)d << 48) | ((uint64_t)p << 32) | (uint64_t)Ck[p];
      } else {
        Ms[2 * Q - 1 - p] = -1.0;
        Mm[2 * Q - 1 - p] = ~0ull;
      }
    }
    block_sync<NT>();
    bitonic_merge<NT>(Ms, Mm, 2 * Q);
    g = min(B, g + l);
    if (g == B) {
      have_kappa = true;
      kappa = Ms[B - 1];
    }
    // next parents: the depth-d nodes kept, at their level positions
    int cnt = 0;
    for (int p = threadIdx.x; p < g; p += NT) {
      const uint64_t mm = Mm[p];
      if (meta_depth(mm) == d) {
        par_s[meta_pos(mm)] = Ms[p];
        ++cnt;
      }
    }
    int tot2;
    (void)block_excl_scan<NT>(cnt, wsum, tot2);
    m_par = tot2;
    if (m_par == 0) break;
  }

  // ---- epilogue: rows in order, parents, ancestors ----
  const int n = g + 1;
  for (int d = threadIdx.x; d < K + 2; d += NT) dcnt[d] = 0;
  block_sync<NT>();
  for (int p = threadIdx.x; p < g; p += NT) atomicAdd(&dcnt[meta_depth(Mm[p])], 1);
  block_sync<NT>();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int d = 0; d < K + 2; ++d) {
      int c = dcnt[d];
      dcnt[d] = acc;  // offset of depth d in `flat`
      acc += c;
    }
  }
  block_sync<NT>();
  for (int p = threadIdx.x; p < g; p += NT) {
    const uint64_t mm = Mm[p];
    flat[dcnt[meta_depth(mm)] + meta_pos(mm)] = p + 1;
  }
  block_sync<NT>();
  const int64_t rb = (int64_t)b * N;
  const int L = ctx_len[b];
  for (int j = threadIdx.x; j < N; j += NT) {
    int pa = -1, to = -1, de = -1, po = -1;
    double sc = 0.0;
    if (j == 0) {
      to = root_token[b];
      de = 0;
      po = L;
      sc = 1.0;
    } else if (j < n) {
      const uint64_t mm = Mm[j - 1];
      const int d = meta_depth(mm);
      pa = d == 1 ? 0 : flat[min(dcnt[d - 1] + meta_parent(mm), N - 1)];
      to = ttab[(d - 1) * k + meta_rank(mm)];
      de = d;
      po = L + d;
      sc = Ms[j - 1];
    }
    rowpar[j] = pa;
    parent[rb + j] = pa;
    token[rb + j] = to;
    depth[rb + j] = de;
    pos[rb + j] = po;
    score[rb + j] = sc;
  }
  if (threadIdx.x == 0) n_nodes[b] = n;
  block_sync<NT>();
  write_ancestors<NT>(rowpar, n, N, W, anc + rb * W);
}

// ---------------------------------------------------------------------------
// ancestors of caller-supplied trees
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(NT) void k_ancestors(const int* __restrict__ parent,
                                                 const int* __restrict__ n_nodes,
                                                 const int* __restrict__ ctx_len, int N,
                                                 int* __restrict__ depth, int* __restrict__ pos,
                                                 uint64_t* __restrict__ anc) {
  __shared__ int par[1024];
  const int b = blockIdx.x;
  const int W = (N + 63) / 64;
  const int64_t rb = (int64_t)b * N;
  const int n = min(max(n_nodes[b], 0), N);
  for (int j = threadIdx.x; j < N; j += NT) par[j] = j < n ? parent[rb + j] : -1;
  __syncthreads();
  const int L = ctx_len[b];
  for (int j = threadIdx.x; j < N; j += NT) {
    int d = -1;
    if (j < n) {
      d = 0;
      int node = j;
      for (int step = 0; step <= N; ++step) {
        const int p = par[node];
        if (p < 0 || p >= node) break;
        node = p;
        ++d;
      }
    }
    depth[rb + j] = d;
    pos[rb + j] = j < n ? L + d : -1;
  }
  write_ancestors<NT>(par, n, N, W, anc + rb * W);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
BuildPlan build_plan(int batch, int K, int V, int topk, int budget) {
  BuildPlan p{};
  p.chunk = kBuildChunk;
  p.C = (V + p.chunk - 1) / p.chunk;
  p.rows = (int64_t)batch * K;
  // candidates one depth can contribute: sum over parents i of min(k, B/(i+1))
  int64_t cmax = 0;
  for (int i = 0; i < budget; ++i) cmax += std::min(topk, budget / (i + 1));
  p.P = pow2ceil((int)std::max<int64_t>(cmax, 1));
  p.Q2 = 2 * pow2ceil(std::max(budget, 1));
  const int N = budget + 1;
  const int Kk = K * topk;
  p.select_lds = (size_t)Kk * 8 + (size_t)p.Q2 * 8 + (size_t)p.P * 8 + (size_t)N * 8 +
                 (size_t)p.Q2 * 8 + (size_t)p.P * 4 + (size_t)Kk * 4 + (size_t)N * 4 * 2 +
                 (size_t)(K + 2) * 4 + 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.off_cval = take((size_t)p.rows * p.C * topk * sizeof(float));
  p.off_cid = take((size_t)p.rows * p.C * topk * sizeof(int));
  p.off_cz = take((size_t)p.rows * p.C * sizeof(uint64_t));
  p.off_ftok = take((size_t)p.rows * topk * sizeof(int));
  p.off_fq = take((size_t)p.rows * topk * sizeof(double));
  p.workspace = off;
  return p;
}

hipError_t launch_build(const BuildPlan& p, const void* draft, bool bf16, int batch, int K,
                        int V, int topk, int budget, float inv_t, const int* root_token,
                        const int* ctx_len, int* parent, int* token, int* depth, int* pos,
                        double* score, uint64_t* anc, int* n_nodes, void* ws,
                        hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  float* cval = reinterpret_cast<float*>(w + p.off_cval);
  int* cid = reinterpret_cast<int*>(w + p.off_cid);
  uint64_t* cz = reinterpret_cast<uint64_t*>(w + p.off_cz);
  int* ftok = reinterpret_cast<int*>(w + p.off_ftok);
  double* fq = reinterpret_cast<double*>(w + p.off_fq);
  constexpr int E1 = kBuildChunk / kBuildNT;
  dim3 g1(p.C, (unsigned)p.rows);
  if (bf16) {
    hipLaunchKernelGGL((k_chunk_topk<uint16_t, E1>), g1, dim3(kBuildNT), 0, stream,
                       static_cast<const uint16_t*>(draft), V, p.C, p.chunk, topk, cval, cid);
    hipLaunchKernelGGL((k_chunk_z<uint16_t>), g1, dim3(kBuildNT), 0, stream,
                       static_cast<const uint16_t*>(draft), V, p.C, p.chunk, topk, inv_t, cval,
                       cz);
  } else {
    hipLaunchKernelGGL((k_chunk_topk<float, E1>), g1, dim3(kBuildNT), 0, stream,
                       static_cast<const float*>(draft), V, p.C, p.chunk, topk, cval, cid);
    hipLaunchKernelGGL((k_chunk_z<float>), g1, dim3(kBuildNT), 0, stream,
                       static_cast<const float*>(draft), V, p.C, p.chunk, topk, inv_t, cval, cz);
  }
  hipLaunchKernelGGL((k_finalize<kFinalizeE>), dim3((unsigned)p.rows), dim3(kBuildNT), 0,
                     stream, V, p.C, p.chunk, topk, inv_t, cval, cid, cz, ftok, fq);
  // small candidate sets: one wave, no workgroup barriers
  if (p.P <= 512)
    hipLaunchKernelGGL((k_select<WAVE>), dim3(batch), dim3(WAVE), p.select_lds, stream, ftok,
                       fq, K, topk, budget, p.P, p.Q2, root_token, ctx_len, parent, token, depth,
                       pos, score, anc, n_nodes);
  else
    hipLaunchKernelGGL((k_select<kBuildNT>), dim3(batch), dim3(kBuildNT), p.select_lds, stream,
                       ftok, fq, K, topk, budget, p.P, p.Q2, root_token, ctx_len, parent, token,
                       depth, pos, score, anc, n_nodes);
  return hipGetLastError();
}

hipError_t launch_ancestors(const int* parent, const int* n_nodes, const int* ctx_len,
                            int batch, int N, int* depth, int* pos, uint64_t* anc,
                            hipStream_t stream) {
  hipLaunchKernelGGL((k_ancestors<kBuildNT>), dim3(batch), dim3(kBuildNT), 0, stream, parent,
                     n_nodes, ctx_len, N, depth, pos, anc);
  return hipGetLastError();
}

}  // namespace tvk
