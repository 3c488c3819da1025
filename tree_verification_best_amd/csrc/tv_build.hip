// tv_build.hip -- draft tree construction on gfx950.
//
// TAPS sec. 4.1 / 4.2 and TreeGraft sec. 3.1: per-position top-k candidates
// of the drafter's marginals, each edge scored by the drafter's probability
// of the child token, path score = product of edge scores from the root,
// and the `budget` best paths form a prefix-closed subtree.
//
// Kernels (one stream, in order):
//   k_chunk_topk   grid (chunks, b*K)  top-k of each 8192-token chunk of a draft row
//   k_chunk_z      grid (chunks, b*K)  fixed-point softmax mass of each chunk; the
//                                      row's last block: row top-k, q = W / Z,
//                                      rank by (q desc, id asc)
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
//   * candidates are put in level order by rank: the rank of a candidate is
//     the number of candidates ahead of it, counted by all workgroup lanes
//     over slices of the list (a depth with more than kRankMax candidates is
//     bitonic-sorted in LDS instead);
//   * the running best-B list and the depth's list are merged by rank too:
//     an item's new place is its place in its own list plus the number of
//     items of the other list ahead of it (a binary search; a best-list item
//     goes first on equal scores, as it is shallower); the first B are kept.
// When a depth adds nothing, no deeper node can enter.  The result is the
// exact B-best set in order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "treeverify.h"
#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

constexpr int kBuildNT = 256;
// per-row hand-off record of k_chunk_z (mass accumulator, arrival count),
// one 256-byte line per row
constexpr int kRowRec = 32;

// ---------------------------------------------------------------------------
template <typename T, int E>
__global__ __launch_bounds__(kBuildNT) void k_chunk_topk(const T* __restrict__ logits, int V,
                                                        int C, int chunk, int k,
                                                        float* __restrict__ cval,
                                                        int* __restrict__ cid,
                                                        uint64_t* __restrict__ rowrec) {
  __shared__ TopkScratch<kBuildNT> sc;
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
  // the row's mass accumulator and arrival count for k_chunk_z, cleared
  // here, one kernel ahead of their use
  if (c == 0 && threadIdx.x < 2) rowrec[row * kRowRec + threadIdx.x] = 0;
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
// A draft row's top-k from its chunks' candidates (val/id, padded with -inf
// and ids >= V) and its mass Z: q = W / Z in fp64, written at rank order
// (q desc, id asc) to ftok/fq[row][.].
template <int E>
__device__ __forceinline__ void finalize_candidates(float (&val)[E], int (&id)[E], uint64_t Z,
                                                    int V, int k, float inv_t,
                                                    TopkScratch<kBuildNT>& sc, float* tv,
                                                    int* ti, double* tq, int* ftok, double* fq,
                                                    int64_t row) {
  block_topk<kBuildNT, E>(val, id, k, sc, tv, ti, V, V);  // ends with a barrier
  const float m = tv[0];                                 // the row maximum
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

// Fixed-point softmax mass of each chunk, and the row's finalisation by the
// row's last block to finish.  The chunk's logits are loaded first; the row
// maximum (over the chunk maxima, the first candidate of every chunk)
// arrives while they are in flight.  Each block adds its mass into the row's
// accumulator rowrec[row][0] (an integer atomic, so the order does not
// matter) and, once that add is performed, counts itself in rowrec[row][1];
// the block that counts last has the whole mass Z and finalises the row
// from the chunks' candidates (written by k_chunk_topk, one kernel before).
template <typename T>
__global__ __launch_bounds__(kBuildNT) void k_chunk_z(const T* __restrict__ logits, int V,
                                                     int C, int chunk, int k, float inv_t,
                                                     const float* __restrict__ cval,
                                                     const int* __restrict__ cid,
                                                     uint64_t* rowrec, int* __restrict__ ftok,
                                                     double* __restrict__ fq) {
  __shared__ TopkScratch<kBuildNT> sc;
  __shared__ float tv[TV_MAX_TOPK_];
  __shared__ int ti[TV_MAX_TOPK_];
  __shared__ double tq[TV_MAX_TOPK_];
  __shared__ uint64_t wsum[kBuildNT / WAVE];
  __shared__ float s_m;
  __shared__ int s_last;
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
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
  static_assert(kBuildChunk / kBuildNT <= 512, "fp64 partial sums must stay exact");
  double accd;
  if (inv_t == 1.0f) {
    accd = (double)weight_f<true>(x[0], m, inv_t);
#pragma unroll
    for (int j = 1; j < kBuildChunk / kBuildNT; ++j)
      accd += (double)weight_f<true>(x[j], m, inv_t);
  } else {
    accd = (double)weight_f(x[0], m, inv_t);
#pragma unroll
    for (int j = 1; j < kBuildChunk / kBuildNT; ++j) accd += (double)weight_f(x[j], m, inv_t);
  }
  const uint64_t acc = wave_sum_u64((uint64_t)accd);
  if (lane_id() == 0) wsum[threadIdx.x / WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t z = 0;
    for (int w = 0; w < kBuildNT / WAVE; ++w) z += wsum[w];
    uint64_t* rec = rowrec + row * kRowRec;
    (void)__hip_atomic_fetch_add(&rec[0], z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the add is performed before the count that announces it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    s_last = __hip_atomic_fetch_add(&rec[1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint64_t)(C - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // the row's last block: the whole mass is in the accumulator.  The C * k
  // candidates take the fewest items per thread that hold them (152 at the
  // 4B shape: one), since every item costs the block top-k its work.
  const int n = C * k;
  const uint64_t Z =
      __hip_atomic_load(&rowrec[row * kRowRec], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto finalize = [&](auto Ec) {
    constexpr int FE = decltype(Ec)::value;
    float val[FE];
    int id[FE];
#pragma unroll
    for (int e = 0; e < FE; ++e) {
      const int j = e * kBuildNT + (int)threadIdx.x;
      const bool ok = j < n;
      val[e] = ok ? cval[row * n + j] : -__builtin_inff();
      id[e] = ok ? cid[row * n + j] : V + C * chunk + j;
    }
    finalize_candidates<FE>(val, id, Z, V, k, inv_t, sc, tv, ti, tq, ftok, fq, row);
  };
  static_assert(kFinalizeE == 8, "the cases below cover up to 8 items per thread");
  if (n <= kBuildNT)
    finalize(std::integral_constant<int, 1>());
  else if (n <= 2 * kBuildNT)
    finalize(std::integral_constant<int, 2>());
  else if (n <= 4 * kBuildNT)
    finalize(std::integral_constant<int, 4>());
  else
    finalize(std::integral_constant<int, 8>());
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

template <int NT>
__device__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = lane_id(), wave = threadIdx.x / WAVE;
  int incl = wave_scan_add_dpp(v);
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

__device__ __forceinline__ int pow2floor(int x) {
  int p = 1;
  while (2 * p <= x) p <<= 1;
  return x > 0 ? p : 0;
}

// Number of the first n items of a best-first list (s) with s > x, or
// s >= x when or_equal.  The predicate holds on a prefix, so an 8-way search
// finds it: each round reads 8 probes, stride apart, all issued together.
__device__ __forceinline__ int count_ahead(const double* s, int n, double x, bool or_equal) {
  if (n <= 0) return 0;
  int stride = 1;
  while (stride * 8 < n) stride *= 8;
  int at = 0;
  for (; stride > 0; stride >>= 3) {
    double y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) y[u] = s[min(at + stride * (u + 1), n) - 1];
    int adv = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      adv += (at + stride * (u + 1) <= n && (y[u] > x || (or_equal && y[u] == x))) ? 1 : 0;
    at += adv * stride;
  }
  return at;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_select(const int* __restrict__ ftok,
                                              const double* __restrict__ fq, int K, int k,
                                              int B, int P, const int* __restrict__ root_token,
                                              const int* __restrict__ ctx_len,
                                              int* __restrict__ parent, int* __restrict__ token,
                                              int* __restrict__ depth, int* __restrict__ pos,
                                              double* __restrict__ score,
                                              uint64_t* __restrict__ anc,
                                              int* __restrict__ n_nodes) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int wsum[NT / WAVE];
  __shared__ int s_kept[2];
  __shared__ int s_total;
  constexpr int NW = NT / WAVE;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  const int b = blockIdx.x;
  const int N = B + 1;
  const int W = (N + 63) / 64;
  const int Kk = K * k;
  const int R = min(P, kRankMax);
  double* qtab = reinterpret_cast<double*>(smem);  // [Kk] candidate probabilities
  double* gs_a = qtab + Kk;                        // [B] best list, two buffers
  double* gs_b = gs_a + B;
  double* Cs = gs_b + B;                           // [P] candidates of one depth
  double* Ls = Cs + P;                             // [B] the depth's level order; next parents
  uint64_t* gm_a = reinterpret_cast<uint64_t*>(Ls + B);
  uint64_t* gm_b = gm_a + B;
  uint32_t* Ck = reinterpret_cast<uint32_t*>(gm_b + B);  // [P] parent << 16 | rank
  uint32_t* Lk = Ck + P;                                 // [B]
  int* rk = reinterpret_cast<int*>(Lk + B);              // [R] ranks
  int* ttab = rk + R;                                    // [Kk]
  int* rowpar = ttab + Kk;                               // [N]
  int* flat = rowpar + N;                                // [N]
  int* dcnt = flat + N;                                  // [K + 2]

  for (int i = tid; i < Kk; i += NT) {
    qtab[i] = fq[(int64_t)b * Kk + i];
    ttab[i] = ftok[(int64_t)b * Kk + i];
  }
  for (int i = tid; i < R; i += NT) rk[i] = 0;
  if (tid == 0) {
    Ls[0] = 1.0;  // the root, sole parent of depth 1
    s_kept[0] = s_kept[1] = 0;
  }
  __syncthreads();

  double* Gs = gs_a;
  double* Gs_n = gs_b;
  uint64_t* Gm = gm_a;
  uint64_t* Gm_n = gm_b;
  int g = 0, m_par = 1;
  bool have_kappa = false;
  double kappa = 0.0;
  for (int d = 1; d <= K && B > 0; ++d) {
    const double* qd = qtab + (d - 1) * k;
    // ---- candidates: a prefix of every parent's children
    // children of parent i (score si) that pass form a prefix (scores fall
    // with the rank); the q values are read eight at a time
    auto count_children = [&](int i, double si, int lim) {
      int cnt = 0;
      for (int c0 = 0; c0 < k; c0 += 8) {
        double qq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) qq[u] = qd[min(c0 + u, k - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          cnt += (c0 + u < lim && (!have_kappa || si * qq[u] > kappa)) ? 1 : 0;
        if (!__any(cnt == c0 + 8 && c0 + 8 < lim)) break;
      }
      return cnt;
    };
    auto write_children = [&](int i, double si, int cnt, int off) {
      for (int c0 = 0; c0 < cnt; c0 += 8) {
        double qq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) qq[u] = qd[min(c0 + u, k - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (c0 + u < cnt) {
            Cs[off + c0 + u] = si * qq[u];
            Ck[off + c0 + u] = ((uint32_t)i << 16) | (uint32_t)(c0 + u);
          }
      }
    };
    int total = 0;
    if (m_par <= WAVE) {
      // up to 64 parents: wave 0 alone, with a wave-level scan, so that one
      // barrier publishes the list and its length
      if (wave == 0) {
        const int i = lane;
        const double si = i < m_par ? Ls[i] : 0.0;
        const int cnt = count_children(i, si, i < m_par ? min(k, B / (i + 1)) : 0);
        const int incl = wave_scan_add_dpp(cnt);
        write_children(i, si, cnt, incl - cnt);
        if (lane == WAVE - 1) s_total = incl;
      }
      __syncthreads();
      total = s_total;
      if (total == 0) break;
      // s_kept[(d + 1) & 1] was last read (as m_par) before this barrier;
      // the next depth's merge, which counts into it, is barriers away
      if (tid == 0) s_kept[(d + 1) & 1] = 0;
    } else {
      for (int i0 = 0; i0 < m_par; i0 += NT) {
        const int i = i0 + tid;
        const double si = i < m_par ? Ls[i] : 0.0;
        const int cnt = count_children(i, si, i < m_par ? min(k, B / (i + 1)) : 0);
        int tot;
        const int off = total + block_excl_scan<NT>(cnt, wsum, tot);
        write_children(i, si, cnt, off);
        total += tot;
      }
      if (total == 0) break;
      if (tid == 0) s_kept[(d + 1) & 1] = 0;
      __syncthreads();
    }
    const int l = min(total, B);
    if (total <= kRankMax) {
      // ---- level order by rank: wave w counts over its slice of the list
      const int slice = (total + NW - 1) / NW;
      const int i_lo = wave * slice, i_hi = min(total, i_lo + slice);
      for (int j0 = 0; j0 < total; j0 += WAVE) {
        const int j = min(j0 + lane, total - 1);
        const double xs = Cs[j];
        const uint32_t xk = Ck[j];
        int ahead = 0;
        for (int i0 = i_lo; i0 < i_hi; i0 += 8) {
          double ys[8];
          uint32_t yk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = min(i0 + u, i_hi - 1);
            ys[u] = Cs[i];
            yk[u] = Ck[i];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            ahead += (i0 + u < i_hi) &
                     ((int)(ys[u] > xs) | ((int)(ys[u] == xs) & (int)(yk[u] < xk)));
        }
        if (j0 + lane < total && ahead > 0) atomicAdd(&rk[j], ahead);
      }
      __syncthreads();
      for (int j = tid; j < total; j += NT) {
        const int r = rk[j];
        rk[j] = 0;
        if (r < l) {
          Ls[r] = Cs[j];
          Lk[r] = Ck[j];
        }
      }
    } else {
      const int Pn = pow2ceil(total);
      for (int t = total + tid; t < Pn; t += NT) {
        Cs[t] = -1.0;
        Ck[t] = 0xFFFFFFFFu;
      }
      __syncthreads();
      bitonic_sort<NT, uint32_t>(Cs, Ck, Pn);
      for (int j = tid; j < l; j += NT) {
        Ls[j] = Cs[j];
        Lk[j] = Ck[j];
      }
    }
    __syncthreads();

    // ---- merge into the best list: items 0..g-1 are the best list, g..g+l-1
    // the depth's list
    int last_kept = 0;
    for (int t = tid; t < g + l; t += NT) {
      if (t < g) {
        const double x = Gs[t];
        const int np = t + count_ahead(Ls, l, x, false);
        if (np < B) {
          Gs_n[np] = x;
          Gm_n[np] = Gm[t];
        }
      } else {
        const int c = t - g;
        const double x = Ls[c];
        const int np = c + count_ahead(Gs, g, x, true);
        if (np < B) {
          Gs_n[np] = x;
          Gm_n[np] = ((uint64_t)d << 48) | ((uint64_t)c << 32) | (uint64_t)Lk[c];
          last_kept = c + 1;  // kept candidates are a prefix of the level order
        }
      }
    }
    last_kept = __builtin_amdgcn_readlane(wave_scan_max_dpp(last_kept), WAVE - 1);
    if (lane == 0 && last_kept > 0) atomicMax(&s_kept[d & 1], last_kept);
    __syncthreads();
    g = min(B, g + l);
    if (g == B) {
      have_kappa = true;
      kappa = Gs_n[B - 1];
    }
    double* ts = Gs;
    Gs = Gs_n;
    Gs_n = ts;
    uint64_t* tm = Gm;
    Gm = Gm_n;
    Gm_n = tm;
    m_par = s_kept[d & 1];  // the kept depth-d nodes, Ls[0..m_par), parent the next depth
    if (m_par == 0) break;
  }

  // ---- epilogue: rows in best-first order, parents, ancestors ----
  const int n = g + 1;
  for (int dd = tid; dd < K + 2; dd += NT) dcnt[dd] = 0;
  __syncthreads();
  for (int p = tid; p < g; p += NT) atomicAdd(&dcnt[meta_depth(Gm[p])], 1);
  __syncthreads();
  if (wave == 0) {
    // exclusive prefix over the K + 2 depth counts, two per lane:
    // dcnt[dd] becomes the offset of depth dd in `flat`
    static_assert(TV_MAX_POSITIONS + 2 <= 2 * WAVE, "two depth counts per lane");
    const int e0 = 2 * lane, e1 = e0 + 1;
    const int c0 = e0 < K + 2 ? dcnt[e0] : 0, c1 = e1 < K + 2 ? dcnt[e1] : 0;
    const int ex = wave_scan_add_dpp(c0 + c1) - (c0 + c1);
    if (e0 < K + 2) dcnt[e0] = ex;
    if (e1 < K + 2) dcnt[e1] = ex + c0;
  }
  __syncthreads();
  for (int p = tid; p < g; p += NT) {
    const uint64_t mm = Gm[p];
    flat[dcnt[meta_depth(mm)] + meta_pos(mm)] = p + 1;
  }
  __syncthreads();
  const int64_t rb = (int64_t)b * N;
  const int L = ctx_len[b];
  for (int j = tid; j < N; j += NT) {
    int pa = -1, to = -1, de = -1, po = -1;
    double sc = 0.0;
    if (j == 0) {
      to = root_token[b];
      de = 0;
      po = L;
      sc = 1.0;
    } else if (j < n) {
      const uint64_t mm = Gm[j - 1];
      const int dd = meta_depth(mm);
      pa = dd == 1 ? 0 : flat[min(dcnt[dd - 1] + meta_parent(mm), N - 1)];
      to = ttab[(dd - 1) * k + meta_rank(mm)];
      de = dd;
      po = L + dd;
      sc = Gs[j - 1];
    }
    rowpar[j] = pa;
    parent[rb + j] = pa;
    token[rb + j] = to;
    depth[rb + j] = de;
    pos[rb + j] = po;
    score[rb + j] = sc;
  }
  if (tid == 0) n_nodes[b] = n;
  __syncthreads();
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
// cost-aware tree size (TAPS sec. 3.2 and sec. 4.1, third stage): keep the
// best-first prefix of n* draft nodes, n* = the smallest n maximising
// (1 + S_n) / c[n], S_n = s_1 + ... + s_n summed left to right in fp64.
// One wave per sequence: the prefix sums are made in order (a uniform
// chain over the lanes' scores), then each lane rates its sizes and the
// best is found over the lanes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(WAVE) void k_tree_budget(const double* __restrict__ score,
                                                     const int* __restrict__ n_nodes,
                                                     const double* __restrict__ cost, int N,
                                                     int* n_out) {
  constexpr int NC = 16;  // 64-row chunks of a tree of up to 1024 rows
  __shared__ double S[1024];
  const int b = blockIdx.x, lane = lane_id();
  // every load leaves at once: the scores and costs of rows below N exist
  // whatever n_nodes says (chunk k holds scores 1 + 64 k + lane, costs
  // 64 k + lane)
  double x[NC], c[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int i = 1 + 64 * k + lane, m = 64 * k + lane;
    x[k] = i < N ? score[(int64_t)b * N + i] : 0.0;
    c[k] = m < N ? cost[m] : 1.0;
  }
  const int n = n_nodes[b];
  if (n < 1 || n > N) {
    if (lane == 0) n_out[b] = n;
    return;
  }
  // S_i = S_{i-1} + s_i in order: a uniform chain over the lanes' scores
  double run = 0.0;
  if (lane == 0) S[0] = 0.0;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int i0 = 1 + 64 * k;
    if (i0 < n) {
      const int m = min(WAVE, n - i0);
      double mine = 0.0;
      for (int j = 0; j < m; ++j) {
        run = run + readlane_d(x[k], j);
        if (lane == j) mine = run;
      }
      if (lane < m) S[i0 + lane] = mine;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // each lane rates its sizes m = 64 k + lane (ascending, so a strict
  // improvement keeps the smallest size on ties), then the wave takes the
  // largest ratio and, among equal ratios, the smallest size.  Ratios are
  // positive, so their bit patterns order as the values do.
  double best_r = -1.0;
  int best_n = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int m = 64 * k + lane;
    if (m < n) {
      const double r = (1.0 + S[m]) / c[k];
      if (r > best_r) {
        best_r = r;
        best_n = m;
      }
    }
  }
  const uint64_t key = best_r > 0.0 ? __builtin_bit_cast(uint64_t, best_r) : 0ull;
  const uint64_t top = ~wave_min_u64(~key);
  const uint64_t bn = wave_min_u64(key == top ? (uint64_t)best_n : ~0ull);
  if (lane == 0) n_out[b] = (int)bn + 1;
}

// A tree of capacity N holding only its root (row 0), in the row layout of
// the build: the start of a layer-wise build.
__global__ __launch_bounds__(kBuildNT) void k_tree_root(
    const int* __restrict__ root_token, const int* __restrict__ ctx_len, int N,
    int* __restrict__ parent, int* __restrict__ token, int* __restrict__ depth,
    int* __restrict__ pos, double* __restrict__ score, uint64_t* __restrict__ anc,
    int* __restrict__ n_nodes) {
  const int b = blockIdx.x;
  const int Wd = (N + 63) / 64;
  const int64_t rb = (int64_t)b * N;
  const int tk = root_token[b], L = ctx_len[b];
  for (int i = threadIdx.x; i < N; i += kBuildNT) {
    const bool root = i == 0;
    parent[rb + i] = -1;
    token[rb + i] = root ? tk : -1;
    depth[rb + i] = root ? 0 : -1;
    pos[rb + i] = root ? L : -1;
    score[rb + i] = root ? 1.0 : 0.0;
  }
  for (int e = threadIdx.x; e < N * Wd; e += kBuildNT) anc[rb * Wd + e] = e == 0 ? 1ull : 0ull;
  if (threadIdx.x == 0) n_nodes[b] = 1;
}

// ---------------------------------------------------------------------------
// Layer-wise frontier expansion (TreeGraft sec. 3.1, standard single-drafter
// expansion): the candidates of each frontier slot (top-m of its next-token
// row, q desc) become children appended in slot, then rank order; the next
// frontier is the W best new rows by (score desc, row asc), found by
// counting.  Parents are existing rows, children new rows, so no row is both
// read and written.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(NT) void k_expand(
    const int* __restrict__ ftok, const double* __restrict__ fq, int W, int m, int N,
    const int* __restrict__ ctx_len, const int* __restrict__ frontier, int* __restrict__ parent,
    int* __restrict__ token, int* __restrict__ depth, int* __restrict__ pos,
    double* __restrict__ score, uint64_t* __restrict__ anc, int* __restrict__ n_nodes,
    int* __restrict__ next_frontier) {
  __shared__ int s_base[64], s_node[64];
  __shared__ int s_valid;
  __shared__ double s_new[1024];
  const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id();
  const int n0 = n_nodes[b];
  const int Wd = (N + 63) / 64;
  const int64_t rb = (int64_t)b * N;
  if (n0 < 1 || n0 > N) {  // not a tree: left as it is
    for (int w = tid; w < W; w += NT) next_frontier[(int64_t)b * W + w] = -1;
    return;
  }
  if (tid < WAVE) {
    const int f = tid < W ? frontier[(int64_t)b * W + tid] : -1;
    const bool ok = f >= 0 && f < n0;
    const uint64_t bal = __ballot(ok);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    s_base[tid] = ok ? n0 + before * m : -1;
    s_node[tid] = f;
    if (tid == 0) s_valid = __popcll(bal);
  }
  __syncthreads();
  const int n1 = min(N, n0 + s_valid * m);
  const int L = ctx_len[b];
  for (int e = tid; e < W * m; e += NT) {
    const int w = e / m, r = e - w * m;
    const int base = s_base[w];
    if (base < 0 || base + r >= N) continue;
    const int row = base + r, f = s_node[w];
    const int64_t ci = ((int64_t)b * W + w) * m + r;
    const double sc = score[rb + f] * fq[ci];
    const int d = depth[rb + f] + 1;
    parent[rb + row] = f;
    token[rb + row] = ftok[ci];
    depth[rb + row] = d;
    pos[rb + row] = L + d;
    score[rb + row] = sc;
    for (int j = 0; j < Wd; ++j)
      anc[(rb + row) * Wd + j] =
          anc[(rb + f) * Wd + j] | (j == row / 64 ? 1ull << (row % 64) : 0ull);
    s_new[row - n0] = sc;
  }
  __syncthreads();
  const int nn = n1 - n0;
  for (int e = tid; e < nn; e += NT) {
    const double x = s_new[e];
    int rank = 0;
    for (int j0 = 0; j0 < nn; j0 += 8) {
      double y[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) y[q] = s_new[min(j0 + q, nn - 1)];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q;
        rank += (j < nn && (y[q] > x || (y[q] == x && j < e))) ? 1 : 0;
      }
    }
    if (rank < W) next_frontier[(int64_t)b * W + rank] = n0 + e;
  }
  for (int w = nn + tid; w < W; w += NT) next_frontier[(int64_t)b * W + w] = -1;
  if (tid == 0) n_nodes[b] = n1;
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
  const int N = budget + 1;
  const int Kk = K * topk;
  const int R = std::min(p.P, kRankMax);
  p.select_lds = (size_t)8 * (Kk + 3 * (size_t)budget + p.P) + (size_t)16 * budget +
                 (size_t)4 * (p.P + budget + R + Kk + 2 * (size_t)N + K + 2);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.off_cval = take((size_t)p.rows * p.C * topk * sizeof(float));
  p.off_cid = take((size_t)p.rows * p.C * topk * sizeof(int));
  p.off_ftok = take((size_t)p.rows * topk * sizeof(int));
  p.off_fq = take((size_t)p.rows * topk * sizeof(double));
  p.off_rowrec = take((size_t)p.rows * kRowRec * sizeof(uint64_t));
  p.workspace = off;
  return p;
}

// Top-k, q = W / Z and ranks of p.rows logit rows into ftok/fq.
template <typename T>
static void launch_row_topk(const BuildPlan& p, const T* logits, int V, int k, float inv_t,
                            char* w, hipStream_t stream) {
  float* cval = reinterpret_cast<float*>(w + p.off_cval);
  int* cid = reinterpret_cast<int*>(w + p.off_cid);
  int* ftok = reinterpret_cast<int*>(w + p.off_ftok);
  double* fq = reinterpret_cast<double*>(w + p.off_fq);
  uint64_t* rowrec = reinterpret_cast<uint64_t*>(w + p.off_rowrec);
  constexpr int E1 = kBuildChunk / kBuildNT;
  const dim3 g1(p.C, (unsigned)p.rows);
  hipLaunchKernelGGL((k_chunk_topk<T, E1>), g1, dim3(kBuildNT), 0, stream, logits, V, p.C,
                     p.chunk, k, cval, cid, rowrec);
  hipLaunchKernelGGL((k_chunk_z<T>), g1, dim3(kBuildNT), 0, stream, logits, V, p.C, p.chunk, k,
                     inv_t, cval, cid, rowrec, ftok, fq);
}

// The selection's lists live in dynamic LDS, beyond 64 KB for large budgets
// (gfx950 gives a workgroup up to 160 KB once the kernel allows it): the
// limit is raised once per device and kernel, to the largest the host's
// checks admit (kMaxSelectLds), outside the per-call path.
template <int NT>
static hipError_t allow_select_lds(size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  static std::atomic<int> done[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<int>& flag = done[dev & 63];
  if (flag.load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select<NT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxSelectLds);
  if (e == hipSuccess) flag.store(1, std::memory_order_release);
  return e;
}

hipError_t launch_build(const BuildPlan& p, const void* draft, bool bf16, int batch, int K,
                        int V, int topk, int budget, float inv_t, const int* root_token,
                        const int* ctx_len, int* parent, int* token, int* depth, int* pos,
                        double* score, uint64_t* anc, int* n_nodes, void* ws,
                        hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  int* ftok = reinterpret_cast<int*>(w + p.off_ftok);
  double* fq = reinterpret_cast<double*>(w + p.off_fq);
  if (bf16)
    launch_row_topk<uint16_t>(p, static_cast<const uint16_t*>(draft), V, topk, inv_t, w, stream);
  else
    launch_row_topk<float>(p, static_cast<const float*>(draft), V, topk, inv_t, w, stream);
  // one workgroup per sequence; larger budgets have longer candidate lists,
  // whose counting passes gain from more waves (measured: 256 threads up to
  // budget 127, 512 up to 511, then 1024)
#define TV_SELECT(NT)                                                                          \
  do {                                                                                         \
    const hipError_t e = allow_select_lds<NT>(p.select_lds);                                   \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((k_select<NT>), dim3(batch), dim3(NT), p.select_lds, stream, ftok, fq,  \
                       K, topk, budget, p.P, root_token, ctx_len, parent, token, depth, pos,    \
                       score, anc, n_nodes);                                                   \
  } while (0)
  if (budget < 128)
    TV_SELECT(256);
  else if (budget < 512)
    TV_SELECT(512);
  else
    TV_SELECT(1024);
#undef TV_SELECT
  return hipGetLastError();
}

hipError_t launch_tree_expand(const BuildPlan& p, const void* logits, bool bf16, int batch, int W,
                              int V, int m, float inv_t, int N, const int* ctx_len,
                              const int* frontier, int* parent, int* token, int* depth, int* pos,
                              double* score, uint64_t* anc, int* n_nodes, int* next_frontier,
                              void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  int* ftok = reinterpret_cast<int*>(w + p.off_ftok);
  double* fq = reinterpret_cast<double*>(w + p.off_fq);
  // the frontier slots' rows take the place of the draft positions
  if (bf16)
    launch_row_topk<uint16_t>(p, static_cast<const uint16_t*>(logits), V, m, inv_t, w, stream);
  else
    launch_row_topk<float>(p, static_cast<const float*>(logits), V, m, inv_t, w, stream);
  hipLaunchKernelGGL((k_expand<kBuildNT>), dim3(batch), dim3(kBuildNT), 0, stream, ftok, fq, W, m,
                     N, ctx_len, frontier, parent, token, depth, pos, score, anc, n_nodes,
                     next_frontier);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Structural check of caller-supplied trees (PTD sec. 3.1: every node but the
// root has one parent, and a node's ancestors precede it).  status[b] = 0 for
// a well-formed tree, 1 for n_nodes outside [1, N], else 2 + the first row
// that breaks a rule: parent[0] = -1, 0 <= parent[i] < i for 1 <= i < n,
// and, when depth is given, depth[0] = 0 and depth[i] = depth[parent[i]] + 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBuildNT) void k_tree_check(const int* __restrict__ parent,
                                                        const int* __restrict__ depth,
                                                        const int* __restrict__ n_nodes, int N,
                                                        int* __restrict__ status) {
  __shared__ uint64_t wmin[kBuildNT / WAVE];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = n_nodes[b];
  if (n < 1 || n > N) {
    if (tid == 0) status[b] = 1;
    return;
  }
  const int64_t rb = (int64_t)b * N;
  int first = 0x7fffffff;
  for (int i = tid; i < n && first == 0x7fffffff; i += kBuildNT) {
    const int p = parent[rb + i];
    bool ok = i == 0 ? p == -1 : (p >= 0 && p < i);
    if (ok && depth) ok = i == 0 ? depth[rb] == 0 : depth[rb + i] == depth[rb + p] + 1;
    if (!ok) first = i;
  }
  const uint64_t m = wave_min_u64((uint64_t)(uint32_t)first);
  if (lane_id() == 0) wmin[tid / WAVE] = m;
  __syncthreads();
  if (tid == 0) {
    uint64_t f = wmin[0];
    for (int w = 1; w < kBuildNT / WAVE; ++w) f = umin64(f, wmin[w]);
    status[b] = f == 0x7fffffffull ? 0 : 2 + (int)f;
  }
}

hipError_t launch_tree_check(const int* parent, const int* depth, const int* n_nodes, int batch,
                             int N, int* status, hipStream_t stream) {
  hipLaunchKernelGGL(k_tree_check, dim3(batch), dim3(kBuildNT), 0, stream, parent, depth,
                     n_nodes, N, status);
  return hipGetLastError();
}

hipError_t launch_tree_root(const int* root_token, const int* ctx_len, int batch, int N,
                            int* parent, int* token, int* depth, int* pos, double* score,
                            uint64_t* anc, int* n_nodes, hipStream_t stream) {
  hipLaunchKernelGGL(k_tree_root, dim3(batch), dim3(kBuildNT), 0, stream, root_token, ctx_len, N,
                     parent, token, depth, pos, score, anc, n_nodes);
  return hipGetLastError();
}

hipError_t launch_tree_budget(const double* score, const int* n_nodes, const double* cost,
                              int batch, int N, int* n_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_tree_budget, dim3(batch), dim3(WAVE), 0, stream, score, n_nodes, cost, N,
                     n_out);
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
