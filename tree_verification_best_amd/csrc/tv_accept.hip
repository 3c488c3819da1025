// tv_accept.hip -- the acceptance walk of one verification round on gfx950.
//
// Primer ("acceptance and rejection"): greedy verification keeps the drafts
// the target agrees with and substitutes the target's token at the first
// disagreement; sampled verification accepts a draft with min(1, p/q) and,
// at the first rejection, draws from the normalised residual (p - q)+.  For
// a tree of deterministic candidates the proposal of each child is a point
// mass, so the residual after rejecting token t is p with t removed.
//
// Kernels:
//   k_rowmax       grid (chunks, rows)  (max, argmax) of each 4096-token chunk
//                                       of every target row (and draft row in
//                                       DRAFT mode), stored chunk-major
//   k_rowz         grid (chunks, rows)  fixed-point softmax mass of each chunk
//                                       and of its sixteen 256-token segments
//                                       (sampled modes)
//   k_walk         grid (batch)         four waves gather the tree, the row
//                                       statistics, the children's weights and
//                                       every Philox draw into LDS; one wave
//                                       then walks the tree and makes the final
//                                       draw chunk -> segment -> token
//   k_draft_resid  grid (chunks, batch) DRAFT rejection: chunk sums of the
//                                       residual (p - q)+ of the rejected node
//   k_draft_pick   grid (batch)         DRAFT rejection: the residual draw
// The passes read every row; the walk only ever visits rows < n_nodes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

constexpr int kAccNT = 256;
constexpr int kAccE = kAcceptChunk / kAccNT;  // 16 tokens per thread and chunk
constexpr int kSeg = 256;                     // tokens per segment of the final draw
constexpr int kSegs = kAcceptChunk / kSeg;    // 16 segments per chunk
constexpr int kMaxN = 1024;                   // rows per sequence
constexpr int kMaxDraftRows = 64;             // drafter positions (DRAFT proposal)
constexpr int kMaxChunks = 64;                // chunks per row (V <= 2^18)

enum WalkMode { kGreedy = 0, kPointMass = 1, kDraft = 2 };

template <typename T>
__device__ __forceinline__ const T* row_ptr(const T* target, const T* draft, int64_t r,
                                            int64_t trows, int V) {
  return r < trows ? target + r * (int64_t)V : draft + (r - trows) * (int64_t)V;
}

// orders LDS traffic between the lanes of one wave (LDS operations of a wave
// execute in issue order; this keeps the compiler from reordering them)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Vector loads of a 4096-token chunk: thread t holds tokens
// [base + t*16, base + t*16 + 16) (16 consecutive tokens, ids ascending).
// fp32 rows load 4 x 16 bytes, bf16 rows 2 x 16 bytes, all issued before use.
// Tokens past the end of the row are -inf.
template <typename T>
struct ChunkLoad;
template <>
struct ChunkLoad<float> {
  static __device__ __forceinline__ void load(const float* p, int base, int V, float (&x)[16]) {
    const int i0 = base + (int)threadIdx.x * 16;
    if (i0 + 16 <= V && (V & 3) == 0) {
      float4 a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const float4*>(p + i0 + 4 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[4 * j] = a[j].x;
        x[4 * j + 1] = a[j].y;
        x[4 * j + 2] = a[j].z;
        x[4 * j + 3] = a[j].w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = i0 + j < V ? p[i0 + j] : -__builtin_inff();
    }
  }
};
template <>
struct ChunkLoad<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, int base, int V,
                                              float (&x)[16]) {
    const int i0 = base + (int)threadIdx.x * 16;
    if (i0 + 16 <= V && (V & 7) == 0) {
      uint4 a[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) a[j] = *reinterpret_cast<const uint4*>(p + i0 + 8 * j);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w[4] = {a[j].x, a[j].y, a[j].z, a[j].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          x[8 * j + 2 * h] = __builtin_bit_cast(float, w[h] << 16);
          x[8 * j + 2 * h + 1] = __builtin_bit_cast(float, w[h] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        x[j] = i0 + j < V ? bf16_to_f32(p[i0 + j]) : -__builtin_inff();
    }
  }
};

// four consecutive tokens [v0, v0 + 4) of a row; -inf past the end
template <typename T>
__device__ __forceinline__ void load4(const T* p, int v0, int V, float (&x)[4]);
template <>
__device__ __forceinline__ void load4(const float* p, int v0, int V, float (&x)[4]) {
  if (v0 + 4 <= V && (V & 3) == 0) {
    const float4 a = *reinterpret_cast<const float4*>(p + v0);
    x[0] = a.x;
    x[1] = a.y;
    x[2] = a.z;
    x[3] = a.w;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = v0 + q < V ? p[v0 + q] : -__builtin_inff();
  }
}
template <>
__device__ __forceinline__ void load4(const uint16_t* p, int v0, int V, float (&x)[4]) {
  if (v0 + 4 <= V && (V & 3) == 0) {
    const uint2 a = *reinterpret_cast<const uint2*>(p + v0);
    x[0] = __builtin_bit_cast(float, a.x << 16);
    x[1] = __builtin_bit_cast(float, a.x & 0xFFFF0000u);
    x[2] = __builtin_bit_cast(float, a.y << 16);
    x[3] = __builtin_bit_cast(float, a.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = v0 + q < V ? bf16_to_f32(p[v0 + q]) : -__builtin_inff();
  }
}

// (max, argmax lowest id) of each 4096-token chunk of every row, stored at
// [chunk][row].  Rows past n_nodes are read too (they are inside the array)
// and never used.  Without ARG only the maximum is kept.
template <typename T, bool ARG>
__global__ __launch_bounds__(kAccNT) void k_rowmax(const T* __restrict__ target,
                                                  const T* __restrict__ draft, int V,
                                                  int64_t trows, int64_t rows,
                                                  float* __restrict__ cmax,
                                                  int* __restrict__ carg) {
  __shared__ float sv[kAccNT / WAVE];
  __shared__ int si[kAccNT / WAVE];
  const int c = blockIdx.x;
  const int64_t r = blockIdx.y;
  const T* p = row_ptr(target, draft, r, trows, V);
  const int base = c * kAcceptChunk;
  float x[16];
  ChunkLoad<T>::load(p, base, V, x);
  float bv = x[0];
  int bi = base + (int)threadIdx.x * 16;
  if (ARG) {
#pragma unroll
    for (int j = 1; j < 16; ++j)
      if (x[j] > bv) {  // strict: the lowest id among equal values stays
        bv = x[j];
        bi = base + (int)threadIdx.x * 16 + j;
      }
    if (bi >= V) bi = 0x7fffffff;
    wave_argmax(bv, bi);
  } else {
#pragma unroll
    for (int j = 1; j < 16; ++j) bv = fmaxf(bv, x[j]);
    bv = wave_max_f(bv);
  }
  if (lane_id() == 0) {
    sv[threadIdx.x / WAVE] = bv;
    si[threadIdx.x / WAVE] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kAccNT / WAVE; ++w) {
      if (ARG) {
        if (vi_better(sv[w], si[w], bv, bi)) {
          bv = sv[w];
          bi = si[w];
        }
      } else {
        bv = fmaxf(bv, sv[w]);
      }
    }
    cmax[(int64_t)c * rows + r] = bv;
    if (ARG) carg[(int64_t)c * rows + r] = bi;
  }
}

// Fixed-point softmax mass of each chunk (at [chunk][row]) and of each of its
// 256-token segments (at [row][chunk][segment]).  The chunk's logits are
// loaded first; the row maximum (from the chunk maxima) arrives while they
// are in flight.  A segment is the 16 lanes of one DPP row.
template <typename T>
__global__ __launch_bounds__(kAccNT) void k_rowz(const T* __restrict__ target,
                                                const T* __restrict__ draft, int V, int C,
                                                int64_t trows, int64_t rows, float inv_t,
                                                const float* __restrict__ cmax,
                                                uint64_t* __restrict__ cz,
                                                uint64_t* __restrict__ cseg) {
  __shared__ float s_m;
  __shared__ uint64_t wsum[kAccNT / WAVE];
  const int c = blockIdx.x;
  const int64_t r = blockIdx.y;
  const int lane = lane_id();
  const T* p = row_ptr(target, draft, r, trows, V);
  const int base = c * kAcceptChunk;
  float x[16];
  ChunkLoad<T>::load(p, base, V, x);
  if (threadIdx.x < WAVE) {
    float m = -__builtin_inff();
    for (int j = lane; j < C; j += WAVE) m = fmaxf(m, cmax[(int64_t)j * rows + r]);
    m = wave_max_f(m);
    if (lane == 0) s_m = m;
  }
  __syncthreads();
  const float m = s_m;
  uint64_t acc = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc += weight(x[j], m, inv_t);  // -inf padding weighs 0
  // inclusive sums within each row of 16 lanes: lane 15 of a row holds the
  // mass of its segment
  acc += dpp_u64<0x111, 0xF>(acc);
  acc += dpp_u64<0x112, 0xF>(acc);
  acc += dpp_u64<0x114, 0xF>(acc);
  acc += dpp_u64<0x118, 0xF>(acc);
  if ((lane & 15) == 15) cseg[((int64_t)r * C + c) * kSegs + threadIdx.x / 16] = acc;
  const uint64_t wt = readlane_u64(acc, 15) + readlane_u64(acc, 31) + readlane_u64(acc, 47) +
                      readlane_u64(acc, 63);
  if (lane == 0) wsum[threadIdx.x / WAVE] = wt;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t z = 0;
    for (int w = 0; w < kAccNT / WAVE; ++w) z += wsum[w];
    cz[(int64_t)c * rows + r] = z;
  }
}

// ---------------------------------------------------------------------------
// walk
// ---------------------------------------------------------------------------
// DRAFT rejection handed from the walk to the residual kernels
struct DraftPending {
  int flag, u, dd, len;
  float mu, mq;
  uint64_t zu, zq, d0, d1;
};

// A child's acceptance weight with its token, packed for the exclusion
// passes: bit 63 = token inside the vocabulary, bits 18..62 = weight
// (at most 2^44), bits 0..17 = token.
__device__ __forceinline__ uint64_t pack_excl(bool valid, uint64_t w, int t) {
  return valid ? (1ull << 63) | (w << 18) | (uint64_t)(uint32_t)t : 0ull;
}
__device__ __forceinline__ bool excl_valid(uint64_t e) { return (e >> 63) != 0; }
__device__ __forceinline__ uint64_t excl_w(uint64_t e) { return (e >> 18) & ((1ull << 45) - 1); }
__device__ __forceinline__ int excl_t(uint64_t e) { return (int)(e & 0x3FFFFu); }

struct WalkShared {
  int par[kMaxN], tkn[kMaxN];
  int off[kMaxN + 1];  // children per node, then their offsets (CSR, row order)
  int kids[kMaxN];     // gather: owner of each CSR entry; walk: children of u
  float rmax[kMaxN];   // row maximum
  union {
    int rarg[kMaxN];  // greedy: row argmax, lowest id on ties
    struct {
      uint64_t rz[kMaxN];    // row mass Z
      uint64_t wc[kMaxN];    // weight of node c's token in its parent's row
      uint64_t draw[kMaxN];  // word 0 of the acceptance draw of each CSR entry
    } s;
  } u;
  union {
    uint64_t kex[kMaxN];  // point mass: packed (token, effective weight) of u's children
    double qt[kMaxN];     // DRAFT: q of node c's token at its depth (NaN: depth outside [1, K])
  } v;
  uint64_t rd0[kAccNT], rd1[kAccNT];  // final draws of nodes < nres
  float pmax[kAccNT];                 // per-part row statistics
  int parg[kAccNT];
  uint64_t pz[kAccNT];
  float dmax[kMaxDraftRows];
  uint64_t dz[kMaxDraftRows];
  int wtot[kAccNT / WAVE];
};

// floor((hi 2^64 + lo) * Z / 2^128), exact
__device__ __forceinline__ uint64_t scaled_draw(uint64_t hi, uint64_t lo, uint64_t Z) {
  const uint64_t h0 = hi * Z, h1 = __umul64hi(hi, Z);
  const uint64_t l1 = __umul64hi(lo, Z);
  const uint64_t s0 = h0 + l1;
  return h1 + (s0 < h0 ? 1ull : 0ull);
}

template <typename T, int MODE>
__global__ __launch_bounds__(kAccNT) void k_walk(
    const T* __restrict__ target, const T* __restrict__ draft, int N, int K, int V, int C,
    const int* __restrict__ parent, const int* __restrict__ token,
    const int* __restrict__ depth, const int* __restrict__ n_nodes, float inv_t,
    uint64_t seed, uint64_t round, int max_depth, const float* __restrict__ cmax,
    const int* __restrict__ carg, const uint64_t* __restrict__ cz,
    const uint64_t* __restrict__ cseg, int64_t trows, int64_t rows,
    int* __restrict__ accept_len, int* __restrict__ accepted_nodes,
    int* __restrict__ out_tokens, DraftPending* __restrict__ pend) {
  constexpr bool kSampled = MODE != kGreedy;
  __shared__ WalkShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  const int width = max_depth + 1;
  const int64_t rb = (int64_t)b * N;
  int* acc_nodes = accepted_nodes + (int64_t)b * width;
  int* out_tok = out_tokens + (int64_t)b * width;
  for (int j = tid; j < width; j += kAccNT) {
    acc_nodes[j] = -1;
    out_tok[j] = -1;
  }
  if (MODE == kDraft && tid == 0) pend[b].flag = 0;
  const int n = n_nodes[b];
  if (n < 1 || n > N) {
    if (tid == 0) accept_len[b] = -1;
    return;
  }

  // ---- 1. the tree (kept in registers until the statistics are in) and the
  // row statistics: rows are split into P parts of the chunk list so that
  // every thread has work; lanes of a part hold consecutive rows, so each
  // chunk-major load is coalesced
  int pv[4], tv[4], dv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tid + k * kAccNT;
    const int64_t at = rb + (c < n ? c : 0);
    pv[k] = parent[at];
    tv[k] = token[at];
    dv[k] = MODE == kDraft ? depth[at] : 0;
    if (c >= n) pv[k] = tv[k] = -1;
  }
  for (int j = tid; j <= n; j += kAccNT) sh.off[j] = 0;
  const int nr = n + (MODE == kDraft ? K : 0);
  const int P = min(C, max(1, kAccNT / nr));
  const int RP = kAccNT / P;
  const int part = tid / RP, rr = tid - part * RP;
  for (int r0 = 0; r0 < nr; r0 += RP) {
    const int r = r0 + rr;
    const bool act = part < P && r < nr;
    const int64_t grow = !act ? 0 : (r < n ? rb + r : trows + (int64_t)b * K + (r - n));
    float m = -__builtin_inff();
    int a = 0x7fffffff;
    uint64_t z = 0;
    for (int j0 = part; act && j0 < C; j0 += 16 * P) {
      float mv[16];
      int av[16];
      uint64_t zv[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int j = j0 + q * P;
        const int64_t at = (int64_t)(j < C ? j : 0) * rows + grow;
        mv[q] = cmax[at];
        if (!kSampled) av[q] = carg[at];
        else zv[q] = cz[at];
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (j0 + q * P >= C) break;
        if (!kSampled) {
          if (vi_better(mv[q], av[q], m, a)) {
            m = mv[q];
            a = av[q];
          }
        } else {
          m = fmaxf(m, mv[q]);
          z += zv[q];
        }
      }
    }
    if (part < P) {
      sh.pmax[tid] = m;
      sh.parg[tid] = a;
      sh.pz[tid] = z;
    }
    __syncthreads();
    if (tid < RP && r0 + tid < nr) {
      const int rw = r0 + tid;
      float bm = sh.pmax[tid];
      int ba = sh.parg[tid];
      uint64_t bz = sh.pz[tid];
      for (int q = 1; q < P; ++q) {
        const int i = q * RP + tid;
        if (!kSampled) {
          if (vi_better(sh.pmax[i], sh.parg[i], bm, ba)) {
            bm = sh.pmax[i];
            ba = sh.parg[i];
          }
        } else {
          bm = fmaxf(bm, sh.pmax[i]);
          bz += sh.pz[i];
        }
      }
      if (rw < n) {
        sh.rmax[rw] = bm;
        if (!kSampled) sh.u.rarg[rw] = ba;
        else sh.u.s.rz[rw] = bz;
      } else {
        sh.dmax[rw - n] = bm;
        sh.dz[rw - n] = bz;
      }
    }
    __syncthreads();
  }

  // ---- 2. tree into LDS, children counted, logits of the children's tokens
  float lt[4], lq[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tid + k * kAccNT;
    if (c < n) {
      sh.par[c] = pv[k];
      sh.tkn[c] = tv[k];
    }
    const bool child = c >= 1 && c < n && pv[k] >= 0 && pv[k] < n;
    if (kSampled && child) atomicAdd(&sh.off[pv[k]], 1);
    const bool okt = child && tv[k] >= 0 && tv[k] < V;
    lt[k] = 0.f;
    lq[k] = 0.f;
    if (kSampled) {
      lt[k] = Elem<T>::load(target + (rb + (okt ? pv[k] : 0)) * (int64_t)V, okt ? tv[k] : 0);
      if (MODE == kDraft) {
        const bool okq = okt && dv[k] >= 1 && dv[k] <= K;
        lq[k] = Elem<T>::load(draft + ((int64_t)b * K + (okq ? dv[k] - 1 : 0)) * (int64_t)V,
                              okq ? tv[k] : 0);
      }
    }
  }
  __syncthreads();

  if (kSampled) {
    // ---- 3. CSR offsets of the children (exclusive scan of the counts) and
    // the acceptance weights
    int a4[4];
    int s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * tid + q;
      a4[q] = i < n ? sh.off[i] : 0;
      s += a4[q];
    }
    const int incl = wave_incl_scan_i(s);
    if (lane == WAVE - 1) sh.wtot[wave] = incl;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + k * kAccNT;
      if (c >= n) continue;
      const bool child = c >= 1 && pv[k] >= 0 && pv[k] < n;
      const bool okt = child && tv[k] >= 0 && tv[k] < V;
      sh.u.s.wc[c] = okt ? weight(lt[k], sh.rmax[pv[k]], inv_t) : 0ull;
      if (MODE == kDraft) {
        double q = __builtin_nan("");
        if (dv[k] >= 1 && dv[k] <= K)
          q = okt ? (double)weight(lq[k], sh.dmax[dv[k] - 1], inv_t) / (double)sh.dz[dv[k] - 1]
                  : 0.0;
        sh.v.qt[c] = q;
      }
    }
    __syncthreads();
    int ex = incl - s;
    for (int w = 0; w < wave; ++w) ex += sh.wtot[w];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * tid + q;
      if (i < n) sh.off[i] = ex;
      ex += a4[q];
    }
    if (tid == 0) sh.off[n] = sh.wtot[0] + sh.wtot[1] + sh.wtot[2] + sh.wtot[3];
    __syncthreads();

    // ---- 4. every draw the walk can use: the acceptance draw of each
    // (node, child slot) entry, then the final draw of as many nodes as the
    // idle threads of the last pass can take
    for (int u = tid; u < n; u += kAccNT) {
      const int o1 = sh.off[u + 1];
      for (int i = sh.off[u]; i < o1; ++i) sh.kids[i] = u;
    }
    __syncthreads();
  }
  const int E = kSampled ? sh.off[n] : 0;
  const int slots = max(1, (E + kAccNT - 1) / kAccNT) * kAccNT;
  const int nres = kSampled ? min(n, slots - E) : 0;
  if (kSampled) {
    for (int j = tid; j < slots; j += kAccNT) {
      const bool accd = j < E;
      const int uu = accd ? sh.kids[j] : j - E;
      if (accd || uu < n) {
        const uint64_t slot = accd ? (uint64_t)(j - sh.off[uu]) : kResidualSlot;
        const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)uu, slot, seed, 0);
        if (accd) {
          sh.u.s.draw[j] = d.v[0];
        } else {
          sh.rd0[uu] = d.v[0];
          sh.rd1[uu] = d.v[1];
        }
      }
    }
    __syncthreads();
  }

  // ---- the walk: one wave, LDS only except the final draw
  if (wave != 0) return;
  const uint64_t lt_mask = (1ull << lane) - 1ull;

  // children of u in row order into sh.kids[0..nk)
  auto list_children = [&](int u, int nk) {
    int found = 0;
    for (int base = 1; found < nk && base < n; base += 4 * WAVE) {
      int pq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = base + q * WAVE + lane;
        pq[q] = sh.par[c < n ? c : 0];
        if (c >= n) pq[q] = -1;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool is = pq[q] == u;
        const uint64_t bal = __ballot(is);
        if (is) sh.kids[found + __popcll(bal & lt_mask)] = base + q * WAVE + lane;
        found += __popcll(bal);
      }
    }
    wave_lds_sync();
  };
  // f(packed child) for each of the nk children of u, in order (uniform)
  auto for_each_excl = [&](int nk, auto&& f) {
    for (int g = 0; g < nk; g += WAVE) {
      const uint64_t e = sh.v.kex[g + (g + lane < nk ? lane : 0)];
      const int m = min(WAVE, nk - g);
      for (int j = 0; j < m; ++j) f(readlane_u64(e, j));
    }
  };
  // Final draw at u from the target row with the children's tokens removed:
  // chunk, then 256-token segment, then token, each by a wave scan of exact
  // integer sums.  czu: lane j holds the mass of chunk j of row u.
  auto final_draw = [&](int u, uint64_t Z, int nk, uint64_t czu) -> int {
    uint64_t d0, d1;
    if (u < nres) {
      d0 = sh.rd0[u];
      d1 = sh.rd1[u];
    } else {
      const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)u, kResidualSlot, seed, 0);
      d0 = d.v[0];
      d1 = d.v[1];
    }
    const uint64_t R = scaled_draw(d0, d1, Z);
    uint64_t cw = lane < C ? czu : 0ull;
    for_each_excl(nk, [&](uint64_t e) {
      if (excl_valid(e) && (excl_t(e) >> 12) == lane) cw -= excl_w(e);
    });
    const uint64_t incl = wave_incl_scan_u64(cw);
    const uint64_t hit = __ballot(lane < C && incl > R);
    if (!hit) return -1;
    const int cs = __ffsll((unsigned long long)hit) - 1;
    const uint64_t R2 = R - readlane_u64(incl - cw, cs);
    uint64_t sw = cseg[((rb + u) * C + cs) * kSegs + (lane < kSegs ? lane : 0)];
    if (lane >= kSegs) sw = 0;
    for_each_excl(nk, [&](uint64_t e) {
      const int t = excl_t(e);
      if (excl_valid(e) && (t >> 12) == cs && ((t >> 8) & (kSegs - 1)) == lane) sw -= excl_w(e);
    });
    const uint64_t incl2 = wave_incl_scan_u64(sw);
    const uint64_t hit2 = __ballot(lane < kSegs && incl2 > R2);
    if (!hit2) return -1;
    const int ss = __ffsll((unsigned long long)hit2) - 1;
    const uint64_t R3 = R2 - readlane_u64(incl2 - sw, ss);
    const int v0 = cs * kAcceptChunk + ss * kSeg + 4 * lane;
    float x[4];
    load4(target + (rb + u) * (int64_t)V, v0, V, x);
    const float m = sh.rmax[u];
    uint64_t w4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w4[q] = weight(x[q], m, inv_t);
    for_each_excl(nk, [&](uint64_t e) {
      const int t = excl_t(e);
      if (excl_valid(e)) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (t == v0 + q) w4[q] = 0;
      }
    });
    const uint64_t s4 = w4[0] + w4[1] + w4[2] + w4[3];
    const uint64_t incl3 = wave_incl_scan_u64(s4);
    const uint64_t hit3 = __ballot(incl3 > R3);
    if (!hit3) return -1;
    const int L = __ffsll((unsigned long long)hit3) - 1;
    uint64_t run = incl3 - s4;
    int tok = v0 + 3;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      // smallest q with run + w4[0..q] > R3
      uint64_t pre = run;
      for (int k = 0; k <= q; ++k) pre += w4[k];
      if (pre > R3) tok = v0 + q;
    }
    return readlane_i(tok, L);
  };

  if (lane == 0) acc_nodes[0] = 0;
  int u = 0, len = 0, bonus = -1;
  bool err = false, pending = false;
  if (MODE == kGreedy) {
    for (;;) {
      const int a = sh.u.rarg[u];
      int nxt = -1;
      if (len < max_depth) {
        for (int base = 1; base < n && nxt < 0; base += 4 * WAVE) {
          int pq[4], tq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = base + q * WAVE + lane;
            pq[q] = sh.par[c < n ? c : 0];
            tq[q] = sh.tkn[c < n ? c : 0];
            if (c >= n) pq[q] = -1;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint64_t bal = __ballot(pq[q] == u && tq[q] == a);
            if (bal && nxt < 0) nxt = base + q * WAVE + __ffsll((unsigned long long)bal) - 1;
          }
        }
      }
      if (nxt < 0) {
        bonus = a;
        break;
      }
      ++len;
      if (lane == 0) {
        acc_nodes[len] = nxt;
        out_tok[len - 1] = a;
      }
      u = nxt;
    }
  } else if (MODE == kPointMass) {
    for (;;) {
      // chunk masses of row u, for the final draw if every child is rejected
      const uint64_t czu = cz[(int64_t)(lane < C ? lane : 0) * rows + rb + u];
      const int o = sh.off[u];
      const int nk = len < max_depth ? sh.off[u + 1] - o : 0;
      uint64_t Zres = sh.u.s.rz[u];
      int nxt = -1;
      if (nk > 0) {
        list_children(u, nk);
        for (int g = 0; g < nk && nxt < 0; g += WAVE) {
          const int i = g + lane;
          const bool live = i < nk;
          const int c = sh.kids[live ? i : 0];
          const int t = sh.tkn[c];
          const uint64_t w0 = sh.u.s.wc[c];
          const uint64_t d = sh.u.s.draw[o + (live ? i : 0)];
          // a token already tried by an earlier child weighs nothing
          bool dup = false;
          const int m = min(WAVE, nk - g);
          for (int j = 0; j < m - 1; ++j) dup |= (j < lane) && (readlane_i(t, j) == t);
          for (int j = 0; j < g; ++j) dup |= excl_valid(sh.v.kex[j]) && excl_t(sh.v.kex[j]) == t;
          const bool okt = t >= 0 && t < V;
          const uint64_t w = (live && !dup) ? w0 : 0ull;
          if (live) sh.v.kex[i] = pack_excl(okt, w, t);
          const uint64_t incl = wave_incl_scan_u64(w);
          const uint64_t zres = Zres - (incl - w);
          const bool ok = live && (__umul64hi(d, zres) < w);
          const uint64_t bal = __ballot(ok);
          if (bal) nxt = readlane_i(c, __ffsll((unsigned long long)bal) - 1);
          Zres -= readlane_u64(incl, WAVE - 1);
        }
        wave_lds_sync();
      }
      if (nxt >= 0) {
        ++len;
        if (lane == 0) {
          acc_nodes[len] = nxt;
          out_tok[len - 1] = sh.tkn[nxt];
        }
        u = nxt;
        continue;
      }
      bonus = final_draw(u, Zres, nk, czu);
      break;
    }
  } else {  // DRAFT proposal: chains only
    for (;;) {
      const uint64_t czu = cz[(int64_t)(lane < C ? lane : 0) * rows + rb + u];
      const int o = sh.off[u];
      const int nk = len < max_depth ? sh.off[u + 1] - o : 0;
      if (nk > 1) {
        err = true;
        break;
      }
      const uint64_t Zu = sh.u.s.rz[u];
      if (nk == 0) {
        // end of the chain: the emitted token comes from the target row
        bonus = final_draw(u, Zu, 0, czu);
        break;
      }
      list_children(u, 1);
      const int c = sh.kids[0];
      const double qt = sh.v.qt[c];
      if (qt != qt) {  // depth outside [1, K]
        err = true;
        break;
      }
      const int t = sh.tkn[c];
      const double pt = (t >= 0 && t < V) ? (double)sh.u.s.wc[c] / (double)Zu : 0.0;
      const uint64_t d = sh.u.s.draw[o];
      const double u53 = (double)(d >> 11) * 0x1p-53;
      // min(1, p/q): a token the target gives no mass is never accepted
      if (pt > 0.0 && (pt >= qt || u53 < pt / qt)) {
        ++len;
        if (lane == 0) {
          acc_nodes[len] = c;
          out_tok[len - 1] = t;
        }
        u = c;
        continue;
      }
      // rejection: the residual (p - q)+ is drawn by the kernels that follow
      if (lane == 0) {
        const int dd = depth[rb + c];
        DraftPending pd;
        pd.flag = 1;
        pd.u = u;
        pd.dd = dd;
        pd.len = len;
        pd.mu = sh.rmax[u];
        pd.mq = sh.dmax[dd - 1];
        pd.zu = Zu;
        pd.zq = sh.dz[dd - 1];
        if (u < nres) {
          pd.d0 = sh.rd0[u];
          pd.d1 = sh.rd1[u];
        } else {
          const u64x4 dr = philox4x64_10(round, (uint64_t)b, (uint64_t)u, kResidualSlot, seed, 0);
          pd.d0 = dr.v[0];
          pd.d1 = dr.v[1];
        }
        pend[b] = pd;
      }
      pending = true;
      break;
    }
  }
  if (lane == 0) {
    if (err) {
      accept_len[b] = -1;
    } else if (!pending) {
      accept_len[b] = len;
      out_tok[len] = bonus;
    }
  }
}

// ---------------------------------------------------------------------------
// DRAFT rejection: residual weights rint(max(0, p - q) * 2^62) in fp64
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t resid_weight(float x, float y, const DraftPending& pd,
                                                 float inv_t) {
  const double p = (double)weight(x, pd.mu, inv_t) / (double)pd.zu;
  const double q = (double)weight(y, pd.mq, inv_t) / (double)pd.zq;
  const double r = p - q;
  return r > 0.0 ? (uint64_t)__builtin_rint(r * 0x1p62) : 0ull;
}

// chunk sums of the residual of each pending sequence, at [b][chunk]
template <typename T>
__global__ __launch_bounds__(kAccNT) void k_draft_resid(const T* __restrict__ target,
                                                       const T* __restrict__ draft, int N,
                                                       int K, int V, float inv_t,
                                                       const DraftPending* __restrict__ pend,
                                                       uint64_t* __restrict__ rcz) {
  __shared__ uint64_t wsum[kAccNT / WAVE];
  const int c = blockIdx.x, b = blockIdx.y;
  const DraftPending pd = pend[b];
  if (!pd.flag) return;
  const T* prow = target + ((int64_t)b * N + pd.u) * (int64_t)V;
  const T* qrow = draft + ((int64_t)b * K + (pd.dd - 1)) * (int64_t)V;
  const int base = c * kAcceptChunk;
  float x[16], y[16];
  ChunkLoad<T>::load(prow, base, V, x);
  ChunkLoad<T>::load(qrow, base, V, y);
  uint64_t s = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += resid_weight(x[j], y[j], pd, inv_t);
  s = wave_sum_u64(s);
  if (lane_id() == 0) wsum[threadIdx.x / WAVE] = s;
  __syncthreads();
  if (threadIdx.x == 0) rcz[(int64_t)b * kMaxChunks + c] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// Smallest token of chunk `base` whose running sum exceeds R, given the 16
// consecutive weights of each thread (thread t: tokens base + 16t ...).
__device__ int block_pick(const uint64_t (&w)[16], int base, uint64_t R, uint64_t* tsum,
                          int* tok) {
  const int tid = threadIdx.x;
  uint64_t run = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) run += w[j];
  tsum[tid] = run;
  if (tid == 0) *tok = 0x7fffffff;
  __syncthreads();
  if (tid < WAVE) {
    const uint64_t a0 = tsum[4 * tid], a1 = tsum[4 * tid + 1], a2 = tsum[4 * tid + 2],
                   a3 = tsum[4 * tid + 3];
    const uint64_t s4 = a0 + a1 + a2 + a3;
    uint64_t ex = wave_incl_scan_u64(s4) - s4;
    tsum[4 * tid] = ex;
    ex += a0;
    tsum[4 * tid + 1] = ex;
    ex += a1;
    tsum[4 * tid + 2] = ex;
    ex += a2;
    tsum[4 * tid + 3] = ex;
  }
  __syncthreads();
  uint64_t acc = tsum[tid];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc += w[j];
    if (acc > R) {
      atomicMin(tok, base + 16 * tid + j);
      break;
    }
  }
  __syncthreads();
  return *tok;
}

// the residual draw of each pending sequence (the target row itself if the
// residual is empty to rounding)
template <typename T>
__global__ __launch_bounds__(kAccNT) void k_draft_pick(
    const T* __restrict__ target, const T* __restrict__ draft, int N, int K, int V, int C,
    float inv_t, int max_depth, int64_t rows, const uint64_t* __restrict__ cz,
    const DraftPending* __restrict__ pend, const uint64_t* __restrict__ rcz,
    int* __restrict__ accept_len, int* __restrict__ out_tokens) {
  __shared__ uint64_t tsum[kAccNT];
  __shared__ int s_cs, s_tok;
  __shared__ uint64_t s_r;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id();
  const DraftPending pd = pend[b];
  if (!pd.flag) return;
  const int64_t grow = (int64_t)b * N + pd.u;
  if (tid < WAVE) {
    const uint64_t rw = lane < C ? rcz[(int64_t)b * kMaxChunks + lane] : 0ull;
    const uint64_t ZR = wave_sum_u64(rw);
    const bool resid = ZR > 0;
    const uint64_t cw = resid ? rw : (lane < C ? cz[(int64_t)lane * rows + grow] : 0ull);
    const uint64_t R = scaled_draw(pd.d0, pd.d1, resid ? ZR : pd.zu);
    const uint64_t incl = wave_incl_scan_u64(cw);
    const uint64_t hit = __ballot(lane < C && incl > R);
    const int cs = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
    const uint64_t before = cs >= 0 ? readlane_u64(incl - cw, cs) : 0ull;
    if (lane == 0) {
      s_cs = resid ? cs : -2 - cs;  // the target-row draw is marked by a negative code
      s_r = R - before;
    }
  }
  __syncthreads();
  const int code = s_cs;
  const bool resid = code >= 0;
  const int cs = resid ? code : -2 - code;
  int tok = -1;
  if (cs >= 0) {
    const int base = cs * kAcceptChunk;
    float x[16], y[16];
    ChunkLoad<T>::load(target + grow * (int64_t)V, base, V, x);
    uint64_t w[16];
    if (resid) {
      ChunkLoad<T>::load(draft + ((int64_t)b * K + (pd.dd - 1)) * (int64_t)V, base, V, y);
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = resid_weight(x[j], y[j], pd, inv_t);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = weight(x[j], pd.mu, inv_t);
    }
    tok = block_pick(w, base, s_r, tsum, &s_tok);
    if (tok == 0x7fffffff) tok = -1;
  }
  if (tid == 0) {
    const int width = max_depth + 1;
    accept_len[b] = pd.len;
    out_tokens[(int64_t)b * width + pd.len] = tok;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
AcceptPlan accept_plan(int batch, int N, int K, int V, bool sampled, bool draft) {
  AcceptPlan p{};
  p.chunk = kAcceptChunk;
  p.C = (V + p.chunk - 1) / p.chunk;
  p.draft_rows = draft;
  p.rows = (int64_t)batch * N + (draft ? (int64_t)batch * K : 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.off_cmax = take((size_t)p.rows * p.C * sizeof(float));
  p.off_carg = take((size_t)p.rows * p.C * sizeof(int));
  p.off_cz = sampled ? take((size_t)p.rows * p.C * sizeof(uint64_t)) : 0;
  p.off_cseg = sampled ? take((size_t)p.rows * p.C * kSegs * sizeof(uint64_t)) : 0;
  p.off_rcz = draft ? take((size_t)batch * kMaxChunks * sizeof(uint64_t)) : 0;
  p.off_pend = draft ? take((size_t)batch * sizeof(DraftPending)) : 0;
  p.workspace = off;
  return p;
}

template <typename T>
static void launch_accept_t(const AcceptPlan& p, const T* target, const T* draft, int batch,
                            int N, int K, int V, const int* parent, const int* token,
                            const int* depth, const int* n_nodes, bool sampled, float inv_t,
                            bool draft_proposal, uint64_t seed, uint64_t round,
                            int max_depth, int* accept_len, int* accepted_nodes,
                            int* out_tokens, char* w, hipStream_t stream) {
  float* cmax = reinterpret_cast<float*>(w + p.off_cmax);
  int* carg = reinterpret_cast<int*>(w + p.off_carg);
  uint64_t* cz = sampled ? reinterpret_cast<uint64_t*>(w + p.off_cz) : nullptr;
  uint64_t* cseg = sampled ? reinterpret_cast<uint64_t*>(w + p.off_cseg) : nullptr;
  uint64_t* rcz = draft_proposal ? reinterpret_cast<uint64_t*>(w + p.off_rcz) : nullptr;
  DraftPending* pend =
      draft_proposal ? reinterpret_cast<DraftPending*>(w + p.off_pend) : nullptr;
  const int64_t trows = (int64_t)batch * N;
  const dim3 g(p.C, (unsigned)p.rows);
  const dim3 blk(kAccNT);
  if (sampled) {
    hipLaunchKernelGGL((k_rowmax<T, false>), g, blk, 0, stream, target, draft, V, trows,
                       p.rows, cmax, carg);
    hipLaunchKernelGGL((k_rowz<T>), g, blk, 0, stream, target, draft, V, p.C, trows, p.rows,
                       inv_t, cmax, cz, cseg);
  } else {
    hipLaunchKernelGGL((k_rowmax<T, true>), g, blk, 0, stream, target, draft, V, trows, p.rows,
                       cmax, carg);
  }
#define TV_WALK(M)                                                                            \
  hipLaunchKernelGGL((k_walk<T, M>), dim3(batch), blk, 0, stream, target, draft, N, K, V, p.C, \
                     parent, token, depth, n_nodes, inv_t, seed, round, max_depth, cmax, carg, \
                     cz, cseg, trows, p.rows, accept_len, accepted_nodes, out_tokens, pend)
  if (!sampled) {
    TV_WALK(kGreedy);
  } else if (!draft_proposal) {
    TV_WALK(kPointMass);
  } else {
    TV_WALK(kDraft);
    hipLaunchKernelGGL((k_draft_resid<T>), dim3(p.C, batch), blk, 0, stream, target, draft, N,
                       K, V, inv_t, pend, rcz);
    hipLaunchKernelGGL((k_draft_pick<T>), dim3(batch), blk, 0, stream, target, draft, N, K, V,
                       p.C, inv_t, max_depth, p.rows, cz, pend, rcz, accept_len, out_tokens);
  }
#undef TV_WALK
}

hipError_t launch_accept(const AcceptPlan& p, const void* target, const void* draft,
                         bool bf16, int batch, int N, int K, int V, const int* parent,
                         const int* token, const int* depth, const int* n_nodes, bool sampled,
                         float inv_t, bool draft_proposal, uint64_t seed, uint64_t round,
                         int max_depth, int* accept_len, int* accepted_nodes, int* out_tokens,
                         void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  if (bf16)
    launch_accept_t<uint16_t>(p, static_cast<const uint16_t*>(target),
                              static_cast<const uint16_t*>(draft), batch, N, K, V, parent,
                              token, depth, n_nodes, sampled, inv_t, draft_proposal, seed, round,
                              max_depth, accept_len, accepted_nodes, out_tokens, w, stream);
  else
    launch_accept_t<float>(p, static_cast<const float*>(target),
                           static_cast<const float*>(draft), batch, N, K, V, parent, token,
                           depth, n_nodes, sampled, inv_t, draft_proposal, seed, round,
                           max_depth, accept_len, accepted_nodes, out_tokens, w, stream);
  return hipGetLastError();
}

}  // namespace tvk
