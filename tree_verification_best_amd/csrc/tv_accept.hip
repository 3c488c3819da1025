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
//   k_rowmax       grid (chunks, rows)  greedy: (max, argmax) of each
//                                       4096-token chunk of every target row,
//                                       stored chunk-major
//   k_rowstat      grid (J * Cb)        sampled: one pass over every target
//                                       row (and draft row in DRAFT mode) that
//                                       keeps its span of the row in registers
//                                       while the row's maximum is agreed on,
//                                       then the chunks' maxima, fixed-point
//                                       softmax masses and the weight of each
//                                       child's token, chunk-major
//   k_walk         grid (batch)         gathers the tree, the row statistics,
//                                       the children's weights and every Philox
//                                       draw into LDS, decides every node in
//                                       parallel, follows the decisions from the
//                                       root and makes the final draw (chunk,
//                                       then token within the chunk)
//   k_draft_resid  grid (chunks, batch) DRAFT rejection: chunk sums of the
//                                       residual (p - q)+ of the rejected node
//   k_draft_pick   grid (batch)         DRAFT rejection: the residual draw
// The passes read every row; the walk only ever visits rows < n_nodes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

constexpr int kAccNT = 256;
constexpr int kMaxN = 1024;                   // rows per sequence
constexpr int kMaxDraftRows = 64;             // drafter positions (DRAFT proposal)
constexpr int kMaxChunks = 64;                // chunks per row (V <= 2^18)
// the rows' mass accumulators of the sampled row pass are one 256-byte line
// apart, so that the blocks adding to one row do not meet other rows' there
constexpr int kRowzStride = 32;

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
// Vector loads of E * 256 tokens of a row: thread t holds tokens
// [base + t*E, base + t*E + E) (E consecutive tokens, ids ascending), E a
// multiple of 16.  fp32 rows load E/4 x 16 bytes, bf16 rows E/8 x 16 bytes,
// all issued before use.  Tokens past the end of the row are -inf.
template <typename T>
struct ChunkLoad;
template <>
struct ChunkLoad<float> {
  template <int E>
  static __device__ __forceinline__ void load(const float* p, int base, int V, float (&x)[E]) {
    const int i0 = base + (int)threadIdx.x * E;
    if (i0 + E <= V && (V & 3) == 0) {
      float4 a[E / 4];
#pragma unroll
      for (int j = 0; j < E / 4; ++j) a[j] = *reinterpret_cast<const float4*>(p + i0 + 4 * j);
#pragma unroll
      for (int j = 0; j < E / 4; ++j) {
        x[4 * j] = a[j].x;
        x[4 * j + 1] = a[j].y;
        x[4 * j + 2] = a[j].z;
        x[4 * j + 3] = a[j].w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) x[j] = i0 + j < V ? p[i0 + j] : -__builtin_inff();
    }
  }
};
template <>
struct ChunkLoad<uint16_t> {
  template <int E>
  static __device__ __forceinline__ void load(const uint16_t* p, int base, int V,
                                              float (&x)[E]) {
    const int i0 = base + (int)threadIdx.x * E;
    if (i0 + E <= V && (V & 7) == 0) {
      uint4 a[E / 8];
#pragma unroll
      for (int j = 0; j < E / 8; ++j) a[j] = *reinterpret_cast<const uint4*>(p + i0 + 8 * j);
#pragma unroll
      for (int j = 0; j < E / 8; ++j) {
        const uint32_t w[4] = {a[j].x, a[j].y, a[j].z, a[j].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          x[8 * j + 2 * h] = __builtin_bit_cast(float, w[h] << 16);
          x[8 * j + 2 * h + 1] = __builtin_bit_cast(float, w[h] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j)
        x[j] = i0 + j < V ? bf16_to_f32(p[i0 + j]) : -__builtin_inff();
    }
  }
};

// (max, argmax lowest id) of each 4096-token chunk of every row, stored at
// [chunk][row] (greedy mode).  Rows past n_nodes are read too (they are
// inside the array) and never used.
template <typename T>
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
#pragma unroll
  for (int j = 1; j < 16; ++j)
    if (x[j] > bv) {  // strict: the lowest id among equal values stays
      bv = x[j];
      bi = base + (int)threadIdx.x * 16 + j;
    }
  if (bi >= V) bi = 0x7fffffff;
  wave_argmax(bv, bi);
  if (lane_id() == 0) {
    sv[threadIdx.x / WAVE] = bv;
    si[threadIdx.x / WAVE] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kAccNT / WAVE; ++w)
      if (vi_better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    cmax[(int64_t)c * rows + r] = bv;
    carg[(int64_t)c * rows + r] = bi;
  }
}

// Fixed-point softmax mass of the E/16 chunks of 4096 tokens that the block
// holds of row r (x from ChunkLoad at base = cb * E * 256, m: the row
// maximum), stored at cz[c][r] for each chunk c < C.  With the tree given
// (wtg non-null), the block also stores the weight of every child's token
// that falls in its tokens: wtg[b][x] = W of token(x) in the row of
// parent(x); in DRAFT mode (wqg non-null) a draft row's block stores
// wqg[b][x] = W of token(x) in draft row depth(x) - 1.  Ends with a barrier.
// A thread's share of one sequence's tree (nodes 1 + t + 256 k), kept in
// registers by the pipelined row pass, whose blocks take many rows of the
// same sequence: the children of each row's node are then found without
// reloading the tree for every row.
// Each entry packs the node's token (below 2^18) over its parent (below
// 2^10): tok << 10 | parent, all ones for no node.
struct TreeCache {
  int seq, nn;
  uint32_t pt[kMaxN / kAccNT];
};

__device__ __forceinline__ void load_tree(TreeCache& tc, int bb, int N,
                                          const int* __restrict__ parent,
                                          const int* __restrict__ token,
                                          const int* __restrict__ n_nodes) {
  const int64_t o = (int64_t)bb * N;
  tc.seq = bb;
  tc.nn = n_nodes[bb];
#pragma unroll
  for (int k = 0; k < kMaxN / kAccNT; ++k) {
    const int xx = 1 + (int)threadIdx.x + k * kAccNT;
    tc.pt[k] = xx < N ? ((uint32_t)token[o + xx] << 10) | ((uint32_t)parent[o + xx] & 1023u)
                      : 0xFFFFFFFFu;
  }
}

template <typename T, int E, bool CACHE>
__device__ __forceinline__ void chunk_mass(const float (&x)[E], const T* p, int V, int C, int cb,
                                           int64_t r, int64_t trows, int64_t rows, float m,
                                           float inv_t, uint64_t* wsum, uint64_t* cz, int N,
                                           int K, const int* parent, const int* token,
                                           const int* depth, const int* n_nodes,
                                           uint64_t* wtg, uint64_t* wqg, TreeCache& tc) {
  static_assert(E % 16 == 0 && E <= 512, "fp64 partial sums must stay exact");
  constexpr int kSpan = E * kAccNT;
  const int base = cb * kSpan;
  // E weights of at most 2^44 add exactly in fp64; -inf pads weigh 0
  double accd;
  if (inv_t == 1.0f) {
    accd = (double)weight_f<true>(x[0], m, inv_t);
#pragma unroll
    for (int j = 1; j < E; ++j) accd += (double)weight_f<true>(x[j], m, inv_t);
  } else {
    accd = (double)weight_f(x[0], m, inv_t);
#pragma unroll
    for (int j = 1; j < E; ++j) accd += (double)weight_f(x[j], m, inv_t);
  }
  const uint64_t acc = wave_sum_u64((uint64_t)accd);
  if (lane_id() == 0) wsum[threadIdx.x / WAVE] = acc;
  if (wtg) {
    // children whose tokens fall in the block's span (the logit is re-read:
    // the block has just brought it into the cache)
    const bool trow = r < trows;
    if (trow || wqg) {
      const int64_t j = trow ? r : r - trows;
      const int bb = (int)(j / (trow ? N : K));
      const int uu = (int)(j - (int64_t)bb * (trow ? N : K));
      const int64_t o = (int64_t)bb * N;
      if (CACHE && trow) {
        if (tc.seq != bb) load_tree(tc, bb, N, parent, token, n_nodes);
        const int nn = tc.nn;
        if (nn >= 1 && nn <= N && uu < nn) {
#pragma unroll
          for (int k = 0; k < kMaxN / kAccNT; ++k) {
            const int xx = 1 + (int)threadIdx.x + k * kAccNT;
            const int t = (int)(tc.pt[k] >> 10);
            if (xx < nn && (int)(tc.pt[k] & 1023u) == uu && t >= base && t < base + kSpan &&
                t < V)
              wtg[o + xx] = weight(Elem<T>::load(p, t), m, inv_t);
          }
        }
      } else if (const int nn = n_nodes[bb]; nn >= 1 && nn <= N && (!trow || uu < nn)) {
        for (int xx = 1 + (int)threadIdx.x; xx < nn; xx += kAccNT) {
          const bool mine = trow ? parent[o + xx] == uu : depth[o + xx] == uu + 1;
          if (!mine) continue;
          const int t = token[o + xx];
          if (t >= base && t < base + kSpan && t < V)
            (trow ? wtg : wqg)[o + xx] = weight(Elem<T>::load(p, t), m, inv_t);
        }
      }
    }
  }
  __syncthreads();
  // chunk k of the span is held by waves [k * W4, (k + 1) * W4)
  constexpr int kWaves = kAccNT / WAVE, W4 = kWaves / (E / 16);
  if ((int)threadIdx.x < E / 16) {
    const int k = threadIdx.x, c = cb * (E / 16) + k;
    if (c < C) {
      uint64_t z = 0;
      for (int w = k * W4; w < (k + 1) * W4; ++w) z += wsum[w];
      cz[(int64_t)c * rows + r] = z;
    }
  }
  __syncthreads();  // wsum is reused by the block's next row
}

// One pass over the rows for the sampled walks: each logit is read once and
// kept in registers while its row's maximum is agreed on.  A block holds
// E * 256 tokens (E / 16 chunks of 4096) of a row; Cb = ceil(V / (E * 256))
// blocks cover a row.  Block g takes span cb = g % Cb of rows g / Cb,
// g / Cb + J, g / Cb + 2J, ... (J = gridDim.x / Cb groups).  For each row
// the block posts its maximum in the row's slot cb, waits until all Cb
// slots of the row are posted, takes the row maximum and weighs its span
// (chunk_mass).  A block with several rows (J < rows) either loads and posts
// its next row after weighing the current one, or (PIPE) pipelines one row
// deep: the next row's span is loaded during the wait and posted before the
// current span is weighed.
//
// Slots: slot[r * slot_stride + cb] = tag << 32 | bits of the span maximum,
// an agent-scope atomic store; a reader's wave polls the row's Cb slots with
// agent-scope atomic loads until every one carries this call's tag.  The tag
// is 2 * generation + 1, the generation a word of the workspace that the
// walk advances once per call, so slots never need clearing: a slot holds
// zero (a new workspace) or the previous call's tag until it is posted.  One store and one
// load per hand-off, no cache-wide maintenance.  The maxima of the 4096-token
// chunks also go to cmax[c][r] for the walk.
//
// The wait needs the Cb blocks of a group resident together; the host sizes
// the grid within what the device holds at once.  The wait is bounded all
// the same: a block that has polled spin_limit times in vain (other work
// holding the device, say) takes the row maximum from the whole row itself,
// which gives the same value, so the results never depend on the schedule.
// The rows' mass accumulators must be zero at the start: a new workspace is
// zero-filled by its owner, and k_walk, their last reader, returns them to
// zero (so no clearing launch is needed and replays of a captured call find
// them as the first call did).  Each row's slots start on a 256-byte line of
// their own, and each row's mass on another.
template <int E>
__device__ __forceinline__ void post_span_max(const float (&x)[E], float* sv, float* cmax,
                                              uint64_t* slot, int C, int cb, int64_t r,
                                              int64_t rows, int slot_stride, uint32_t tag) {
  float bv = x[0];
#pragma unroll
  for (int j = 1; j < E; ++j) bv = fmaxf(bv, x[j]);
  bv = wave_max_f(bv);
  if (lane_id() == 0) sv[threadIdx.x / WAVE] = bv;
  __syncthreads();
  constexpr int kWaves = kAccNT / WAVE, W4 = kWaves / (E / 16);
  if (threadIdx.x == 0) {
    float all = -__builtin_inff();
    for (int k = 0; k < E / 16; ++k) {
      float ck = sv[k * W4];
      for (int w = k * W4 + 1; w < (k + 1) * W4; ++w) ck = fmaxf(ck, sv[w]);
      const int c = cb * (E / 16) + k;
      if (c < C) cmax[(int64_t)c * rows + r] = ck;
      all = fmaxf(all, ck);
    }
    const uint64_t v = ((uint64_t)tag << 32) | __builtin_bit_cast(uint32_t, all);
    __hip_atomic_store(&slot[r * slot_stride + cb], v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int E, bool PIPE>
__global__ __launch_bounds__(kAccNT) void k_rowstat(const T* __restrict__ target,
                                                   const T* __restrict__ draft, int V, int C,
                                                   int Cb, int64_t trows, int64_t rows,
                                                   float inv_t, float* __restrict__ cmax,
                                                   uint64_t* slot, int slot_stride,
                                                   uint64_t* __restrict__ cz,
                                                   float* __restrict__ rowm, uint64_t* rowz,
                                                   int N, int K,
                                                   const int* __restrict__ parent,
                                                   const int* __restrict__ token,
                                                   const int* __restrict__ depth,
                                                   const int* __restrict__ n_nodes,
                                                   uint64_t* __restrict__ wtg,
                                                   uint64_t* __restrict__ wqg,
                                                   const uint32_t* __restrict__ gen,
                                                   int spin_limit) {
  __shared__ float sv[kAccNT / WAVE];
  __shared__ float sl[kAccNT / WAVE];
  __shared__ uint64_t wsum[kAccNT / WAVE];
  __shared__ float s_m;
  __shared__ int s_late;
  constexpr int kSpan = E * kAccNT;
  const int cb = (int)(blockIdx.x % (unsigned)Cb);
  const int64_t J = gridDim.x / (unsigned)Cb;
  const int lane = lane_id();
  int64_t r = blockIdx.x / (unsigned)Cb;
  if (r >= rows) return;
  // this call's slot tag: odd, so never the zero of a new workspace, and
  // different from the previous call's (the walk advances the generation)
  const uint32_t tag = (gen[0] << 1) | 1u;
  TreeCache tc;
  tc.seq = -1;
  if constexpr (PIPE) {
    // the tree of the first row's sequence, loaded while the row is agreed on
    if (wtg && r < trows) load_tree(tc, (int)(r / N), N, parent, token, n_nodes);
  }
  float x[E];
  ChunkLoad<T>::load(row_ptr(target, draft, r, trows, V), cb * kSpan, V, x);
  post_span_max(x, sv, cmax, slot, C, cb, r, rows, slot_stride, tag);
  for (; r < rows; r += J) {
    const T* p = row_ptr(target, draft, r, trows, V);
    const int64_t rn = r + J;
    float y[PIPE ? E : 1];
    if constexpr (PIPE) {
      if (rn < rows) ChunkLoad<T>::load(row_ptr(target, draft, rn, trows, V), cb * kSpan, V, y);
    }
    if (threadIdx.x < WAVE) {
      // lane j < Cb watches slot j of the row
      const uint64_t* mine = slot + r * slot_stride + min(lane, Cb - 1);
      uint64_t v = 0;
      int late = 0, spins = 0;
      while (true) {
        v = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__all((uint32_t)(v >> 32) == tag)) break;
        if (spins >= spin_limit) {
          late = 1;
          break;
        }
        ++spins;
        __builtin_amdgcn_s_sleep(2);
      }
      const float m = late ? -__builtin_inff()
                           : wave_max_f(__builtin_bit_cast(float, (uint32_t)v));
      if (lane == 0) {
        s_m = m;
        s_late = late;
      }
    }
    __syncthreads();
    float m = s_m;
    if (s_late) {  // the whole row, by this block alone
      float mm = -__builtin_inff();
      for (int i = (int)threadIdx.x; i < V; i += kAccNT) mm = fmaxf(mm, Elem<T>::load(p, i));
      mm = wave_max_f(mm);
      if (lane == 0) sl[threadIdx.x / WAVE] = mm;
      __syncthreads();
      m = sl[0];
      for (int w = 1; w < kAccNT / WAVE; ++w) m = fmaxf(m, sl[w]);
    }
    if constexpr (PIPE) {
      if (rn < rows) post_span_max(y, sv, cmax, slot, C, cb, rn, rows, slot_stride, tag);
    }
    chunk_mass<T, E, PIPE>(x, p, V, C, cb, r, trows, rows, m, inv_t, wsum, cz, N, K, parent,
                           token, depth, n_nodes, wtg, wqg, tc);
    // the row's totals for the walk: its maximum, and its mass as the sum of
    // the spans' masses (integer atomics, so the order does not matter).  The
    // last wave sends them: wave 0 polls, and a wave's loads wait for its own
    // outstanding atomics.
    if (threadIdx.x == kAccNT - WAVE) {
      uint64_t z = 0;
      for (int w = 0; w < kAccNT / WAVE; ++w) z += wsum[w];
      __hip_atomic_fetch_add(&rowz[r * kRowzStride], z, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      if (cb == 0) rowm[r] = m;
    }
    if (rn < rows) {
      if constexpr (PIPE) {
#pragma unroll
        for (int j = 0; j < E; ++j) x[j] = y[j];
      } else {
        ChunkLoad<T>::load(row_ptr(target, draft, rn, trows, V), cb * kSpan, V, x);
        post_span_max(x, sv, cmax, slot, C, cb, rn, rows, slot_stride, tag);
      }
    }
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

// Decision at each node, filled before the walk: the child the walk moves
// to (>= 0), or one of these codes.
constexpr int kNextNone = 0x7fffffff;  // no child accepted (or no child): final draw here
constexpr int kNextErr = -2;           // DRAFT: more than one child, or a bad depth
__device__ __forceinline__ int draft_reject_code(int c) { return -3 - c; }  // DRAFT rejection of c

struct WalkShared {
  int par[kMaxN], tkn[kMaxN];  // par[] holds the excluded tokens during the final draw
  int off[kMaxN + 1];          // children per node, then CSR offsets
  uint32_t list[kMaxN];        // children in CSR order: node | valid << 10 | token << 11
  uint64_t kexl[kMaxN];        // children in CSR order: node | effective weight << 10
  int next[kMaxN];             // decision at each node
  float rmax[kMaxN];           // row maximum
  union {
    int rarg[kMaxN];     // greedy: row argmax, lowest id on ties
    uint64_t rz[kMaxN];  // sampled: row mass Z
  } r;
  uint64_t adraw[kMaxN];              // word 0 of each node's acceptance draw
  uint64_t rd0[kAccNT], rd1[kAccNT];  // final draws of nodes < 256
  float pmax[kAccNT];                 // per-part row statistics
  int parg[kAccNT];
  uint64_t pz[kAccNT];  // then the thread sums of the final draw
  float dmax[kMaxDraftRows];
  uint64_t dz[kMaxDraftRows];
  uint64_t czsub[kMaxChunks];  // rejected children's mass per chunk (final draw)
  int wtot[kAccNT / WAVE];
  int wfirst[kAccNT / WAVE];
  int cs, tok;
  uint64_t r2;
};

__device__ __forceinline__ uint32_t pack_sib(int x, bool valid, int t) {
  return (uint32_t)x | (valid ? 1u << 10 : 0u) | (valid ? (uint32_t)t << 11 : 0u);
}
__device__ __forceinline__ int sib_node(uint32_t e) { return (int)(e & 1023u); }
__device__ __forceinline__ bool sib_valid(uint32_t e) { return (e >> 10) & 1u; }
__device__ __forceinline__ int sib_tok(uint32_t e) { return (int)(e >> 11); }

// floor((hi 2^64 + lo) * Z / 2^128), exact
__device__ __forceinline__ uint64_t scaled_draw(uint64_t hi, uint64_t lo, uint64_t Z) {
  const uint64_t h0 = hi * Z, h1 = __umul64hi(hi, Z);
  const uint64_t l1 = __umul64hi(lo, Z);
  const uint64_t s0 = h0 + l1;
  return h1 + (s0 < h0 ? 1ull : 0ull);
}

// Smallest token of chunk `base` whose running sum exceeds R, given the 16
// consecutive weights of each thread (thread t: tokens base + 16t ...).
// Whole block; every thread returns the token (0x7fffffff if none).  The
// thread sums are monotone in thread order, so the token lies in the first
// thread whose inclusive sum exceeds R: found by ballots, not by atomics
// (a same-address LDS atomic from many lanes is serialised lane by lane).
__device__ int block_pick(const uint64_t (&w)[16], int base, uint64_t R, uint64_t* tsum,
                          int* wfirst, int* tok) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  uint64_t run = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) run += w[j];
  tsum[tid] = run;
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
  const uint64_t ex = tsum[tid];
  const uint64_t bal = __ballot(ex + run > R);
  if (lane == 0) wfirst[wave] = bal ? __ffsll((unsigned long long)bal) - 1 : WAVE;
  __syncthreads();
  int first = -1;
  for (int w2 = 0; w2 < kAccNT / WAVE; ++w2) {
    const int f = wfirst[w2];
    if (f < WAVE) {
      first = w2 * WAVE + f;
      break;
    }
  }
  if (first < 0) return 0x7fffffff;
  if (tid == first) {
    uint64_t acc = ex;
    int jj = 15;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      acc += w[j];
      if (!found && acc > R) {
        jj = j;
        found = true;
      }
    }
    *tok = base + 16 * tid + jj;
  }
  __syncthreads();
  return *tok;
}

// The acceptance of a child depends only on its parent's row and on its
// earlier siblings, never on the path that reaches the parent: with
// Z_res(c) = Z_p - (mass of the distinct tokens of the siblings before c),
// child c of p passes iff U(c) * Z_res(c) < W_eff(c) * 2^64, where
// W_eff(c) = 0 for a token an earlier sibling already carries.  So every
// decision is made in parallel before the walk, and the walk follows next[]
// from the root.
template <typename T, int MODE>
__global__ __launch_bounds__(kAccNT) void k_walk(
    const T* __restrict__ target, const T* __restrict__ draft, int N, int K, int V, int C,
    const int* __restrict__ parent, const int* __restrict__ token,
    const int* __restrict__ depth, const int* __restrict__ n_nodes, float inv_t,
    uint64_t seed, uint64_t round, int max_depth, const float* __restrict__ cmax,
    const int* __restrict__ carg, const uint64_t* __restrict__ cz,
    const float* __restrict__ rowm, uint64_t* rowz, uint32_t* gen,
    const uint64_t* __restrict__ wtg, const uint64_t* __restrict__ wqg, int64_t trows,
    int64_t rows, int* __restrict__ accept_len, int* __restrict__ accepted_nodes,
    int* __restrict__ out_tokens, DraftPending* __restrict__ pend) {
  constexpr bool kSampled = MODE != kGreedy;
  __shared__ WalkShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  const int width = max_depth + 1;
  const int64_t rb = (int64_t)b * N;
  int* acc_nodes = accepted_nodes + (int64_t)b * width;
  int* out_tok = out_tokens + (int64_t)b * width;

  // ---- 1. every load that needs nothing but the shapes, issued together:
  // the tree and the children's weights (thread t owns nodes t + 256 k, all
  // N rows are inside the arrays), the row statistics, and n_nodes.  Rows are
  // all N of the sequence, then its K draft rows in DRAFT mode.  Sampled
  // modes read each row's (maximum, mass) totals (thread t: rows t + 256 k).
  // Greedy reads the chunk records: the rows are split into P parts of the
  // chunk list so that every thread has work; lanes of a part hold
  // consecutive rows, so each chunk-major load is coalesced.
  int pv[4], tv[4], dv[4];
  uint64_t wv[4], qv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tid + k * kAccNT;
    const int64_t at = rb + (c < N ? c : 0);
    pv[k] = parent[at];
    tv[k] = token[at];
    dv[k] = MODE == kDraft ? depth[at] : 0;
    wv[k] = kSampled ? wtg[at] : 0ull;
    qv[k] = MODE == kDraft ? wqg[at] : 0ull;
  }
  const int nr = N + (MODE == kDraft ? K : 0);
  const int P = min(C, max(1, kAccNT / nr));
  const int RP = kAccNT / P;
  const int part = tid / RP, rr = tid - part * RP;
  // greedy: a batch of kGB chunks of row pass r0 (addresses clamped inside
  // the arrays for idle threads and past the last chunk).  Batches of 48
  // (one per pass at 151936 tokens) measured the same as batches of 16.
  constexpr int kGB = kSampled ? 1 : 16;
  float mv[kGB];
  int av[kGB];
  auto load_batch = [&](int r0, int j0) {
    const int r = r0 + rr;
    const bool act = part < P && r < nr;
    const int64_t grow = !act ? 0 : (r < N ? rb + r : trows + (int64_t)b * K + (r - N));
#pragma unroll
    for (int q = 0; q < kGB; ++q) {
      const int j = j0 + q * P;
      const int64_t at = (int64_t)(j < C ? j : 0) * rows + grow;
      mv[q] = cmax[at];
      av[q] = carg[at];
    }
  };
  constexpr int kRowsPer = (kMaxN + kMaxDraftRows + kAccNT - 1) / kAccNT;
  float tmv[kRowsPer];
  uint64_t tzv[kRowsPer];
  // the root row's chunk masses, for a final draw at the root (the usual
  // end of a walk): wave 0, lane j < C holds chunk j
  uint64_t cz_root = 0;
  if constexpr (kSampled) {
    if (wave == 0 && lane < C) cz_root = cz[(int64_t)lane * rows + rb];
#pragma unroll
    for (int k = 0; k < kRowsPer; ++k) {
      const int r = tid + k * kAccNT;
      const int64_t grow = r >= nr ? 0 : (r < N ? rb + r : trows + (int64_t)b * K + (r - N));
      tmv[k] = rowm[grow];
      tzv[k] = rowz[grow * kRowzStride];
    }
    // the rows' mass accumulators go back to zero for the next call (each
    // thread clears what it has just read), and the next call's row pass
    // tags its slots anew (every row pass of this call has ended)
    if (b == 0 && tid == 0) gen[0] = gen[0] + 1u;
#pragma unroll
    for (int k = 0; k < kRowsPer; ++k) {
      const int r = tid + k * kAccNT;
      if (r < nr) {
        const int64_t grow = r < N ? rb + r : trows + (int64_t)b * K + (r - N);
        rowz[grow * kRowzStride] = 0;
      }
    }
  } else {
    load_batch(0, part);
  }
  const int n = n_nodes[b];
  for (int j = tid; j < width; j += kAccNT) {
    acc_nodes[j] = -1;
    out_tok[j] = -1;
  }
  if (MODE == kDraft && tid == 0) pend[b].flag = 0;
  if (n < 1 || n > N) {
    if (tid == 0) accept_len[b] = -1;
    return;
  }
  for (int j = tid; j <= n; j += kAccNT) sh.off[j] = 0;
  for (int j = tid; j < n; j += kAccNT) sh.next[j] = kNextNone;

  // every draw: acceptance draws of nodes 1..n-1, then final draws of
  // nodes < 256
  auto make_draws = [&]() {
    const int na = n - 1, nf = min(n, kAccNT);
    for (int jj = tid; jj < na + nf; jj += kAccNT) {
      const bool accd = jj < na;
      const int node = accd ? jj + 1 : jj - na;
      const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)node,
                                    accd ? 0ull : kResidualSlot, seed, 0);
      if (accd) {
        sh.adraw[node] = d.v[0];
      } else {
        sh.rd0[node] = d.v[0];
        sh.rd1[node] = d.v[1];
      }
    }
  };
  if constexpr (kSampled) {
    make_draws();  // while the row totals are in flight
#pragma unroll
    for (int k = 0; k < kRowsPer; ++k) {
      const int rw = tid + k * kAccNT;
      if (rw < N) {
        sh.rmax[rw] = tmv[k];
        sh.r.rz[rw] = tzv[k];
      } else if (rw < nr) {
        sh.dmax[rw - N] = tmv[k];
        sh.dz[rw - N] = tzv[k];
      }
    }
    __syncthreads();
  }
  for (int r0 = 0; r0 < (kSampled ? 0 : nr); r0 += RP) {
    const int r = r0 + rr;
    const bool act = part < P && r < nr;
    float m = -__builtin_inff();
    int a = 0x7fffffff;
    auto reduce_batch = [&](int j0) {
#pragma unroll
      for (int q = 0; q < kGB; ++q) {
        const bool in = j0 + q * P < C;  // no early exit: the loads stay batched
        if (in && vi_better(mv[q], av[q], m, a)) {
          m = mv[q];
          a = av[q];
        }
      }
    };
    if (r0 > 0) load_batch(r0, part);
    if (act) {
      reduce_batch(part);
      for (int j0 = part + kGB * P; j0 < C; j0 += kGB * P) {
        load_batch(r0, j0);
        reduce_batch(j0);
      }
    }
    if (part < P) {
      sh.pmax[tid] = m;
      sh.parg[tid] = a;
    }
    __syncthreads();
    if (tid < RP && r0 + tid < nr) {
      const int rw = r0 + tid;
      float bm = sh.pmax[tid];
      int ba = sh.parg[tid];
      for (int q = 1; q < P; ++q) {
        const int i = q * RP + tid;
        if (vi_better(sh.pmax[i], sh.parg[i], bm, ba)) {
          bm = sh.pmax[i];
          ba = sh.parg[i];
        }
      }
      sh.rmax[rw] = bm;  // greedy has no draft rows: rw < N
      sh.r.rarg[rw] = ba;
    }
    __syncthreads();
  }

  // ---- 2. tree into LDS; children counted (the returned count is the
  // child's place in its parent's list)
  bool child[4], okt[4];
  int pos[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tid + k * kAccNT;
    if (c >= n) pv[k] = tv[k] = -1;
    if (c < n) {
      sh.par[c] = pv[k];
      sh.tkn[c] = tv[k];
    }
    child[k] = c >= 1 && c < n && pv[k] >= 0 && pv[k] < n;
    okt[k] = child[k] && tv[k] >= 0 && tv[k] < V;
    pos[k] = (kSampled && child[k]) ? atomicAdd(&sh.off[pv[k]], 1) : 0;
  }
  __syncthreads();

  if (MODE == kGreedy) {
    // the first child in row order whose token is the row's argmax
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (child[k] && tv[k] == sh.r.rarg[pv[k]]) atomicMin(&sh.next[pv[k]], tid + k * kAccNT);
    __syncthreads();
  } else {
    // ---- 3. CSR offsets: exclusive scan of the counts
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
    int slot[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      slot[k] = child[k] ? sh.off[pv[k]] + pos[k] : 0;
      if (child[k]) sh.list[slot[k]] = pack_sib(tid + k * kAccNT, okt[k], tv[k]);
    }
    __syncthreads();

    // ---- 4. per child: whether an earlier sibling carries the same token,
    // and its effective weight; DRAFT: the decision at the parent
    uint64_t wef[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + k * kAccNT;
      wef[k] = 0;
      if (!child[k]) continue;
      const int p = pv[k], t = tv[k];
      const int o0 = sh.off[p], o1 = sh.off[p + 1];
      const uint64_t w = okt[k] ? wv[k] : 0ull;
      if (MODE == kPointMass) {
        bool dup = false;
        for (int e0 = o0; e0 < o1; e0 += 8) {
          uint32_t sb[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) sb[q] = sh.list[min(e0 + q, o1 - 1)];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            dup |= sib_node(sb[q]) < c && sib_valid(sb[q]) && sib_tok(sb[q]) == t;
        }
        wef[k] = dup ? 0ull : w;
        sh.kexl[slot[k]] = (uint64_t)c | (wef[k] << 10);
      } else {
        // DRAFT: p(t) and q(t); a chain node has one child
        if (o1 - o0 > 1 || dv[k] < 1 || dv[k] > K) {
          sh.next[p] = kNextErr;
        } else {
          const double pt = okt[k] ? (double)w / (double)sh.r.rz[p] : 0.0;
          const double qt = okt[k] ? (double)qv[k] / (double)sh.dz[dv[k] - 1] : 0.0;
          const double u53 = (double)(sh.adraw[c] >> 11) * 0x1p-53;
          // min(1, p/q): a token the target gives no mass is never accepted
          const bool ok = pt > 0.0 && (pt >= qt || u53 < pt / qt);
          sh.next[p] = ok ? c : draft_reject_code(c);
        }
      }
    }
    __syncthreads();

    if (MODE == kPointMass) {
      // ---- 5. per child: the residual mass it is tested against
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = tid + k * kAccNT;
        if (!child[k]) continue;
        const int p = pv[k];
        const int o0 = sh.off[p], o1 = sh.off[p + 1];
        uint64_t before = 0;
        for (int e0 = o0; e0 < o1; e0 += 8) {
          uint64_t kb[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) kb[q] = sh.kexl[min(e0 + q, o1 - 1)];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (e0 + q < o1 && (int)(kb[q] & 1023u) < c) before += kb[q] >> 10;
        }
        const uint64_t zres = sh.r.rz[p] - before;
        if (__umul64hi(sh.adraw[c], zres) < wef[k]) atomicMin(&sh.next[p], c);
      }
      __syncthreads();
    }
  }

  // ---- the walk: every wave follows next[] from the root (LDS reads only)
  if (tid == 0) acc_nodes[0] = 0;
  int u = 0, len = 0, nx = kNextNone;
  for (;;) {
    nx = len < max_depth ? sh.next[u] : kNextNone;
    if (nx < 0 || nx == kNextNone) break;
    ++len;
    if (tid == 0) {
      acc_nodes[len] = nx;
      out_tok[len - 1] = sh.tkn[nx];
    }
    u = nx;
  }
  int bonus = -1;
  bool err = false, pending = false;
  if (MODE == kGreedy) {
    bonus = sh.r.rarg[u];
  } else if (MODE == kDraft && nx == kNextErr) {
    err = true;
  } else if (MODE == kDraft && nx != kNextNone) {
    // rejection of child c: the residual (p - q)+ is drawn by the kernels
    // that follow
    const int c = -3 - nx;
    if (tid == 0) {
      const int dd = depth[rb + c];
      DraftPending pd;
      pd.flag = 1;
      pd.u = u;
      pd.dd = dd;
      pd.len = len;
      pd.mu = sh.rmax[u];
      pd.mq = sh.dmax[dd - 1];
      pd.zu = sh.r.rz[u];
      pd.zq = sh.dz[dd - 1];
      if (u < kAccNT) {
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
  } else {
    // ---- final draw at u from the target row with u's children removed
    // (none past the depth limit, and none in DRAFT mode where u is a leaf):
    // wave 0 picks the chunk from the exact chunk masses, then the block
    // weighs that chunk's 4096 tokens and picks the token.
    const int64_t grow = rb + u;
    const int o0 = sh.off[u];
    const int nk = (MODE == kPointMass && len < max_depth) ? sh.off[u + 1] - o0 : 0;
    if (wave == 0) {
      const int jl = lane < C ? lane : 0;
      const uint64_t czu = u == 0 ? cz_root : cz[(int64_t)jl * rows + grow];
      uint64_t d0, d1;
      if (u < kAccNT) {
        d0 = sh.rd0[u];
        d1 = sh.rd1[u];
      } else {
        const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)u, kResidualSlot, seed, 0);
        d0 = d.v[0];
        d1 = d.v[1];
      }
      // the rejected children's mass, per chunk (an LDS histogram) and in
      // total; their tokens go to par[] for the token-level exclusion
      sh.czsub[lane] = 0;
      wave_lds_sync();
      uint64_t zx = 0;
      for (int g = 0; g < nk; g += WAVE) {
        const int i = g + lane;
        if (i < nk) {
          const uint32_t sb = sh.list[o0 + i];
          const uint64_t we = sh.kexl[o0 + i] >> 10;
          sh.par[i] = sib_valid(sb) ? sib_tok(sb) : -1;
          if (we) atomicAdd((unsigned long long*)&sh.czsub[sib_tok(sb) >> 12],
                            (unsigned long long)we);
          zx += we;
        }
      }
      wave_lds_sync();
      const uint64_t Zres = sh.r.rz[u] - wave_sum_u64(zx);
      const uint64_t cw = lane < C ? czu - sh.czsub[lane] : 0ull;
      const uint64_t R = scaled_draw(d0, d1, Zres);
      const uint64_t incl = wave_incl_scan_u64(cw);
      const uint64_t hit = __ballot(lane < C && incl > R);
      const int cs = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
      const uint64_t before = cs >= 0 ? readlane_u64(incl - cw, cs) : 0ull;
      if (lane == 0) {
        sh.cs = cs;
        sh.r2 = R - before;
      }
    }
    __syncthreads();
    const int cs = sh.cs;
    if (cs >= 0) {
      const int base = cs * kAcceptChunk;
      float x[16];
      ChunkLoad<T>::load(target + grow * (int64_t)V, base, V, x);
      const float m = sh.rmax[u];
      uint64_t w[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = weight(x[j], m, inv_t);
      // excluded tokens among this thread's 16, as a bit mask
      const int lo = base + 16 * tid;
      uint32_t xm = 0;
      for (int e0 = 0; e0 < nk; e0 += 8) {
        int te[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) te[q] = sh.par[min(e0 + q, nk - 1)];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t rel = (uint32_t)(te[q] - lo);
          xm |= rel < 16u ? 1u << rel : 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((xm >> j) & 1u) w[j] = 0;
      const int tok = block_pick(w, base, sh.r2, sh.pz, sh.wfirst, &sh.tok);
      bonus = tok == 0x7fffffff ? -1 : tok;
    }
  }
  if (tid == 0) {
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
  __shared__ int s_wfirst[kAccNT / WAVE];
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
    tok = block_pick(w, base, s_r, tsum, s_wfirst, &s_tok);
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
  p.off_wtg = sampled ? take((size_t)batch * N * sizeof(uint64_t)) : 0;
  p.off_wqg = draft ? take((size_t)batch * N * sizeof(uint64_t)) : 0;
  p.off_rcz = draft ? take((size_t)batch * kMaxChunks * sizeof(uint64_t)) : 0;
  p.off_pend = draft ? take((size_t)batch * sizeof(DraftPending)) : 0;
  p.slot_stride = (p.C + 31) & ~31;  // 256-byte rows of slots
  p.off_slot = sampled ? take((size_t)p.rows * p.slot_stride * sizeof(uint64_t)) : 0;
  p.off_rowz = sampled ? take((size_t)p.rows * kRowzStride * sizeof(uint64_t)) : 0;
  p.off_rowm = sampled ? take((size_t)p.rows * sizeof(float)) : 0;
  p.off_gen = sampled ? take(sizeof(uint32_t)) : 0;  // the slots' generation
  p.workspace = off;
  return p;
}

// Polls of the row-maximum wait before a k_rowstat block reads the whole row
// itself (each an agent-scope load, about 1 us under the pass's traffic):
// tens of microseconds, against the few polls a resident group needs, so
// that a block delayed by other work on the device costs a bounded detour.
// tv_debug_set_spin_limit lowers it so that tests take the fallback.
constexpr int kSpinLimit = 48;
std::atomic<int> g_rowstat_spin_limit{kSpinLimit};

int set_rowstat_spin_limit(int polls) {
  const int old = g_rowstat_spin_limit.load();
  g_rowstat_spin_limit.store(polls < 0 ? kSpinLimit : std::min(polls, kSpinLimit));
  return old;
}

// Blocks of one k_rowstat instance the device holds at once (cached per
// device).
template <typename T, int E, bool PIPE>
static int64_t rowstat_capacity() {
  static std::atomic<int> resident[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::atomic<int>& slot = resident[dev & 63];
  int cap = slot.load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&k_rowstat<T, E, PIPE>), kAccNT, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu < 1 || cus < 1) {
      per_cu = 1;
      cus = 64;
    }
    cap = per_cu * cus;
    slot.store(cap, std::memory_order_relaxed);
  }
  return cap;
}

// The row pass's shape: one row per block when the device holds all the
// (row, 8192-token span) blocks at once, else all the (row, 4096-token
// chunk) blocks; else the pipelined kernel over 4096-token chunks with J
// groups of Cb blocks within what the device holds, as many groups as keep
// the rows balanced (ceil(rows / J) each).  (Measured on the 4B/8B-class
// rounds: of the multi-row forms, 8192-token spans without or with the
// pipeline were 9 and 13 % slower than this one.)
struct RowstatShape {
  int E;
  bool pipe;
  int Cb;
  unsigned grid;
};

template <typename T, int E, bool PIPE>
static RowstatShape rowstat_groups(int64_t rows, int Cb) {
  int64_t J = std::max<int64_t>(1, rowstat_capacity<T, E, PIPE>() / Cb);
  J = std::min<int64_t>(J, rows);
  const int64_t iters = (rows + J - 1) / J;
  J = (rows + iters - 1) / iters;
  return {E, PIPE, Cb, (unsigned)(J * Cb)};
}

template <typename T>
static RowstatShape rowstat_shape(int64_t rows, int V) {
  const int cb32 = (V + 32 * kAccNT - 1) / (32 * kAccNT);
  const int cb16 = (V + 16 * kAccNT - 1) / (16 * kAccNT);
  if (rows * cb32 <= rowstat_capacity<T, 32, false>())
    return {32, false, cb32, (unsigned)(rows * cb32)};
  if (rows * cb16 <= rowstat_capacity<T, 16, false>())
    return {16, false, cb16, (unsigned)(rows * cb16)};
  return rowstat_groups<T, 16, true>(rows, cb16);
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
  uint64_t* wtg = sampled ? reinterpret_cast<uint64_t*>(w + p.off_wtg) : nullptr;
  uint64_t* wqg = draft_proposal ? reinterpret_cast<uint64_t*>(w + p.off_wqg) : nullptr;
  uint64_t* rcz = draft_proposal ? reinterpret_cast<uint64_t*>(w + p.off_rcz) : nullptr;
  DraftPending* pend =
      draft_proposal ? reinterpret_cast<DraftPending*>(w + p.off_pend) : nullptr;
  uint64_t* rowz = sampled ? reinterpret_cast<uint64_t*>(w + p.off_rowz) : nullptr;
  float* rowm = sampled ? reinterpret_cast<float*>(w + p.off_rowm) : nullptr;
  uint64_t* slot = sampled ? reinterpret_cast<uint64_t*>(w + p.off_slot) : nullptr;
  uint32_t* gen = sampled ? reinterpret_cast<uint32_t*>(w + p.off_gen) : nullptr;
  const int64_t trows = (int64_t)batch * N;
  const dim3 g(p.C, (unsigned)p.rows);
  const dim3 blk(kAccNT);
  RowstatShape sh{};
  if (sampled) {
    sh = rowstat_shape<T>(p.rows, V);
    const int spin = g_rowstat_spin_limit.load(std::memory_order_relaxed);
#define TV_ROWSTAT(E, PIPE)                                                                    \
  hipLaunchKernelGGL((k_rowstat<T, E, PIPE>), dim3(sh.grid), blk, 0, stream, target, draft, V, \
                     p.C, sh.Cb, trows, p.rows, inv_t, cmax, slot, p.slot_stride, cz, rowm,    \
                     rowz, N, K, parent, token, depth, n_nodes, wtg, wqg, gen, spin)
    if (sh.E == 32)
      TV_ROWSTAT(32, false);
    else if (!sh.pipe)
      TV_ROWSTAT(16, false);
    else
      TV_ROWSTAT(16, true);
#undef TV_ROWSTAT
  } else {
    hipLaunchKernelGGL((k_rowmax<T>), g, blk, 0, stream, target, draft, V, trows, p.rows,
                       cmax, carg);
  }
#define TV_WALK(M)                                                                            \
  hipLaunchKernelGGL((k_walk<T, M>), dim3(batch), blk, 0, stream, target, draft, N, K, V, p.C, \
                     parent, token, depth, n_nodes, inv_t, seed, round, max_depth, cmax, carg, \
                     cz, rowm, rowz, gen, wtg, wqg, trows, p.rows, accept_len, accepted_nodes, \
                     out_tokens, pend)
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

// Test hook: the fixed-point weight of every fp32 value whose bit pattern is
// first + i, 0 <= i < count, as the logit of a row with maximum m (the
// inv_t == 1 form used by the row passes when unit is set).
__global__ __launch_bounds__(256) void k_debug_weights(uint32_t first, uint32_t count, float m,
                                                       float inv_t, int unit,
                                                       uint64_t* __restrict__ out) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const float x = __builtin_bit_cast(float, first + (uint32_t)i);
  out[i] = unit ? (uint64_t)weight_f<true>(x, m, inv_t) : weight(x, m, inv_t);
}

hipError_t launch_debug_weights(uint32_t first, uint32_t count, float m, float inv_t, bool unit,
                                uint64_t* out, hipStream_t stream) {
  const unsigned grid = (unsigned)(((uint64_t)count + 255) / 256);
  hipLaunchKernelGGL(k_debug_weights, dim3(grid), dim3(256), 0, stream, first, count, m, inv_t,
                     unit ? 1 : 0, out);
  return hipGetLastError();
}

}  // namespace tvk
