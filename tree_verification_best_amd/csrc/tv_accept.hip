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
//   k_rowmax  grid (chunks, rows)  (max, argmax) of each 4096-token chunk of
//                                  every target row (and draft row in DRAFT mode)
//   k_rowz    grid (chunks, rows)  fixed-point softmax mass of each chunk
//                                  (sampled modes only)
//   k_walk    grid (batch)         the walk: children of the current node,
//                                  acceptance draws, final draw by exact
//                                  integer inverse CDF over the chunk sums
// The passes read every row; the walk only ever visits rows < n_nodes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

constexpr int kAccNT = 256;
constexpr int kAccE = kAcceptChunk / kAccNT;  // 16 tokens per thread and chunk

enum WalkMode { kGreedy = 0, kPointMass = 1, kDraft = 2 };

template <typename T>
__device__ __forceinline__ const T* row_ptr(const T* target, const T* draft, int64_t r,
                                            int64_t trows, int V) {
  return r < trows ? target + r * (int64_t)V : draft + (r - trows) * (int64_t)V;
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

// (max, argmax lowest id) of each 4096-token chunk of every row.  Rows past
// n_nodes are read too (they are inside the array) and never used.
template <typename T>
__global__ __launch_bounds__(kAccNT) void k_rowmax(const T* __restrict__ target,
                                                  const T* __restrict__ draft, int V, int C,
                                                  int64_t trows, float* __restrict__ cmax,
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
    cmax[r * C + c] = bv;
    carg[r * C + c] = bi;
  }
}

__device__ __forceinline__ float row_max_from_chunks(const float* cm, int C) {
  // called by one full wave
  float m = -__builtin_inff();
  for (int j = lane_id(); j < C; j += WAVE) m = fmaxf(m, cm[j]);
  return wave_max_f(m);
}

// Fixed-point softmax mass of each chunk.  The chunk's logits are loaded
// first; the row maximum (from the chunk maxima) arrives while they are in
// flight.
template <typename T>
__global__ __launch_bounds__(kAccNT) void k_rowz(const T* __restrict__ target,
                                                const T* __restrict__ draft, int V, int C,
                                                int64_t trows, float inv_t,
                                                const float* __restrict__ cmax,
                                                uint64_t* __restrict__ cz) {
  __shared__ float s_m;
  __shared__ uint64_t wsum[kAccNT / WAVE];
  const int c = blockIdx.x;
  const int64_t r = blockIdx.y;
  const T* p = row_ptr(target, draft, r, trows, V);
  const int base = c * kAcceptChunk;
  float x[16];
  ChunkLoad<T>::load(p, base, V, x);
  if (threadIdx.x < WAVE) {
    const float m = row_max_from_chunks(cmax + r * C, C);
    if (threadIdx.x == 0) s_m = m;
  }
  __syncthreads();
  const float m = s_m;
  uint64_t acc = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc += weight(x[j], m, inv_t);  // -inf padding weighs 0
  acc = wave_sum_u64(acc);
  if (lane_id() == 0) wsum[threadIdx.x / WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t z = 0;
    for (int w = 0; w < kAccNT / WAVE; ++w) z += wsum[w];
    cz[r * C + c] = z;
  }
}

// ---------------------------------------------------------------------------
// walk
// ---------------------------------------------------------------------------
struct WalkShared {
  int kids[1024];
  int ktok[1024];
  uint64_t kw[1024];
  uint64_t chunk_w[64];
  uint64_t tsum[kAccNT];
  unsigned char excl[kAcceptChunk];
  int nk, next, bonus, err, tok, cstar;
  uint64_t zres, zq, before;
  float m, mq;
};

// floor((hi 2^64 + lo) * Z / 2^128), exact
__device__ __forceinline__ uint64_t scaled_draw(uint64_t hi, uint64_t lo, uint64_t Z) {
  const uint64_t h0 = hi * Z, h1 = __umul64hi(hi, Z);
  const uint64_t l1 = __umul64hi(lo, Z);
  const uint64_t s0 = h0 + l1;
  return h1 + (s0 < h0 ? 1ull : 0ull);
}

// Smallest token v with (sum of w over tokens <= v) > R, given the chunk
// sums in sh.chunk_w[0..C) and a per-token weight functor w(v) (0 for
// excluded tokens).  Whole block; returns the same value in every thread.
template <typename WF>
__device__ int chunked_inverse_cdf(WalkShared& sh, int C, int V, uint64_t R, WF w,
                                   const int* excl_tok, const uint64_t* excl_w, int nexcl) {
  const int tid = threadIdx.x;
  if (tid < WAVE) {
    const uint64_t cw = tid < C ? sh.chunk_w[tid] : 0ull;
    const uint64_t incl = wave_incl_scan_u64(cw);
    const uint64_t hit = __ballot(tid < C && incl > R);
    const int cstar = hit ? __ffsll((unsigned long long)hit) - 1 : C - 1;
    const uint64_t before = readlane_u64(incl - cw, cstar);
    if (tid == 0) {
      sh.cstar = cstar;
      sh.before = before;
      sh.tok = 0x7fffffff;
    }
  }
  __syncthreads();
  const int cstar = sh.cstar;
  const uint64_t before = sh.before;
  const int base = cstar * kAcceptChunk;
  for (int j = tid; j < kAcceptChunk; j += kAccNT) sh.excl[j] = 0;
  __syncthreads();
  for (int e = tid; e < nexcl; e += kAccNT) {
    const int t = excl_tok[e];
    if (excl_w[e] > 0 && t >= base && t < base + kAcceptChunk) sh.excl[t - base] = 1;
  }
  __syncthreads();
  uint64_t loc[kAccE];
  uint64_t run = 0;
#pragma unroll
  for (int j = 0; j < kAccE; ++j) {
    const int v = base + tid * kAccE + j;
    uint64_t x = 0;
    if (v < V && !sh.excl[v - base]) x = w(v);
    run += x;
    loc[j] = run;
  }
  sh.tsum[tid] = run;
  __syncthreads();
  // exclusive prefix of the thread totals (256 values, one wave scans 4 each)
  if (tid < WAVE) {
    uint64_t a0 = sh.tsum[4 * tid], a1 = sh.tsum[4 * tid + 1], a2 = sh.tsum[4 * tid + 2],
             a3 = sh.tsum[4 * tid + 3];
    const uint64_t s4 = a0 + a1 + a2 + a3;
    const uint64_t incl = wave_incl_scan_u64(s4);
    uint64_t ex = incl - s4;
    sh.tsum[4 * tid] = ex;
    ex += a0;
    sh.tsum[4 * tid + 1] = ex;
    ex += a1;
    sh.tsum[4 * tid + 2] = ex;
    ex += a2;
    sh.tsum[4 * tid + 3] = ex;
  }
  __syncthreads();
  const uint64_t off = before + sh.tsum[tid];
#pragma unroll
  for (int j = 0; j < kAccE; ++j) {
    const int v = base + tid * kAccE + j;
    if (v < V && off + loc[j] > R) {
      atomicMin(&sh.tok, v);
      break;
    }
  }
  __syncthreads();
  const int tok = sh.tok;
  __syncthreads();
  return tok;
}

template <typename T>
__global__ __launch_bounds__(kAccNT) void k_walk(
    const T* __restrict__ target, const T* __restrict__ draft, int N, int K, int V, int C,
    const int* __restrict__ parent, const int* __restrict__ token,
    const int* __restrict__ depth, const int* __restrict__ n_nodes, int mode, float inv_t,
    uint64_t seed, uint64_t round, int max_depth, const float* __restrict__ cmax,
    const int* __restrict__ carg, const uint64_t* __restrict__ cz, int64_t trows,
    int* __restrict__ accept_len, int* __restrict__ accepted_nodes,
    int* __restrict__ out_tokens) {
  __shared__ WalkShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id();
  const int width = max_depth + 1;
  const int64_t rb = (int64_t)b * N;
  int* acc_nodes = accepted_nodes + (int64_t)b * width;
  int* out_tok = out_tokens + (int64_t)b * width;
  for (int j = tid; j < width; j += kAccNT) {
    acc_nodes[j] = -1;
    out_tok[j] = -1;
  }
  const int n = n_nodes[b];
  if (n < 1 || n > N) {
    if (tid == 0) accept_len[b] = -1;
    return;
  }
  __syncthreads();
  if (tid == 0) acc_nodes[0] = 0;
  int u = 0, len = 0;
  int bonus = -1;
  bool err = false;
  for (int iter = 0; iter <= max_depth; ++iter) {
    const int64_t r = rb + u;
    // ---- children of u, in row order (a node at depth max_depth is a leaf)
    if (tid < WAVE) {
      int cnt = 0;
      if (len < max_depth)
        for (int base = 1; base < n; base += WAVE) {
          const int c = base + lane;
          const bool is = c < n && parent[rb + c] == u;
          const uint64_t bal = __ballot(is);
          if (is) {
            const int at = cnt + __popcll(bal & ((1ull << lane) - 1ull));
            sh.kids[at] = c;
          }
          cnt += __popcll(bal);
        }
      if (tid == 0) {
        sh.nk = cnt;
        sh.next = -1;
        sh.err = 0;
      }
    }
    __syncthreads();
    const int nk = sh.nk;
    if (mode == kGreedy) {
      if (tid < WAVE) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
        for (int j = lane; j < C; j += WAVE) {
          const float x = cmax[r * C + j];
          const int xi = carg[r * C + j];
          if (vi_better(x, xi, bv, bi)) {
            bv = x;
            bi = xi;
          }
        }
        wave_argmax(bv, bi);
        int nxt = -1;
        for (int base = 0; base < nk && nxt < 0; base += WAVE) {
          const int i = base + lane;
          const bool m = i < nk && token[rb + sh.kids[i]] == bi;
          const uint64_t bal = __ballot(m);
          if (bal) nxt = sh.kids[base + __ffsll((unsigned long long)bal) - 1];
        }
        if (tid == 0) {
          sh.next = nxt;
          sh.bonus = bi;
        }
      }
      __syncthreads();
    } else if (mode == kPointMass) {
      if (tid < WAVE) {
        const float m = row_max_from_chunks(cmax + r * C, C);
        uint64_t Zu = 0;
        for (int j = lane; j < C; j += WAVE) Zu += cz[r * C + j];
        Zu = wave_sum_u64(Zu);
        const T* rowp = target + r * (int64_t)V;
        uint64_t carried = 0;
        int nxt = -1;
        for (int base = 0; base < nk && nxt < 0; base += WAVE) {
          const int i = base + lane;
          const bool live = i < nk;
          const int t = live ? token[rb + sh.kids[i]] : -1;
          if (live) sh.ktok[i] = t;
          bool dup = false;
          if (live)
            for (int j = 0; j < i; ++j) dup |= (sh.ktok[j] == t);
          uint64_t w = 0;
          if (live && !dup && t >= 0 && t < V) w = weight(Elem<T>::load(rowp, t), m, inv_t);
          if (live) sh.kw[i] = w;
          const uint64_t incl = wave_incl_scan_u64(w);
          const uint64_t zres = Zu - carried - (incl - w);
          const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)u, (uint64_t)i, seed, 0);
          const bool ok = live && (__umul64hi(d.v[0], zres) < w);
          const uint64_t bal = __ballot(ok);
          if (bal) nxt = sh.kids[base + __ffsll((unsigned long long)bal) - 1];
          carried += readlane_u64(incl, WAVE - 1);
        }
        if (tid == 0) {
          sh.next = nxt;
          sh.zres = Zu - carried;
          sh.m = m;
        }
        if (nxt < 0)
          for (int j = lane; j < C; j += WAVE) sh.chunk_w[j] = cz[r * C + j];
      }
      __syncthreads();
      if (sh.next < 0) {
        // exclusions leave their chunks
        if (tid < C) {
          uint64_t s = 0;
          for (int e = 0; e < nk; ++e) {
            const int t = sh.ktok[e];
            if (sh.kw[e] > 0 && t / kAcceptChunk == tid) s += sh.kw[e];
          }
          sh.chunk_w[tid] -= s;
        }
        const uint64_t Z = sh.zres;
        const float m = sh.m;
        __syncthreads();
        const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)u, kResidualSlot, seed, 0);
        const uint64_t R = scaled_draw(d.v[0], d.v[1], Z);
        const T* rowp = target + r * (int64_t)V;
        bonus = chunked_inverse_cdf(
            sh, C, V, R, [&](int v) { return weight(Elem<T>::load(rowp, v), m, inv_t); },
            sh.ktok, sh.kw, nk);
        if (tid == 0) sh.bonus = bonus;
        __syncthreads();
      }
    } else {  // DRAFT proposal, chains only
      const T* rowp = target + r * (int64_t)V;
      float m = 0.f, mq = 0.f;
      uint64_t Zu = 0, Zq = 0;
      int c = -1, t = -1, dd = 0;
      if (nk > 1) {
        err = true;
        break;
      }
      if (tid < WAVE) {
        m = row_max_from_chunks(cmax + r * C, C);
        for (int j = lane; j < C; j += WAVE) Zu += cz[r * C + j];
        Zu = wave_sum_u64(Zu);
      }
      if (nk == 1) {
        c = sh.kids[0];
        t = token[rb + c];
        dd = depth[rb + c];
        if (dd < 1 || dd > K) {
          err = true;
          break;
        }
        const int64_t rq = trows + (int64_t)b * K + (dd - 1);
        if (tid < WAVE) {
          mq = row_max_from_chunks(cmax + rq * C, C);
          for (int j = lane; j < C; j += WAVE) Zq += cz[rq * C + j];
          Zq = wave_sum_u64(Zq);
        }
        if (tid == 0) {
          const T* qrow = draft + ((int64_t)b * K + (dd - 1)) * (int64_t)V;
          double pt = 0.0, qt = 0.0;
          if (t >= 0 && t < V) {
            pt = (double)weight(Elem<T>::load(rowp, t), m, inv_t) / (double)Zu;
            qt = (double)weight(Elem<T>::load(qrow, t), mq, inv_t) / (double)Zq;
          }
          const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)u, 0ull, seed, 0);
          const double u53 = (double)(d.v[0] >> 11) * 0x1p-53;
          const bool ok = (pt >= qt) || (u53 < pt / qt);
          sh.next = ok ? c : -1;
          sh.m = m;
          sh.zres = Zu;
          sh.zq = Zq;
          sh.mq = mq;
        }
      } else if (tid == 0) {
        sh.next = -1;
        sh.m = m;
        sh.zres = Zu;
      }
      __syncthreads();
      if (sh.next < 0) {
        m = sh.m;
        Zu = sh.zres;
        const u64x4 d = philox4x64_10(round, (uint64_t)b, (uint64_t)u, kResidualSlot, seed, 0);
        if (nk == 0) {
          // end of the chain: the bonus token comes from the target row
          if (tid < C) sh.chunk_w[tid] = cz[r * C + tid];
          __syncthreads();
          const uint64_t R = scaled_draw(d.v[0], d.v[1], Zu);
          bonus = chunked_inverse_cdf(
              sh, C, V, R, [&](int v) { return weight(Elem<T>::load(rowp, v), m, inv_t); },
              sh.ktok, sh.kw, 0);
        } else {
          Zq = sh.zq;
          mq = sh.mq;
          __syncthreads();
          const T* qrow = draft + ((int64_t)b * K + (dd - 1)) * (int64_t)V;
          auto resid = [&](int v) -> uint64_t {
            const double p = (double)weight(Elem<T>::load(rowp, v), m, inv_t) / (double)Zu;
            const double q = (double)weight(Elem<T>::load(qrow, v), mq, inv_t) / (double)Zq;
            const double rr = p - q;
            return rr > 0.0 ? (uint64_t)__builtin_rint(rr * 0x1p62) : 0ull;
          };
          // chunk sums of the residual weights
          for (int cc = 0; cc < C; ++cc) {
            uint64_t s = 0;
#pragma unroll
            for (int j = 0; j < kAccE; ++j) {
              const int v = cc * kAcceptChunk + tid * kAccE + j;
              if (v < V) s += resid(v);
            }
            s = wave_sum_u64(s);
            if (lane == 0) sh.tsum[tid / WAVE] = s;
            __syncthreads();
            if (tid == 0) {
              uint64_t z = 0;
              for (int w = 0; w < kAccNT / WAVE; ++w) z += sh.tsum[w];
              sh.chunk_w[cc] = z;
            }
            __syncthreads();
          }
          uint64_t ZR = 0;
          for (int cc = 0; cc < C; ++cc) ZR += sh.chunk_w[cc];
          __syncthreads();
          if (ZR > 0) {
            const uint64_t R = scaled_draw(d.v[0], d.v[1], ZR);
            bonus = chunked_inverse_cdf(sh, C, V, R, resid, sh.ktok, sh.kw, 0);
          } else {
            if (tid < C) sh.chunk_w[tid] = cz[r * C + tid];
            __syncthreads();
            const uint64_t R = scaled_draw(d.v[0], d.v[1], Zu);
            bonus = chunked_inverse_cdf(
                sh, C, V, R,
                [&](int v) { return weight(Elem<T>::load(rowp, v), m, inv_t); }, sh.ktok,
                sh.kw, 0);
          }
        }
        if (tid == 0) sh.bonus = bonus;
        __syncthreads();
      }
    }
    const int nxt = sh.next;
    if (nxt >= 0) {
      ++len;
      if (tid == 0) {
        acc_nodes[len] = nxt;
        out_tok[len - 1] = token[rb + nxt];
      }
      u = nxt;
      __syncthreads();
      continue;
    }
    bonus = sh.bonus;
    break;
  }
  if (tid == 0) {
    if (err) {
      accept_len[b] = -1;
    } else {
      accept_len[b] = len;
      out_tok[len] = bonus;
    }
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
  const int64_t trows = (int64_t)batch * N;
  dim3 g(p.C, (unsigned)p.rows);
  hipLaunchKernelGGL((k_rowmax<T>), g, dim3(kAccNT), 0, stream, target, draft, V, p.C, trows,
                     cmax, carg);
  if (sampled)
    hipLaunchKernelGGL((k_rowz<T>), g, dim3(kAccNT), 0, stream, target, draft, V, p.C, trows,
                       inv_t, cmax, cz);
  const int mode = !sampled ? kGreedy : (draft_proposal ? kDraft : kPointMass);
  hipLaunchKernelGGL((k_walk<T>), dim3(batch), dim3(kAccNT), 0, stream, target, draft, N, K,
                     V, p.C, parent, token, depth, n_nodes, mode, inv_t, seed, round,
                     max_depth, cmax, carg, cz, trows, accept_len, accepted_nodes, out_tokens);
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
