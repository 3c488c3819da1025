// tv_attention.hip -- tree-masked GQA attention of one target layer on gfx950.
//
// PTD sec. 3.1: node v sees only its ancestor set pi(v) = {v} U pi(P(v));
// primer ("why the target can verify in parallel"): the target reads the
// whole context plus the drafts in one pass.  Node i of sequence b, query
// head h, attends to context keys [0, L_b) and tree keys L_b + j, j in pi(i).
//
// bf16 path, per KV head g of sequence b:
//   * the G = Hq / Hkv query heads of every node share the KV head, so the
//     rows (node, head-in-group) are packed into the MFMA dimension: one
//     wave owns 32 rows, a workgroup 1..4 waves, and every K/V tile staged
//     in LDS serves all of them;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the output lane l holds
//     query row l % 32 and 16 of the tile's 32 keys, so the online softmax
//     (row max, rescale, row sum) stays in the lane plus one exchange with
//     lane l ^ 32;
//   * O^T += V^T P^T with the same instruction: P^T leaves the registers of
//     the S^T accumulator as the B operand directly (same lane = same row);
//     V is stored transposed in LDS so the A operand is two 8-byte reads;
//   * split-K over the context: split s < S covers keys [s*KS, (s+1)*KS), the
//     extra split S covers the tree keys with the ancestor mask (the only
//     masked tile); partials (m, l, O) go to the workspace and k_combine
//     merges them with their log-sum-exp weights.
// f32 path: a plain vector-ALU kernel (used for fp32 inputs).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 32;     // keys per tile
constexpr int kAttnMaxWaves = 4;

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

template <int D>
__global__ __launch_bounds__(kAttnMaxWaves * WAVE) void k_attn_partial(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int* __restrict__ ctx_len,
    const uint64_t* __restrict__ anc, const int* __restrict__ n_nodes, int N, int Hq, int Hkv,
    int cap, int S, int KS, float scale_log2, float* __restrict__ Opart,
    float* __restrict__ Mpart, float* __restrict__ Lpart, int batch) {
  constexpr int KPAD = D + 8;       // K tile row stride (bf16)
  constexpr int VPAD = kTile + 8;   // V^T tile row stride (bf16)
  __shared__ __align__(16) uint16_t Ks[kTile * KPAD];
  __shared__ __align__(16) uint16_t Vt[D * VPAD];

  const int split = blockIdx.x;
  const int mt = blockIdx.y;
  const int bg = blockIdx.z;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  // ctx_len <= max_ctx and max_ctx + N <= cap are preconditions; the clamp
  // keeps every key row inside the cache whatever the caller passes
  const int L = min(max(ctx_len[b], 0), cap - N);
  const int n = min(n_nodes[b], N);
  const int W = (N + 63) / 64;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid / WAVE, lane = tid % WAVE;
  const int half = lane >> 5, l32 = lane & 31;
  const int nwaves = nthreads / WAVE;

  const int row = (mt * nwaves + wave) * 32 + l32;
  const int node = row / G;
  const int h = g * G + row % G;
  const bool row_ok = node < n;

  int k0, k1;
  if (split < S) {
    k0 = split * KS;
    k1 = min(L, k0 + KS);
  } else {
    k0 = L;
    k1 = L + n;
  }

  // Q fragments: lane holds Q[row][c*16 + half*8 .. +8] for c < D/16
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = q + (((int64_t)b * N + (row_ok ? node : 0)) * Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint4 raw = row_ok ? *reinterpret_cast<const uint4*>(qp + c * 16 + half * 8)
                         : make_uint4(0, 0, 0, 0);
      qf[c] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  uint64_t anc_word_cache = 0;
  int anc_word_idx = -1;
  const uint64_t* arow = anc + ((int64_t)b * N + (row_ok ? node : 0)) * W;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const uint16_t* kbase = kc + ((int64_t)b * Hkv + g) * (int64_t)cap * D;
  const uint16_t* vbase = vc + ((int64_t)b * Hkv + g) * (int64_t)cap * D;
  constexpr int kChunksPerRow = D / 8;  // 16-byte pieces per key row

  for (int kt = k0; kt < k1; kt += kTile) {
    // ---- stage K (row-major) and V (transposed) for keys kt .. kt+31
    for (int idx = tid; idx < kTile * kChunksPerRow; idx += nthreads) {
      const int key = idx / kChunksPerRow;
      const int col = (idx % kChunksPerRow) * 8;
      uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
      if (kt + key < k1) {
        kr = *reinterpret_cast<const uint4*>(kbase + (int64_t)(kt + key) * D + col);
        vr = *reinterpret_cast<const uint4*>(vbase + (int64_t)(kt + key) * D + col);
      }
      *reinterpret_cast<uint4*>(&Ks[key * KPAD + col]) = kr;
      const uint16_t* vv = reinterpret_cast<const uint16_t*>(&vr);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vt[(col + j) * VPAD + key] = vv[j];
    }
    __syncthreads();

    // ---- visibility of this tile's keys (the ancestor mask on the tree
    // tile).  Computed before the matrix products so that their results are
    // consumed in straight-line code: the MFMA result latency is covered by
    // the wait states the compiler inserts inside one basic block.
    uint32_t tmask = 0xFFFFFFFFu;
    if (split == S) {
      const int j0 = kt - L;  // multiple of 32
      const int wi = j0 >> 6;
      if (wi != anc_word_idx) {
        anc_word_cache = row_ok ? arow[wi] : 0ull;
        anc_word_idx = wi;
      }
      tmask = (uint32_t)(anc_word_cache >> (j0 & 63));
    }
    uint32_t vis = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = 8 * (i >> 2) + 4 * half + (i & 3);
      const bool ok = row_ok && (kt + kl < k1) && ((tmask >> kl) & 1u);
      vis |= (ok ? 1u : 0u) << i;
    }

    // ---- S^T = K Q^T  (32 keys x 32 rows)
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 a =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&Ks[l32 * KPAD + c * 16 + half * 8]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s, 0, 0, 0);
    }

    // ---- online softmax (log2 domain)
    float x[16];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = ((vis >> i) & 1u) ? s[i] * scale_log2 : -__builtin_inff();
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    float alpha, psum = 0.f;
    float p[16];
    if (m_new == -__builtin_inff()) {
      alpha = 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = 0.f;
    } else {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
        psum += p[i];
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 bp;
#pragma unroll
      for (int j = 0; j < 8; ++j) bp[j] = (__bf16)p[8 * t + j];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vrow = &Vt[(32 * db + l32) * VPAD + 4 * half + 16 * t];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        const uint4 raw = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw), bp,
                                                          oacc[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- partials.  The accumulators were last written by an MFMA in the
  // loop body, a different basic block: wait out the result latency before
  // the stores read them.
  __builtin_amdgcn_s_sleep(2);
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const int64_t pr = (((int64_t)split * batch + b) * N + node) * Hq + h;
    if (half == 0) {
      Mpart[pr] = m_run;
      Lpart[pr] = l_tot;
    }
    float* op = Opart + pr * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * half;
        *reinterpret_cast<float4*>(op + d0) =
            make_float4(oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2],
                        oacc[db][4 * j + 3]);
      }
  }
}

// Merge the S + 1 partials of every (sequence, node, head) row.
template <typename OutT>
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ Opart,
                                                     const float* __restrict__ Mpart,
                                                     const float* __restrict__ Lpart,
                                                     const int* __restrict__ n_nodes, int batch,
                                                     int N, int Hq, int D, int S1,
                                                     OutT* __restrict__ out,
                                                     float* __restrict__ lse) {
  const int64_t rowid = blockIdx.x;  // (b * N + node) * Hq + h
  const int b = (int)(rowid / ((int64_t)N * Hq));
  const int node = (int)((rowid / Hq) % N);
  const bool ok = node < min(n_nodes[b], N);
  const int64_t plane = (int64_t)batch * N * Hq;
  float M = -__builtin_inff();
  if (ok)
    for (int s = 0; s < S1; ++s) M = fmaxf(M, Mpart[s * plane + rowid]);
  float lsum = 0.f;
  if (ok && M != -__builtin_inff())
    for (int s = 0; s < S1; ++s) {
      const float ms = Mpart[s * plane + rowid];
      if (ms != -__builtin_inff()) lsum += exp2f(ms - M) * Lpart[s * plane + rowid];
    }
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    if (ok && lsum > 0.f)
      for (int s = 0; s < S1; ++s) {
        const float ms = Mpart[s * plane + rowid];
        if (ms != -__builtin_inff()) acc += exp2f(ms - M) * Opart[(s * plane + rowid) * D + d];
      }
    const float o = (ok && lsum > 0.f) ? acc / lsum : 0.f;
    if constexpr (sizeof(OutT) == 2)
      out[rowid * D + d] = f32_to_bf16_bits(o);
    else
      out[rowid * D + d] = o;
  }
  if (lse && threadIdx.x == 0)
    lse[rowid] = (ok && lsum > 0.f) ? (M + log2f(lsum)) * 0.69314718055994531f
                                    : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// fp32 path: one workgroup per (sequence, node, head); two passes over keys.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_attn_f32(const float* __restrict__ q,
                                                 const float* __restrict__ kc,
                                                 const float* __restrict__ vc,
                                                 const int* __restrict__ ctx_len,
                                                 const uint64_t* __restrict__ anc,
                                                 const int* __restrict__ n_nodes, int N, int Hq,
                                                 int Hkv, int D, int cap, float scale,
                                                 float* __restrict__ out,
                                                 float* __restrict__ lse) {
  __shared__ float qs[128];
  __shared__ float ps[256];
  __shared__ float red[256 / WAVE];
  const int64_t rowid = blockIdx.x;
  const int b = (int)(rowid / ((int64_t)N * Hq));
  const int node = (int)((rowid / Hq) % N);
  const int h = (int)(rowid % Hq);
  const int g = h / (Hq / Hkv);
  const int n = min(n_nodes[b], N);
  const int tid = threadIdx.x;
  if (node >= n) {
    for (int d = tid; d < D; d += 256) out[rowid * D + d] = 0.f;
    if (lse && tid == 0) lse[rowid] = -__builtin_inff();
    return;
  }
  const int L = min(max(ctx_len[b], 0), cap - N);
  const int W = (N + 63) / 64;
  const uint64_t* arow = anc + ((int64_t)b * N + node) * W;
  const float* kb = kc + ((int64_t)b * Hkv + g) * (int64_t)cap * D;
  const float* vb = vc + ((int64_t)b * Hkv + g) * (int64_t)cap * D;
  for (int d = tid; d < D; d += 256) qs[d] = q[rowid * D + d];
  __syncthreads();
  const int nk = L + n;
  auto visible = [&](int key) {
    if (key < L) return true;
    const int j = key - L;
    return ((arow[j >> 6] >> (j & 63)) & 1ull) != 0ull;
  };
  auto score = [&](int key) {
    const float* kr = kb + (int64_t)key * D;
    float a = 0.f;
    for (int d = 0; d < D; ++d) a += qs[d] * kr[d];
    return a * scale;
  };
  float mx = -__builtin_inff();
  for (int key = tid; key < nk; key += 256)
    if (visible(key)) mx = fmaxf(mx, score(key));
  mx = wave_max_f(mx);
  if (tid % WAVE == 0) red[tid / WAVE] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < 256 / WAVE; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float acc = 0.f, lsum = 0.f;
  for (int k0 = 0; k0 < nk; k0 += 256) {
    const int key = k0 + tid;
    ps[tid] = (key < nk && visible(key)) ? __expf(score(key) - mx) : 0.f;
    __syncthreads();
    const int cnt = min(256, nk - k0);
    for (int j = 0; j < cnt; ++j) {
      const float pj = ps[j];
      lsum += pj;
      if (tid < D && pj != 0.f) acc += pj * vb[(int64_t)(k0 + j) * D + tid];
    }
    __syncthreads();
  }
  if (tid < D) out[rowid * D + tid] = acc / lsum;
  if (lse && tid == 0) lse[rowid] = mx + __logf(lsum);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
AttnPlan attention_plan(int batch, int N, int Hq, int Hkv, int D, int max_ctx, int splits) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  p.rows_per_kv = G * N;
  p.row_blocks = (p.rows_per_kv + 31) / 32;
  p.mtiles = (p.row_blocks + kAttnMaxWaves - 1) / kAttnMaxWaves;
  p.waves = (p.row_blocks + p.mtiles - 1) / p.mtiles;
  const int tiles_ctx = std::max(1, (max_ctx + kTile - 1) / kTile);
  int S = splits;
  if (S <= 0) {
    // enough workgroups for ~2 per CU, at least 16 key tiles per split
    const int64_t wg_per_split = (int64_t)batch * Hkv * p.mtiles;
    S = (int)std::max<int64_t>(1, (512 + wg_per_split - 1) / wg_per_split);
    S = std::min(S, std::max(1, tiles_ctx / 16));
  }
  S = std::max(1, std::min(S, tiles_ctx));
  p.splits = S;
  p.keys_per_split = ((tiles_ctx + S - 1) / S) * kTile;
  const size_t rows = (size_t)(S + 1) * batch * N * Hq;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.off_o = take(rows * D * sizeof(float));
  p.off_ml = take(rows * 2 * sizeof(float));
  p.workspace = off;
  return p;
}

hipError_t launch_attention(const AttnPlan& p, const void* q, const void* k, const void* v,
                            bool bf16, const int* ctx_len, const uint64_t* anc,
                            const int* n_nodes, int batch, int N, int Hq, int Hkv, int D,
                            int cap, int max_ctx, float scale, void* out, float* lse,
                            void* ws, hipStream_t stream) {
  (void)max_ctx;
  const int64_t rows = (int64_t)batch * N * Hq;
  if (!bf16) {
    hipLaunchKernelGGL(k_attn_f32, dim3((unsigned)rows), dim3(256), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), ctx_len, anc, n_nodes, N, Hq, Hkv, D, cap,
                       scale, static_cast<float*>(out), lse);
    return hipGetLastError();
  }
  char* w = static_cast<char*>(ws);
  float* Opart = reinterpret_cast<float*>(w + p.off_o);
  const size_t prow = (size_t)(p.splits + 1) * rows;
  float* Mpart = reinterpret_cast<float*>(w + p.off_ml);
  float* Lpart = Mpart + prow;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(p.splits + 1, p.mtiles, batch * Hkv);
  dim3 block(p.waves * WAVE);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  if (D == 128)
    hipLaunchKernelGGL((k_attn_partial<128>), grid, block, 0, stream, q16, k16, v16, ctx_len,
                       anc, n_nodes, N, Hq, Hkv, cap, p.splits, p.keys_per_split, scale_log2,
                       Opart, Mpart, Lpart, batch);
  else
    hipLaunchKernelGGL((k_attn_partial<64>), grid, block, 0, stream, q16, k16, v16, ctx_len,
                       anc, n_nodes, N, Hq, Hkv, cap, p.splits, p.keys_per_split, scale_log2,
                       Opart, Mpart, Lpart, batch);
  hipLaunchKernelGGL((k_attn_combine<uint16_t>), dim3((unsigned)rows), dim3(128), 0, stream,
                     Opart, Mpart, Lpart, n_nodes, batch, N, Hq, D, p.splits + 1,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace tvk
