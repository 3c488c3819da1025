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
//     V is staged row-major, as it sits in the cache, and the A operand
//     (8 keys of one d per lane) comes from two transposing LDS reads
//     (ds_read_b64_tr_b16: within each 16-lane group, lane 4p + q receives
//     element q of the 8-byte rows addressed by lanes p, p + 4, p + 8, p + 12);
//   * split-K over the context: split s < S covers keys [s*KS, (s+1)*KS), the
//     extra split S covers the tree keys with the ancestor mask (the only
//     masked tile); partials (m, l, O) go to the workspace and k_combine
//     merges them with their log-sum-exp weights.
// f32 path: a plain vector-ALU kernel (used for fp32 inputs).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "tv_device.h"
#include "tv_internal.h"

namespace tvk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileKeys = 64;  // keys one wave takes per iteration (two 32-key MFMA sub-tiles)
constexpr int kAttnWaves = 4;  // row blocks per workgroup, 32 query rows each
constexpr int kAttnKH = 2;     // waves per row block: they split each staged tile's keys
constexpr int kAttnThreads = kAttnWaves * WAVE * kAttnKH;
constexpr float kRescaleSlack = 8.0f;  // log2 units: running weights stay below 2^8

typedef short s16x4 __attribute__((ext_vector_type(4)));

// transposing 8-byte LDS read (see the layout note above)
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_s16x4*>(reinterpret_cast<uintptr_t>(p) & 0xFFFFFFFFu));
}


__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its outstanding global loads (a prefetch stays in
// flight across it).  __syncthreads() would also drain the global loads.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


// Work items are (sequence x KV head, split, row tile).  Workgroups are
// dispatched round-robin over the 8 XCDs (workgroup w runs on XCD w % 8).
// The row tiles of one (KV head, split) read the same K/V tiles, so they run
// on one XCD and share its L2; consecutive (KV head, split) units go to
// different XCDs, so that sequences of different context lengths spread over
// all of them.
//
// Within a workgroup, the kAttnKH waves of one row block take the kAttnKH
// 64-key quarters of every staged tile (two waves per SIMD), each with its own
// online softmax; their (m, l, O) are merged through LDS at the end.
template <int D, bool ROPE>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn_partial(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int* __restrict__ ctx_len,
    const uint64_t* __restrict__ anc, const int* __restrict__ n_nodes, int N, int Hq, int Hkv,
    int cap, int S, int KS, int MT, int units, float scale_log2, uint16_t* __restrict__ Opart,
    float* __restrict__ Mpart, float* __restrict__ Lpart, int batch, const int* __restrict__ pos,
    double log2_base) {
  constexpr int KP = D + 8;   // K tile pitch (bf16): 16-byte reads spread over banks
  constexpr int VP = D + 16;  // V tile pitch (bf16): the 16 rows of a transposing read
                              // (4 keys x 4 column groups) fall in distinct banks
  constexpr int KCH = D / 8;  // 16-byte chunks per key row
  constexpr int TK = kTileKeys * kAttnKH;       // keys staged per iteration
  constexpr int KLD = TK * KCH / kAttnThreads;  // K (and V) chunks per thread
  // Two K/V tile buffers (one barrier per tile: a wave stages the next tile
  // into the other buffer as soon as it is done with the current one); the
  // rotary variant keeps one, as its tables would not fit beside two
  constexpr bool kDB = !ROPE;
  constexpr int NB = kDB ? 2 : 1;
  __shared__ __align__(16) uint16_t Ks[NB * TK * KP];
  __shared__ __align__(16) uint16_t Vs[NB * TK * VP];
  __shared__ uint64_t Aw[kAttnWaves * 32 * 16];  // ancestor rows (tree split)
  __shared__ double Rt[ROPE ? D / 2 : 1];         // rotary rate of each pair
  __shared__ int Pk[ROPE ? 1024 : 1];             // position ids of the tree keys

  // Unit u = (sequence x KV head, split) goes to XCD u % 8; the XCD's
  // workgroups w = x, x + 8, ... take its units in order, MT row tiles
  // each.  Units are numbered longest first, so that the workgroups that
  // start in a later round of the CUs are the short ones: the full context
  // splits (split fastest), then every unit's last context split (often
  // shorter), then the tree splits.
  const int w = blockIdx.x;
  const int j = w / 8;
  const int u = w % 8 + 8 * (j / MT);
  if (u >= units) return;  // whole workgroup, before any barrier
  const int mt = j % MT;
  const int BG = units / (S + 1);
  int split, bg;
  if (u < BG * (S - 1)) {
    bg = u / (S - 1);
    split = u % (S - 1);
  } else if (u < BG * S) {
    bg = u - BG * (S - 1);
    split = S - 1;
  } else {
    bg = u - BG * S;
    split = S;
  }
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = Hq / Hkv;
  // ctx_len <= max_ctx and max_ctx + N <= cap are preconditions; the clamp
  // keeps every key row inside the cache whatever the caller passes
  const int L = min(max(ctx_len[b], 0), cap - N);
  const int n = min(n_nodes[b], N);
  const int W = (N + 63) / 64;
  const int tid = threadIdx.x;
  const int wave = tid / WAVE, lane = tid % WAVE;
  const int half = lane >> 5, l32 = lane & 31;
  const int rb = wave % kAttnWaves, kh = wave / kAttnWaves;  // row block, key quarter

  const int row0 = (mt * kAttnWaves + rb) * 32;
  const int row = row0 + l32;
  const int node = row / G;
  const int h = g * G + row % G;
  const bool row_ok = node < n;
  const bool wave_active = row0 < G * n;  // uniform per wave

  int k0, k1;
  if (split < S) {
    k0 = split * KS;
    k1 = min(L, k0 + KS);
  } else {
    k0 = L;
    k1 = L + n;
  }

  bf16x8 qf[D / 16];
  {
    // the address does not depend on n_nodes, so the loads leave before the
    // scalar loads of the lengths return; rows past n_nodes are masked in
    // the loop (their scores are replaced, never used)
    const uint16_t* qp = q + (((int64_t)b * N + min(node, N - 1)) * Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + c * 16 + half * 8));
  }
  // rotary embedding at the tree position ids (pos[b][i] = L + depth): the
  // pair rates and, in the tree split, the keys' position ids go to LDS; the
  // queries are turned once the first tile's loads are in flight
  int qpos = 0;
  if constexpr (ROPE) {
    if (tid < D / 2) Rt[tid] = rope_rate(tid, D, log2_base);
    if (split == S)
      for (int j = tid; j < n; j += kAttnThreads) Pk[j] = pos[(int64_t)b * N + j];
    qpos = row_ok ? pos[(int64_t)b * N + node] : 0;
  }
  const uint64_t* arow = anc + ((int64_t)b * N + (row_ok ? node : 0)) * W;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff();
  // in raw score units (none for a scale so small that it would overflow)
  const float rescale_slack = scale_log2 > 1e-30f ? kRescaleSlack / scale_log2 : 0.f;
  float l_run = 0.f;

  const uint16_t* kbase = kc + ((int64_t)b * Hkv + g) * (int64_t)cap * D;
  const uint16_t* vbase = vc + ((int64_t)b * Hkv + g) * (int64_t)cap * D;

  // register prefetch of one tile: 16-byte K and V chunks, row-major, by
  // buffer loads over this head's cache rows (the tile start in the scalar
  // offset, the thread's chunk in a fixed vector offset).  Rows of the last,
  // partial tile past its end are clamped to its last row (always in
  // bounds) and zeroed when staged.
  const uint32_t head_bytes = (uint32_t)cap * D * 2u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, head_bytes, 0x00020000);
  // the thread's KLD 16-byte chunks of a tile: key row and column.  The
  // rotary tree split takes them in pairs (chunk j, chunk j + KCH/2 of one
  // row), the two halves of a rotation pair
  int ckey[KLD], ccol[KLD];
#pragma unroll
  for (int i = 0; i < KLD; ++i) {
    if (ROPE && split == S) {
      const int pi = tid + (i >> 1) * kAttnThreads;
      ckey[i] = pi / (KCH / 2);
      ccol[i] = (pi % (KCH / 2) + (i & 1) * (KCH / 2)) * 8;
    } else {
      const int c = tid + i * kAttnThreads;
      ckey[i] = c / KCH;
      ccol[i] = (c % KCH) * 8;
    }
  }
  uint4 kreg[KLD], vreg[KLD];
  // the first tile of a context split, before ctx_len is known: rows are
  // clamped to the head's last cache row (always in bounds); rows past the
  // split's end are zeroed when staged
  auto fetch_first = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const uint32_t voff = (uint32_t)(min(kt + ckey[i], cap - 1) * D + ccol[i]) * 2u;
      kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, voff, 0, 0));
      vreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff, 0, 0));
    }
  };
  auto fetch = [&](int kt) {
    if (kt + TK <= k1) {  // whole tile
      const uint32_t soff = (uint32_t)kt * D * 2u;
#pragma unroll
      for (int i = 0; i < KLD; ++i) {
        const uint32_t voff = (uint32_t)(ckey[i] * D + ccol[i]) * 2u;
        kreg[i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       krs, voff, soff, 0));
        vreg[i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       vrs, voff, soff, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < KLD; ++i) {
        const uint32_t voff = (uint32_t)(min(kt + ckey[i], k1 - 1) * D + ccol[i]) * 2u;
        kreg[i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       krs, voff, 0, 0));
        vreg[i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       vrs, voff, 0, 0));
      }
    }
  };
  auto stage = [&](int kt, uint16_t* kd, uint16_t* vd) {
    const bool whole = kt + TK <= k1;
    if constexpr (ROPE) {
      if (split == S) {  // tree keys: turn each pair at the key's position id
#pragma unroll
        for (int i = 0; i < KLD; i += 2) {
          const int t = kt - L + ckey[i];
          const int kp = t < n ? Pk[t] : 0;  // rows past the end: position 0 (masked)
          bf16x8 lo = __builtin_bit_cast(bf16x8, kreg[i]);
          bf16x8 hi = __builtin_bit_cast(bf16x8, kreg[i + 1]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float sn, cs;
            rope_sincos(kp, Rt[ccol[i] + e], sn, cs);
            const float xl = (float)lo[e], xh = (float)hi[e];
            lo[e] = (__bf16)(xl * cs - xh * sn);
            hi[e] = (__bf16)(xh * cs + xl * sn);
          }
          kreg[i] = __builtin_bit_cast(uint4, lo);
          kreg[i + 1] = __builtin_bit_cast(uint4, hi);
        }
      }
    }
    // Rows past the end: their scores are masked to -inf, so K needs no
    // clearing, and P is exactly 0 there; V must then be finite.  fetch()
    // clamps such rows to the last real row, but the first tile of a
    // context split is fetched before ctx_len is known, clamped to the
    // cache's last row, whose contents are arbitrary: only that tile's V
    // rows past the end are zeroed (a uniform branch).
    if (!whole && kt == k0 && split < S) {
#pragma unroll
      for (int i = 0; i < KLD; ++i)
        if (kt + ckey[i] >= k1) vreg[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int key = ckey[i], col = ccol[i];
      *reinterpret_cast<uint4*>(&kd[key * KP + col]) = kreg[i];
      *reinterpret_cast<uint4*>(&vd[key * VP + col]) = vreg[i];
    }
  };
  // transposing-read source of this lane: key offset 4 (lane / 32) +
  // (lane % 16) / 4 and column offset 16 ((lane / 16) % 2) + 4 (lane % 4)
  // inside each (16 keys x 32 d) block of the A operand
  const int tr_key = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // The tree split keeps each row's ancestor words in LDS, so the tile loop
  // issues no global load other than the K/V prefetch: waiting for any other
  // load would also wait for the prefetch (the vector memory counter retires
  // in order).
  uint64_t* aw = &Aw[(rb * 32 + l32) * 16];
  if (split == S && half == 0 && kh == 0)
    for (int j = 0; j < W; ++j) aw[j] = row_ok ? arow[j] : 0ull;

  // a context split's first tile starts at split * KS whatever the context
  // length, so its loads leave without waiting for ctx_len
  if (split < S)
    fetch_first(k0);
  else if (k0 < k1)
    fetch(k0);
  if constexpr (ROPE) {
    // the lane's Q elements d = 16 c + 8 half + e hold both members of each
    // pair (d, d + D/2), in chunks c and c + D/32
    lds_barrier();  // Rt and Pk written (the tile loads stay in flight)
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rope_sincos(qpos, Rt[16 * c + 8 * half + e], sn, cs);
        const float lo = (float)qf[c][e], hi = (float)qf[c + D / 32][e];
        qf[c][e] = (__bf16)(lo * cs - hi * sn);
        qf[c + D / 32][e] = (__bf16)(hi * cs + lo * sn);
      }
  }
  // the products and softmax of this wave's 64 keys of the tile at kt0,
  // staged in (Kt, Vt)
  auto compute = [&](int kt0, const uint16_t* Kt, const uint16_t* Vt) {
    const int kt = kt0 + kTileKeys * kh;  // this wave's 64 keys: tile rows kr0 ..
    const int kr0 = kTileKeys * kh;
    if (wave_active && kt < k1) {
      // visibility of the 64 keys, taken before the matrix products so that
      // their results are consumed in straight-line code.  valid bit j =
      // key kt + j exists for this row; the lane's 32 keys are nibbles
      // 0, 2, ..., 14 of (valid >> 4 * half) (the S^T accumulator layout).
      // A whole context tile needs no mask when every row of the wave is live.
      uint32_t vis = row_ok ? 0xFFFFFFFFu : 0u;
      if (split == S || kt + kTileKeys > k1) {
        uint64_t valid = split == S ? (row_ok ? aw[(kt - L) >> 6] : 0ull) : (row_ok ? ~0ull : 0ull);
        if (k1 - kt < 64) valid &= (1ull << (k1 - kt)) - 1ull;
        uint64_t v = (valid >> (4 * half)) & 0x0F0F0F0F0F0F0F0Full;
        v = (v | (v >> 4)) & 0x00FF00FF00FF00FFull;
        v = (v | (v >> 8)) & 0x0000FFFF0000FFFFull;
        v = (v | (v >> 16)) & 0x00000000FFFFFFFFull;
        vis = (uint32_t)v;
      }
      const bool full = __ballot(vis != 0xFFFFFFFFu) == 0;  // wave-uniform

      // S^T = K Q^T for the two 32-key sub-tiles
      f32x16 s0, s1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = 0.f;
        s1[i] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 a0 = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&Kt[(kr0 + l32) * KP + c * 16 + half * 8]));
        const bf16x8 a1 = __builtin_bit_cast(
            bf16x8,
            *reinterpret_cast<const uint4*>(&Kt[(kr0 + 32 + l32) * KP + c * 16 + half * 8]));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[c], s1, 0, 0, 0);
      }

      // online softmax on raw scores (the scale is positive, so the max
      // commutes with it): p = 2^((s - m) * scale * log2 e)
      float x[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = s0[i];
        x[16 + i] = s1[i];
      }
      if (!full) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          x[i] = ((vis >> i) & 1u) ? x[i] : -__builtin_inff();
      }
      float tmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 32; i += 2) tmax = fmaxf(tmax, fmaxf(x[i], x[i + 1]));
      tmax = fmaxf(tmax, xor32_f(tmax));
      // the reference maximum moves only when a score exceeds it by more than
      // kRescaleSlack in the exponent (weights up to 2^kRescaleSlack are fine
      // in fp32 and bf16), so that most tiles skip the rescale
      const bool grow = tmax > m_run + rescale_slack;
      if (__ballot(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - tmax) * scale_log2) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_run = grow ? tmax : m_run;
      }
      const float moff = m_run == -__builtin_inff() ? 0.f : -m_run * scale_log2;
      float p[32];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], scale_log2, moff));
        psum += p[i];
      }
      l_run += psum;

      // O^T += V^T P^T with P rounded to bf16 (the normaliser l keeps the
      // fp32 weights)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 bp;
#pragma unroll
          for (int j = 0; j < 8; ++j) bp[j] = (__bf16)p[16 * ks + 8 * t + j];
          const int rr = kr0 + 32 * ks + 16 * t + tr_key;  // key rows rr and rr + 8
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            // A = V^T: d = 32 db + lane % 32; k-slots 0..3 and 4..7 of the lane
            // are keys 16 t + 4 half + {0..3} and 16 t + 8 + 4 half + {0..3}
            const uint16_t* vsrc = &Vt[rr * VP + 32 * db + tr_col];
            const s16x4 lo = lds_read_tr16(vsrc);
            const s16x4 hi = lds_read_tr16(vsrc + 8 * VP);
            const bf16x8 a =
                __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, oacc[db], 0, 0, 0);
          }
        }
    }
  };

  if constexpr (kDB) {
    // tile t sits in buffer t % 2.  The barrier at the top of an iteration
    // says that every wave has staged the current tile and finished the
    // previous one, whose buffer the next tile then takes.
    if (k0 < k1) {
      stage(k0, Ks, Vs);
      if (k0 + TK < k1) fetch(k0 + TK);
    }
    int sb = 0;
    for (int kt0 = k0; kt0 < k1; kt0 += TK, sb ^= 1) {
      lds_barrier();
      compute(kt0, Ks + sb * (TK * KP), Vs + sb * (TK * VP));
      if (kt0 + TK < k1) {
        stage(kt0 + TK, Ks + (sb ^ 1) * (TK * KP), Vs + (sb ^ 1) * (TK * VP));
        if (kt0 + 2 * TK < k1) fetch(kt0 + 2 * TK);  // in flight during the next products
      }
    }
  } else {
    for (int kt0 = k0; kt0 < k1; kt0 += TK) {
      stage(kt0, Ks, Vs);
      lds_barrier();
      if (kt0 + TK < k1) fetch(kt0 + TK);  // in flight during the products
      compute(kt0, Ks, Vs);
      lds_barrier();
    }
  }
  lds_barrier();  // every tile read done before the buffers serve the exchange

  // ---- partials.  The accumulators were last written by an MFMA in the
  // loop body, a different basic block: wait out the result latency before
  // the stores read them.
  __builtin_amdgcn_s_sleep(2);
  // Merge the key halves of each row block, the two waves splitting the
  // columns: wave kh keeps columns [kh D/2, (kh + 1) D/2).  Each hands its
  // (m, l) and the other half of its O to its partner through LDS (the tile
  // buffers are free: every wave has passed the loop's last barrier),
  // value-major so that consecutive lanes hit consecutive banks; both then
  // rescale to the larger maximum, wave 0's terms first so that the two
  // compute the same l.
  constexpr int DBH = D / 64;       // accumulator blocks per column half
  constexpr int NH = 16 * DBH + 2;  // floats per lane handed over: half of O, m, l
  static_assert(4 * NH * WAVE * 4 <= TK * KP * 2, "exchange fits the K tile");
  static_assert(kAttnKH == 2, "one partner wave per row block");
  float* xbase = reinterpret_cast<float*>(rb < 2 ? Ks : Vs) + (rb & 1) * 2 * NH * WAVE;
  auto epilogue = [&](auto khc) {
    constexpr int KH = decltype(khc)::value;
    constexpr int MINE = KH * DBH, PART = (1 - KH) * DBH;  // accumulator blocks
    float* xmine = xbase + KH * NH * WAVE;
    float* xpart = xbase + (1 - KH) * NH * WAVE;
#pragma unroll
    for (int e = 0; e < DBH; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) xmine[(e * 16 + i) * WAVE + lane] = oacc[PART + e][i];
    xmine[(NH - 2) * WAVE + lane] = m_run;
    xmine[(NH - 1) * WAVE + lane] = l_run;
    lds_barrier();
    const float mp = xpart[(NH - 2) * WAVE + lane], lp = xpart[(NH - 1) * WAVE + lane];
    const float m0 = KH == 0 ? m_run : mp, m1 = KH == 0 ? mp : m_run;
    const float l0 = KH == 0 ? l_run : lp, l1 = KH == 0 ? lp : l_run;
    const float mm = fmaxf(m0, m1);
    const float a0 = m0 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m0 - mm) * scale_log2);
    const float a1 = m1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m1 - mm) * scale_log2);
    const float am = KH == 0 ? a0 : a1, ap = KH == 0 ? a1 : a0;
    f32x16 o[DBH];
#pragma unroll
    for (int e = 0; e < DBH; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        o[e][i] = oacc[MINE + e][i] * am + xpart[(e * 16 + i) * WAVE + lane] * ap;
    const float lm = l0 * a0 + l1 * a1;
    const float l_tot = lm + xor32_f(lm);
    if (KH == 0 && row_ok && half == 0) {
      const int64_t pr = (((int64_t)split * batch + b) * N + node) * Hq + h;
      Mpart[pr] = mm * scale_log2;  // log2 domain (-inf stays -inf)
      Lpart[pr] = l_tot;
    }
    // O / l in fp16 (a weighted mean of V rows, so it stays within V's
    // range).  The accumulator gives a lane 4-column runs of one row; the
    // rows go through the partner's region (read above, written by no one
    // else now) so that every store is a whole 16-byte chunk.  A row's
    // node and head come from the lane that owns it.
    constexpr int OPH = D / 2 + 8;  // LDS row pitch (fp16)
    static_assert(32 * OPH * 2 <= NH * WAVE * 4, "rows fit the region");
    uint16_t* tw = reinterpret_cast<uint16_t*>(xpart);
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int e = 0; e < DBH; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const _Float16 x0 = (_Float16)(o[e][4 * j + 2 * t] * inv_l);
          const _Float16 x1 = (_Float16)(o[e][4 * j + 2 * t + 1] * inv_l);
          w2[t] = (uint32_t)__builtin_bit_cast(uint16_t, x0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
        }
        *reinterpret_cast<uint2*>(&tw[l32 * OPH + 32 * e + 8 * j + 4 * half]) =
            make_uint2(w2[0], w2[1]);
      }
    constexpr int CPH = D / 16;  // 16-byte chunks per half row
#pragma unroll
    for (int k = 0; k < 32 * CPH / WAVE; ++k) {
      const int ch = k * WAVE + lane, r = ch / CPH, c = ch % CPH;
      const uint4 x = *reinterpret_cast<const uint4*>(&tw[r * OPH + c * 8]);
      const int nd = __shfl(node, r), hh = __shfl(h, r);
      if (nd < n) {
        const int64_t pr = (((int64_t)split * batch + b) * N + nd) * Hq + hh;
        *reinterpret_cast<uint4*>(Opart + pr * D + KH * (D / 2) + c * 8) = x;
      }
    }
  };
  if (kh == 0)
    epilogue(std::integral_constant<int, 0>());
  else
    epilogue(std::integral_constant<int, 1>());
}

// Merge the S + 1 partials of every query row.  Partial s holds O_s / l_s in
// fp16; its weight is 2^(m_s - M) l_s / L with L = sum_s 2^(m_s - M) l_s.
// One thread per (row, head, 8 output columns): the D/8 threads of a row
// read the same (m_s, l_s) words.  Up to kOne = 16 partials are loaded in one
// round (with the sequence's node count alongside; rows past it are written
// as zeros), so the kernel waits on memory once; more splits take batches of
// eight, with the maximum found first.  The sum runs over s in order either
// way.
__device__ __forceinline__ void combine_add(float m, float l, uint4 h, float M, float& lsum,
                                            float (&acc)[8]) {
  const bool live = m != -__builtin_inff();
  const float wgt = live ? __builtin_amdgcn_exp2f(m - M) : 0.f;
  const float wl = wgt * l;  // the partial holds O / l
  lsum += wl;
  const uint32_t w[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += wl * (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
    acc[2 * i + 1] += wl * (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}

template <typename OutT>
__global__ __launch_bounds__(256) void k_attn_combine(const uint16_t* __restrict__ Opart,
                                                     const float* __restrict__ Mpart,
                                                     const float* __restrict__ Lpart,
                                                     const int* __restrict__ n_nodes, int batch,
                                                     int N, int Hq, int D, int S1,
                                                     OutT* __restrict__ out,
                                                     float* __restrict__ lse) {
  constexpr int kOne = 16;  // partials loaded in one round
  constexpr int kB = 8;     // splits per load batch beyond that
  const int D8 = D / 8;
  const int64_t plane = (int64_t)batch * N * Hq;
  const int64_t r = (int64_t)blockIdx.x * (256 / D8) + threadIdx.x / D8;  // (b, node, head)
  if (r >= plane) return;
  const int d8 = threadIdx.x % D8;
  const int64_t bn = r / Hq;
  const int b = (int)(bn / N), node = (int)(bn % N);
  OutT* dst = out + r * D + 8 * d8;
  const uint16_t* ob = Opart + r * D + 8 * d8;
  const int nb = n_nodes[b];
  float M = -__builtin_inff();
  float lsum = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (S1 <= kOne) {
    float ms[kOne], ls[kOne];
    uint4 oh[kOne];
#pragma unroll
    for (int j = 0; j < kOne; ++j) {
      if (j < S1) {  // uniform
        ms[j] = Mpart[j * plane + r];
        ls[j] = Lpart[j * plane + r];
        oh[j] = *reinterpret_cast<const uint4*>(ob + j * plane * D);
      } else {
        ms[j] = -__builtin_inff();
        ls[j] = 0.f;
        oh[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (node >= min(nb, N)) goto pad;
#pragma unroll
    for (int j = 0; j < kOne; ++j)
      if (j < S1) M = fmaxf(M, ms[j]);
#pragma unroll
    for (int j = 0; j < kOne; ++j)
      if (j < S1) combine_add(ms[j], ls[j], oh[j], M, lsum, acc);
  } else {
    if (node >= min(nb, N)) goto pad;
    for (int s0 = 0; s0 < S1; s0 += kB) {
      float ms[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j)
        ms[j] = s0 + j < S1 ? Mpart[(s0 + j) * plane + r] : -__builtin_inff();
#pragma unroll
      for (int j = 0; j < kB; ++j) M = fmaxf(M, ms[j]);
    }
    for (int s0 = 0; s0 < S1; s0 += kB) {
      float ms[kB], ls[kB];
      uint4 oh[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int s = min(s0 + j, S1 - 1);
        ms[j] = Mpart[s * plane + r];
        ls[j] = Lpart[s * plane + r];
        oh[j] = *reinterpret_cast<const uint4*>(ob + s * plane * D);
      }
#pragma unroll
      for (int j = 0; j < kB; ++j)
        if (s0 + j < S1) combine_add(ms[j], ls[j], oh[j], M, lsum, acc);
    }
  }
  {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv;
    if constexpr (sizeof(OutT) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)f32_to_bf16_bits(acc[2 * i]) |
               ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      reinterpret_cast<float4*>(dst)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    if (lse && d8 == 0)
      lse[r] = lsum > 0.f ? (M + log2f(lsum)) * 0.69314718055994531f : -__builtin_inff();
    return;
  }
pad:
  if constexpr (sizeof(OutT) == 2) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(0u, 0u, 0u, 0u);
  } else {
    reinterpret_cast<float4*>(dst)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(dst)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (lse && d8 == 0) lse[r] = -__builtin_inff();
}

// ---------------------------------------------------------------------------
// fp32 path: one workgroup per (sequence, node, head); two passes over keys.
// ---------------------------------------------------------------------------
template <bool ROPE>
__global__ __launch_bounds__(256) void k_attn_f32(const float* __restrict__ q,
                                                 const float* __restrict__ kc,
                                                 const float* __restrict__ vc,
                                                 const int* __restrict__ ctx_len,
                                                 const uint64_t* __restrict__ anc,
                                                 const int* __restrict__ n_nodes, int N, int Hq,
                                                 int Hkv, int D, int cap, float scale,
                                                 float* __restrict__ out,
                                                 float* __restrict__ lse,
                                                 const int* __restrict__ pos,
                                                 double log2_base) {
  __shared__ float qs[128];
  __shared__ double rt[ROPE ? 64 : 1];
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
  if constexpr (ROPE) {  // the query and the tree keys turn at their position ids
    if (tid < D / 2) rt[tid] = rope_rate(tid, D, log2_base);
    __syncthreads();
    if (tid < D / 2) {
      float sn, cs;
      rope_sincos(pos[(int64_t)b * N + node], rt[tid], sn, cs);
      const float lo = qs[tid], hi = qs[tid + D / 2];
      qs[tid] = lo * cs - hi * sn;
      qs[tid + D / 2] = hi * cs + lo * sn;
    }
  }
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
    if (ROPE && key >= L) {
      const int kp = pos[(int64_t)b * N + (key - L)];
      for (int d = 0; d < D / 2; ++d) {
        float sn, cs;
        rope_sincos(kp, rt[d], sn, cs);
        const float lo = kr[d], hi = kr[d + D / 2];
        a += qs[d] * (lo * cs - hi * sn) + qs[d + D / 2] * (hi * cs + lo * sn);
      }
    } else {
      for (int d = 0; d < D; ++d) a += qs[d] * kr[d];
    }
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
  p.waves = kAttnWaves;
  p.mtiles = (p.row_blocks + kAttnWaves - 1) / kAttnWaves;
  const int tiles_ctx = std::max(1, (max_ctx + kTileKeys - 1) / kTileKeys);
  // whole staged tiles (kAttnKH 64-key quarters) per split
  auto tiles_per_split = [&](int S) {
    const int tps = (tiles_ctx + S - 1) / S;
    return ((tps + kAttnKH - 1) / kAttnKH) * kAttnKH;
  };
  int S = splits;
  if (S <= 0) {
    // A cost model fitted to measured times on the 256-CU part: one
    // workgroup per CU at a time, each paying a fixed cost (launch,
    // prologue loads, partial stores) plus ~1 us per 64-key tile; then the
    // combine, ~3.5 us plus its partial reads at ~5 TB/s.  One sequence
    // runs in ceil(workgroups / 256) equal rounds.  A batch may hold
    // contexts of any lengths up to max_ctx, so its workgroups differ and
    // the CUs refill as they finish: the work spread over the CUs plus the
    // longest workgroup.  Fewer splits mean longer loops, more splits more
    // workgroups and more partial traffic.
    const int64_t wg_per_split = (int64_t)batch * Hkv * p.mtiles;
    const double part_bytes = (double)batch * N * Hq * (D * 2 + 8);
    double best = 1e300;
    for (int c = 1; c <= std::min(tiles_ctx, 64); ++c) {
      const int tps = tiles_per_split(c);
      const int sp = (tiles_ctx + tps - 1) / tps;
      if (sp != c) continue;  // the same as a smaller count
      const int64_t wgs = wg_per_split * (sp + 1);
      // fixed cost per workgroup: ~6 us for one sequence (prologue loads and
      // partial stores, as measured by in-kernel stamps), more for a ragged
      // batch (its empty splits and uneven rows), both fitted to sweeps
      const double per_wg = (batch == 1 ? 6.0 : 13.0) + tps;
      const double run = batch == 1 ? (double)((wgs + 255) / 256) * per_wg
                                    : (double)wgs * per_wg / 256.0 + per_wg;
      const double cost = run + 3.5 + part_bytes * (sp + 1) / 5e6;
      if (cost < best) {
        best = cost;
        S = c;
      }
    }
  }
  S = std::max(1, std::min(S, tiles_ctx));
  p.keys_per_split = tiles_per_split(S) * kTileKeys;
  p.splits = (tiles_ctx * kTileKeys + p.keys_per_split - 1) / p.keys_per_split;
  const size_t rows = (size_t)(p.splits + 1) * batch * N * Hq;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.off_o = take(rows * D * sizeof(uint16_t));  // fp16 O / l
  p.off_ml = take(rows * 2 * sizeof(float));
  p.workspace = off;
  return p;
}

namespace {
std::atomic<hipEvent_t> g_pre_event{nullptr}, g_mid_event{nullptr};
}  // namespace

void set_attention_events(hipEvent_t before, hipEvent_t between) {
  g_pre_event.store(before);
  g_mid_event.store(between);
}

hipError_t launch_attention(const AttnPlan& p, const void* q, const void* k, const void* v,
                            bool bf16, const int* ctx_len, const uint64_t* anc,
                            const int* n_nodes, int batch, int N, int Hq, int Hkv, int D,
                            int cap, int max_ctx, float scale, void* out, bool out_f32,
                            float* lse, const int* pos, double log2_base, void* ws,
                            hipStream_t stream) {
  (void)max_ctx;
  const int64_t rows = (int64_t)batch * N * Hq;
  const bool rope = pos != nullptr;
  if (!bf16) {
#define TV_F32(R)                                                                              \
  hipLaunchKernelGGL(k_attn_f32<R>, dim3((unsigned)rows), dim3(256), 0, stream,                \
                     static_cast<const float*>(q), static_cast<const float*>(k),               \
                     static_cast<const float*>(v), ctx_len, anc, n_nodes, N, Hq, Hkv, D, cap,  \
                     scale, static_cast<float*>(out), lse, pos, log2_base)
    if (rope)
      TV_F32(true);
    else
      TV_F32(false);
#undef TV_F32
    return hipGetLastError();
  }
  char* w = static_cast<char*>(ws);
  uint16_t* Opart = reinterpret_cast<uint16_t*>(w + p.off_o);
  const size_t prow = (size_t)(p.splits + 1) * rows;
  float* Mpart = reinterpret_cast<float*>(w + p.off_ml);
  float* Lpart = Mpart + prow;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int units = batch * Hkv * (p.splits + 1);
  const int grid = 8 * ((units + 7) / 8) * p.mtiles;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  if (hipEvent_t ev = g_pre_event.load(std::memory_order_relaxed)) {
    const hipError_t e = hipEventRecord(ev, stream);
    if (e != hipSuccess) return e;
  }
#define TV_PARTIAL(DD, R)                                                                   \
  hipLaunchKernelGGL((k_attn_partial<DD, R>), dim3(grid), dim3(kAttnThreads), 0, stream, q16, \
                     k16, v16, ctx_len, anc, n_nodes, N, Hq, Hkv, cap, p.splits,              \
                     p.keys_per_split, p.mtiles, units, scale_log2, Opart, Mpart, Lpart, batch, \
                     pos, log2_base)
  if (D == 128) {
    if (rope)
      TV_PARTIAL(128, true);
    else
      TV_PARTIAL(128, false);
  } else {
    if (rope)
      TV_PARTIAL(64, true);
    else
      TV_PARTIAL(64, false);
  }
#undef TV_PARTIAL
  if (hipEvent_t ev = g_mid_event.load(std::memory_order_relaxed)) {
    const hipError_t e = hipEventRecord(ev, stream);
    if (e != hipSuccess) return e;
  }
  const unsigned cgrid = (unsigned)((rows + (256 / (D / 8)) - 1) / (256 / (D / 8)));
  if (out_f32)
    hipLaunchKernelGGL((k_attn_combine<float>), dim3(cgrid), dim3(256), 0, stream, Opart, Mpart,
                       Lpart, n_nodes, batch, N, Hq, D, p.splits + 1, static_cast<float*>(out),
                       lse);
  else
    hipLaunchKernelGGL((k_attn_combine<uint16_t>), dim3(cgrid), dim3(256), 0, stream, Opart,
                       Mpart, Lpart, n_nodes, batch, N, Hq, D, p.splits + 1,
                       static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace tvk
