// tv_device.h -- device-side building blocks shared by the gfx950 kernels of
// libtreeverify: the fixed-point softmax weight, Philox4x64-10, 64-lane
// wavefront helpers and a block-wide top-k.
//
// Every translation unit that uses weight_f / weight / Philox for an integer
// decision is compiled with -ffp-contract=off: each float operation below is
// one IEEE operation in the order written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tvk {

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// Fixed-point weight of logit l in a row with maximum m at inverse
// temperature inv_t: W = rint(exp32(x) * 2^44) for x = fl32(fl32(l - m) *
// inv_t), where exp32 is e^x for fp32 x <= 0 and 0 below -32: Cody-Waite
// reduction x = n ln2 + r with n = rint(x * log2e) and ln2 split into a high
// part with 12 significand bits (0x3f317000) and the fp32 rounding of the
// remainder (0x3805fdf4); e^r from its Taylor series to degree 7
// (coefficients fp32(1/i!)) by Horner with fused multiply-adds; the result
// scaled by 2^n exactly.
//
// The evaluation below gives the same W with fewer instructions:
//   * x is clamped at -33 instead of tested against -32: every x below -32
//     has W = 0 either way (e^-32 * 2^44 = 0.22 rounds to 0, and so does the
//     polynomial's value), and NaN (an all -inf row) clamps to -33 as well;
//   * n comes from adding 1.5 * 2^23 + 44 to x * log2e: the sum rounds to an
//     integer (nearest even, as rint does; |x log2e| < 48), its difference
//     with that constant is n exactly, and its low bits hold n + 44;
//   * 2^n * 2^44 is applied by adding (n + 44) << 23 to the bits of the
//     polynomial's value p in [0.70, 1.42]: the product stays a normal
//     number (0.7 * 2^-4 and up), so this is the exact scaling; the 0x4B4
//     exponent bits of the sum shift out of the 32-bit word.
// UNIT = (inv_t == 1): x = l - m without the multiply (the same value).
// weight_f returns W as an integer-valued float (exact: at most 2^44, and
// fp32 holds every integer it rounds to); such integers also add exactly in
// fp64 while a sum stays below 2^53, i.e. for up to 512 weights, which is
// how the streaming kernels sum them before one conversion to uint64.
// ---------------------------------------------------------------------------
template <bool UNIT = false>
__device__ __forceinline__ float weight_f(float l, float m, float inv_t) {
  const float kLog2e = __builtin_bit_cast(float, 0x3fb8aa3bu);
  const float kLn2Hi = __builtin_bit_cast(float, 0x3f317000u);
  const float kLn2Lo = __builtin_bit_cast(float, 0x3805fdf4u);
  const float kRound = 12582956.0f;  // 1.5 * 2^23 + 44
  const float c7 = __builtin_bit_cast(float, 0x39500d01u);
  const float c6 = __builtin_bit_cast(float, 0x3ab60b61u);
  const float c5 = __builtin_bit_cast(float, 0x3c088889u);
  const float c4 = __builtin_bit_cast(float, 0x3d2aaaabu);
  const float c3 = __builtin_bit_cast(float, 0x3e2aaaabu);
  const float c2 = 0.5f;
  const float d = l - m;
  float x = UNIT ? d : d * inv_t;
  x = __builtin_fmaxf(x, -33.0f);
  const float t = x * kLog2e;
  const float f = t + kRound;  // kRound + rint(t)
  const float n = f - kRound;  // rint(t), exact
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = c7;
  p = __builtin_fmaf(p, r, c6);
  p = __builtin_fmaf(p, r, c5);
  p = __builtin_fmaf(p, r, c4);
  p = __builtin_fmaf(p, r, c3);
  p = __builtin_fmaf(p, r, c2);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  const uint32_t s =
      __builtin_bit_cast(uint32_t, p) + (__builtin_bit_cast(uint32_t, f) << 23);  // p 2^(n+44)
  return __builtin_rintf(__builtin_bit_cast(float, s));
}

__device__ __forceinline__ uint64_t weight(float l, float m, float inv_t) {
  return (uint64_t)weight_f(l, m, inv_t);
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon et al., SC'11).
// ---------------------------------------------------------------------------
struct u64x4 {
  uint64_t v[4];
};

__device__ __forceinline__ u64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                               uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    uint64_t n0 = hi1 ^ c1 ^ k0;
    uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  u64x4 r;
  r.v[0] = c0;
  r.v[1] = c1;
  r.v[2] = c2;
  r.v[3] = c3;
  return r;
}

constexpr uint64_t kResidualSlot = 0xFFFFFFFFull;

// ---------------------------------------------------------------------------
// rotary position embedding: dimension i < D/2 pairs with i + D/2 and the pair
// turns by the angle pos * base^(-2i/D) (the half-split pairing of the
// standard rotary embedding)
// ---------------------------------------------------------------------------
// pair i's angle per unit of position, in revolutions: base^(-2i/D) / (2 pi)
__device__ __forceinline__ double rope_rate(int i, int D, double log2_base) {
  return exp2(-2.0 * (double)i / (double)D * log2_base) * 0.15915494309189535;
}

// sin and cos of position pos at `rate`: pos * rate in fp64, reduced to
// f in [-1/2, 1/2] revolutions, then the hardware sine and cosine, which take
// their argument in revolutions (max abs error 1.3e-7 over that range,
// measured against fp64 at 2^22 points)
__device__ __forceinline__ void rope_sincos(int pos, double rate, float& s, float& c) {
  const double r = (double)pos * rate;
  const float f = (float)(r - rint(r));
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

// ---------------------------------------------------------------------------
// element loads
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t h) { return bf16_to_f32(h); }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
};

// E consecutive elements [i0, i0 + E) of a row as fp32, with 16-byte vector
// loads when the run is inside the row and aligned; -inf past the end.
template <typename T, int E>
__device__ __forceinline__ void load_run(const T* p, int i0, int V, float (&x)[E]);

template <int E>
__device__ __forceinline__ void load_run(const float* p, int i0, int V, float (&x)[E]) {
  static_assert(E % 4 == 0, "runs of whole float4s");
  if (i0 + E <= V && ((i0 | V) & 3) == 0) {
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

template <int E>
__device__ __forceinline__ void load_run(const uint16_t* p, int i0, int V, float (&x)[E]) {
  static_assert(E % 8 == 0, "runs of whole 16-byte vectors");
  if (i0 + E <= V && ((i0 | V) & 7) == 0) {
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
      x[j] = i0 + j < V ? __builtin_bit_cast(float, (uint32_t)p[i0 + j] << 16)
                        : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// wavefront helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int readlane_i(int v, int l) {
  return __builtin_amdgcn_readlane(v, l);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  return __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), l));
}

// the value held by lane (lane ^ 32): the gfx950 lane-swap instruction swaps
// the upper half of the first operand with the lower half of the second
__device__ __forceinline__ float xor32_f(float v) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return __builtin_bit_cast(float, (uint32_t)((lane_id() & 32) ? p[0] : p[1]));
}

// ---------------------------------------------------------------------------
// Wave scans and reductions by DPP: row shifts (within rows of 16 lanes)
// then row broadcasts (lane 15 into the next row, lane 31 into rows 2 and 3),
// the standard inclusive-scan pattern; a lane without a source reads the
// operation's identity.  Reductions read the total from lane 63.  All 64
// lanes must be active.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_or(uint32_t identity, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_or<CTRL, ROWS>(0u, (uint32_t)v);
  const uint32_t hi = dpp_or<CTRL, ROWS>(0u, (uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// inclusive prefix sum over lanes
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v += dpp_u64<0x111, 0xF>(v);
  v += dpp_u64<0x112, 0xF>(v);
  v += dpp_u64<0x114, 0xF>(v);
  v += dpp_u64<0x118, 0xF>(v);
  v += dpp_u64<0x142, 0xA>(v);
  v += dpp_u64<0x143, 0xC>(v);
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  return readlane_u64(wave_incl_scan_u64(v), WAVE - 1);
}
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += (int)dpp_or<0x111, 0xF>(0u, (uint32_t)v);
  v += (int)dpp_or<0x112, 0xF>(0u, (uint32_t)v);
  v += (int)dpp_or<0x114, 0xF>(0u, (uint32_t)v);
  v += (int)dpp_or<0x118, 0xF>(0u, (uint32_t)v);
  v += (int)dpp_or<0x142, 0xA>(0u, (uint32_t)v);
  v += (int)dpp_or<0x143, 0xC>(0u, (uint32_t)v);
  return v;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v) {
  const uint32_t ninf = 0xFF800000u;
  return fmaxf(v, __builtin_bit_cast(float, dpp_or<CTRL, ROWS>(ninf, __builtin_bit_cast(uint32_t, v))));
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = dpp_max_step<0x111, 0xF>(v);
  v = dpp_max_step<0x112, 0xF>(v);
  v = dpp_max_step<0x114, 0xF>(v);
  v = dpp_max_step<0x118, 0xF>(v);
  v = dpp_max_step<0x142, 0xA>(v);
  v = dpp_max_step<0x143, 0xC>(v);
  return readlane_f(v, WAVE - 1);
}

// Inclusive scans over the wave by DPP row shifts (within rows of 16 lanes)
// and row broadcasts (lane 15 into the next row, lane 31 into rows 2 and 3);
// lanes with no source read 0.  For non-negative ints (sum and max).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, true);
}
__device__ __forceinline__ int wave_scan_add_dpp(int v) {
  v += dpp_i<0x111>(v);       // row_shr:1
  v += dpp_i<0x112>(v);       // row_shr:2
  v += dpp_i<0x114>(v);       // row_shr:4
  v += dpp_i<0x118>(v);       // row_shr:8
  v += dpp_i<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_i<0x143, 0xC>(v);  // row_bcast:31
  return v;
}
__device__ __forceinline__ int wave_scan_max_dpp(int v) {
  v = max(v, dpp_i<0x111>(v));
  v = max(v, dpp_i<0x112>(v));
  v = max(v, dpp_i<0x114>(v));
  v = max(v, dpp_i<0x118>(v));
  v = max(v, dpp_i<0x142, 0xA>(v));
  v = max(v, dpp_i<0x143, 0xC>(v));
  return v;
}

// ---------------------------------------------------------------------------
// (value, id) order used by top-k and argmax: larger value first, then the
// smaller id.  Ids of padding entries are >= the vocabulary and distinct.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool vi_better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Argmax over a wave of (value, id) pairs in the order above.
template <int CTRL, int ROWS>
__device__ __forceinline__ void dpp_argmax_step(float& v, int& id) {
  const float ov = __builtin_bit_cast(
      float, dpp_or<CTRL, ROWS>(0xFF800000u, __builtin_bit_cast(uint32_t, v)));
  const int oi = (int)dpp_or<CTRL, ROWS>(0x7FFFFFFFu, (uint32_t)id);
  if (vi_better(ov, oi, v, id)) {
    v = ov;
    id = oi;
  }
}
// the wave's best (value, id) in every lane
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  dpp_argmax_step<0x111, 0xF>(v, id);
  dpp_argmax_step<0x112, 0xF>(v, id);
  dpp_argmax_step<0x114, 0xF>(v, id);
  dpp_argmax_step<0x118, 0xF>(v, id);
  dpp_argmax_step<0x142, 0xA>(v, id);
  dpp_argmax_step<0x143, 0xC>(v, id);
  v = readlane_f(v, WAVE - 1);
  id = readlane_i(id, WAVE - 1);
}

// ---------------------------------------------------------------------------
// Order keys: (value, id) pairs in the order above as one unsigned 64-bit
// integer, larger = better: the float's bits made monotone (negative values
// bit-inverted, the sign bit set on the others; -0 is taken as +0, which
// compares equal to it), then the inverted id.  Logits are never NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t order_key(float v, int id) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);  // -0 -> +0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t k = (uint32_t)(key >> 32);
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ int key_id(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)key);
}
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// one step of a wave-wide u64 minimum (lanes without a source read ~0)
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_min_u64_step(uint64_t v) {
  const uint32_t lo = dpp_or<CTRL, ROWS>(0xFFFFFFFFu, (uint32_t)v);
  const uint32_t hi = dpp_or<CTRL, ROWS>(0xFFFFFFFFu, (uint32_t)(v >> 32));
  return umin64(v, ((uint64_t)hi << 32) | lo);
}
// minimum over the wave (every lane gets it)
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  v = dpp_min_u64_step<0x111, 0xF>(v);
  v = dpp_min_u64_step<0x112, 0xF>(v);
  v = dpp_min_u64_step<0x114, 0xF>(v);
  v = dpp_min_u64_step<0x118, 0xF>(v);
  v = dpp_min_u64_step<0x142, 0xA>(v);
  v = dpp_min_u64_step<0x143, 0xC>(v);
  return readlane_u64(v, WAVE - 1);
}

// ---------------------------------------------------------------------------
// Block-wide top-k (k <= 64) of E (value, id) items per thread, in the order
// above.  Result: out_v / out_i [k] in LDS-or-global memory, best first.
// Items with id >= first_pad are padding: they never enter the result; if
// fewer than k real items exist, the remaining slots hold (-inf,
// pad_base + slot).
//
// Each wave takes the k-th best of its 64 per-thread maxima as a threshold
// (every item of the wave's top-k is at least as good, so the survivors
// contain the block's top-k), keeps the items at least as good as its
// threshold, and the survivors are ranked by counting.  All comparisons are
// on order keys; the counting reads LDS in batches of eight.  If a wave
// keeps more than kCap items (heavy ties) the block falls back to k rounds
// of argmax.  Requires blockDim.x == NT, a multiple of 64, and the scratch
// below.
// ---------------------------------------------------------------------------
template <int NT>
struct TopkScratch {
  static constexpr int kWaves = NT / WAVE;
  static constexpr int kCap = 256;
  uint64_t sk[kWaves * kCap];  // survivors' keys, per-wave segments
  union {
    uint64_t lk[NT];  // per-thread best keys
    float lf[NT];     // or best values
  };
  int wcount[kWaves];
  int overflow;
  float rv[kWaves];
  int ri[kWaves];
};

template <int NT, int E>
__device__ void block_topk(float (&val)[E], int (&id)[E], int k, TopkScratch<NT>& sc,
                           float* out_v, int* out_i, int first_pad = 0x7fffffff,
                           int pad_base = 0x7fffffff) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
  constexpr int kCap = TopkScratch<NT>::kCap;
  constexpr int kW = NT / WAVE;
  if (tid == 0) sc.overflow = 0;
  // Survivors: the real items at least as good as the wave threshold, the
  // k-th best of the 64 lane bests (the worst one if fewer than k lanes hold
  // a real item).  They hold every item of the wave's top k, and only they
  // are ranked.  Without a NaN in the block the threshold and the test use
  // the float values (items tied with the threshold survive too), and only
  // the survivors get keys; with one, the keys decide throughout (their
  // order puts NaNs outside +-inf, which float compares do not see).
  float fbest = -__builtin_inff();
  bool nan_here = false;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    nan_here |= val[e] != val[e];
    fbest = id[e] < first_pad ? fmaxf(fbest, val[e]) : fbest;
  }
  sc.lf[tid] = fbest;
  int cnt = 0, incl, total;
  if (!__syncthreads_or(nan_here)) {  // also publishes the overflow flag
    const float* wf = sc.lf + wave * WAVE;
    int rank = 0;
#pragma unroll
    for (int j0 = 0; j0 < WAVE; j0 += 16) {
      float o[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) o[q] = wf[j0 + q];
#pragma unroll
      for (int q = 0; q < 16; ++q) rank += o[q] > fbest ? 1 : 0;
    }
    // the smallest best whose rank is below k (wave minimum as -max(-x))
    const float thr = -wave_max_f(rank < k ? -fbest : -__builtin_inff());
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += (id[e] < first_pad && val[e] >= thr) ? 1 : 0;
    incl = wave_incl_scan_i(cnt);
    total = readlane_i(incl, WAVE - 1);
    if (total > kCap) {
      if (lane == 0) sc.overflow = 1;
    } else {
      int off = wave * kCap + incl - cnt;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (id[e] < first_pad && val[e] >= thr) sc.sk[off++] = order_key(val[e], id[e]);
    }
  } else {
    // keys (padding: 0, below every real key) and the per-thread best
    uint64_t key[E];
    uint64_t best = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      key[e] = id[e] < first_pad ? order_key(val[e], id[e]) : 0ull;
      best = best > key[e] ? best : key[e];
    }
    sc.lk[tid] = best;
    __syncthreads();
    const uint64_t* wk = sc.lk + wave * WAVE;
    int rank = 0;
#pragma unroll
    for (int j0 = 0; j0 < WAVE; j0 += 16) {
      uint64_t o[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) o[q] = wk[j0 + q];
#pragma unroll
      for (int q = 0; q < 16; ++q) rank += o[q] > best ? 1 : 0;
    }
    const uint64_t thr = wave_min_u64(rank < k ? best : ~0ull);
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += (key[e] != 0 && key[e] >= thr) ? 1 : 0;
    incl = wave_incl_scan_i(cnt);
    total = readlane_i(incl, WAVE - 1);
    if (total > kCap) {
      if (lane == 0) sc.overflow = 1;
    } else {
      int off = wave * kCap + incl - cnt;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (key[e] != 0 && key[e] >= thr) sc.sk[off++] = key[e];
    }
  }
  if (lane == 0) sc.wcount[wave] = total;
  __syncthreads();
  if (!sc.overflow) {
    // rank survivors by counting the better ones
    int wc[kW], nsurv = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      wc[w] = sc.wcount[w];
      nsurv += wc[w];
    }
    for (int t = tid; t < nsurv; t += NT) {
      int w = 0, loc = t;
#pragma unroll
      for (int w2 = 0; w2 < kW - 1; ++w2)
        if (w == w2 && loc >= wc[w2]) {
          loc -= wc[w2];
          w = w2 + 1;
        }
      const uint64_t x = sc.sk[w * kCap + loc];
      int r = 0;
#pragma unroll
      for (int w2 = 0; w2 < kW; ++w2) {
        const uint64_t* seg = sc.sk + w2 * kCap;
        for (int j0 = 0; j0 < wc[w2]; j0 += 8) {
          uint64_t o[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) o[q] = seg[min(j0 + q, wc[w2] - 1)];
#pragma unroll
          for (int q = 0; q < 8; ++q) r += (j0 + q < wc[w2] && o[q] > x) ? 1 : 0;
        }
      }
      if (r < k) {
        out_v[r] = key_value(x);
        out_i[r] = key_id(x);
      }
    }
    for (int r = nsurv + tid; r < k; r += NT) {
      out_v[r] = -__builtin_inff();
      out_i[r] = pad_base + r;
    }
    __syncthreads();
    return;
  }
  // fallback: k rounds of block argmax, removing the winner each round
  bool taken[E];
#pragma unroll
  for (int e = 0; e < E; ++e) taken[e] = false;
  for (int r = 0; r < k; ++r) {
    float mv = -__builtin_inff();
    int mi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (!taken[e] && id[e] < first_pad && vi_better(val[e], id[e], mv, mi)) {
        mv = val[e];
        mi = id[e];
      }
    wave_argmax(mv, mi);
    if (lane == 0) {
      sc.rv[wave] = mv;
      sc.ri[wave] = mi;
    }
    __syncthreads();
    float gv = sc.rv[0];
    int gi = sc.ri[0];
    for (int w = 1; w < NT / WAVE; ++w)
      if (vi_better(sc.rv[w], sc.ri[w], gv, gi)) {
        gv = sc.rv[w];
        gi = sc.ri[w];
      }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (id[e] == gi && val[e] == gv) taken[e] = true;
    if (tid == 0) {
      const bool real = gi < first_pad;
      out_v[r] = real ? gv : -__builtin_inff();
      out_i[r] = real ? gi : pad_base + r;
    }
    __syncthreads();
  }
}

}  // namespace tvk
