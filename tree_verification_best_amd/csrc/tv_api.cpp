// tv_api.cpp -- the C ABI of libtreeverify (declared in include/treeverify.h):
// host-side argument checks, workspace sizing and launches on the caller's
// stream.  No call allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "tv_internal.h"
#include "treeverify.h"

namespace {

constexpr int kMaxGridY = 65535;

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }
bool rope_base_ok(double base) { return std::isfinite(base) && base > 1.0; }

bool build_args_ok(int batch, int K, int V, int topk, int budget) {
  return batch >= 1 && K >= 1 && K <= TV_MAX_POSITIONS && V >= 1 && V <= TV_MAX_VOCAB &&
         topk >= 1 && topk <= TV_MAX_TOPK && topk <= V && budget >= 0 &&
         budget <= TV_MAX_BUDGET && K * topk <= 4096;
}

bool attn_args_ok(int batch, int N, int Hq, int Hkv, int D, int max_ctx, int splits) {
  return batch >= 1 && N >= 1 && N <= 1024 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 &&
         (D == 64 || D == 128) && max_ctx >= 0 && splits >= 0;
}

bool accept_args_ok(int batch, int N, int V, int max_depth) {
  return batch >= 1 && N >= 1 && N <= 1024 && V >= 1 && V <= TV_MAX_VOCAB && max_depth >= 1 &&
         max_depth <= 1023;
}

tv_status device_status(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_DEVICE; }

// Checks of tv_tree_build's arguments that need no workspace; fills the plan.
tv_status build_check(const void* draft_logits, tv_dtype dt, int batch, int K, int V, int topk,
                      int budget, float build_temp, const int32_t* root_token,
                      const int32_t* ctx_len, const int32_t* parent, const int32_t* token,
                      const int32_t* depth, const int32_t* pos, const double* score,
                      const uint64_t* anc_mask, const int32_t* n_nodes, tvk::BuildPlan* plan) {
  if (!draft_logits || !root_token || !ctx_len || !parent || !token || !depth || !pos ||
      !score || !anc_mask || !n_nodes)
    return TV_ERR_INVALID;
  if (dt != TV_F32 && dt != TV_BF16) return TV_ERR_INVALID;
  if (!finite_pos(build_temp)) return TV_ERR_INVALID;
  if (batch < 1 || K < 1 || V < 1 || topk < 1 || topk > V || budget < 0) return TV_ERR_INVALID;
  if (!build_args_ok(batch, K, V, topk, budget)) return TV_ERR_UNSUPPORTED;
  *plan = tvk::build_plan(batch, K, V, topk, budget);
  if (plan->C * topk > 256 * tvk::kFinalizeE || plan->select_lds > tvk::kMaxSelectLds ||
      plan->rows > kMaxGridY)
    return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

}  // namespace

// Scratch of tv_tree_build_noalloc: a file-scope device array, one copy per
// GPU, zero at load and held until the process ends.  In host code its name
// is a host-side stand-in, not a device address: the address of a device's
// copy comes from hipGetSymbolAddress, looked up once per device with that
// device current, and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[TV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "TV_OK";
    case TV_ERR_INVALID: return "TV_ERR_INVALID: invalid argument";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED: outside the limits of this build";
    case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE: workspace missing or too small";
    case TV_ERR_DEVICE: return "TV_ERR_DEVICE: HIP launch error";
    default: break;
  }
  return "unknown tv_status";
}

int tv_version(void) { return 10000; }

// ---------------------------------------------------------------------------
size_t tv_tree_build_workspace(int batch, int K, int V, int topk, int budget) {
  if (!build_args_ok(batch, K, V, topk, budget)) return 0;
  return tvk::build_plan(batch, K, V, topk, budget).workspace;
}

tv_status tv_tree_build(const void* draft_logits, tv_dtype dt, int batch, int K, int V,
                        int topk, int budget, float build_temp, const int32_t* root_token,
                        const int32_t* ctx_len, int32_t* parent, int32_t* token,
                        int32_t* depth, int32_t* pos, double* score, uint64_t* anc_mask,
                        int32_t* n_nodes, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  tvk::BuildPlan p{};
  const tv_status st = build_check(draft_logits, dt, batch, K, V, topk, budget, build_temp,
                                   root_token, ctx_len, parent, token, depth, pos, score,
                                   anc_mask, n_nodes, &p);
  if (st != TV_OK) return st;
  if (!workspace || workspace_bytes < p.workspace) return TV_ERR_WORKSPACE;
  return device_status(tvk::launch_build(p, draft_logits, dt == TV_BF16, batch, K, V, topk,
                                         budget, 1.0f / build_temp, root_token, ctx_len, parent,
                                         token, depth, pos, score, anc_mask, n_nodes, workspace,
                                         stream));
}

tv_status tv_tree_build_noalloc(const void* draft_logits, tv_dtype dt, int batch, int K, int V,
                                int topk, int budget, float build_temp,
                                const int32_t* root_token, const int32_t* ctx_len,
                                int32_t* parent, int32_t* token, int32_t* depth, int32_t* pos,
                                double* score, uint64_t* anc_mask, int32_t* n_nodes,
                                hipStream_t stream) {
  tvk::BuildPlan p{};
  const tv_status st = build_check(draft_logits, dt, batch, K, V, topk, budget, build_temp,
                                   root_token, ctx_len, parent, token, depth, pos, score,
                                   anc_mask, n_nodes, &p);
  if (st != TV_OK) return st;
  if (p.workspace > TV_NOALLOC_SCRATCH_BYTES) return TV_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return TV_ERR_DEVICE;
  return device_status(tvk::launch_build(p, draft_logits, dt == TV_BF16, batch, K, V, topk,
                                         budget, 1.0f / build_temp, root_token, ctx_len, parent,
                                         token, depth, pos, score, anc_mask, n_nodes, ws,
                                         stream));
}

tv_status tv_tree_check(const int32_t* parent, const int32_t* depth, const int32_t* n_nodes,
                        int batch, int N, int32_t* status, hipStream_t stream) {
  if (!parent || !n_nodes || !status) return TV_ERR_INVALID;
  if (batch < 1 || N < 1) return TV_ERR_INVALID;
  return device_status(tvk::launch_tree_check(parent, depth, n_nodes, batch, N, status, stream));
}

tv_status tv_tree_root(const int32_t* root_token, const int32_t* ctx_len, int batch, int N,
                       int32_t* parent, int32_t* token, int32_t* depth, int32_t* pos,
                       double* score, uint64_t* anc_mask, int32_t* n_nodes, hipStream_t stream) {
  if (!root_token || !ctx_len || !parent || !token || !depth || !pos || !score || !anc_mask ||
      !n_nodes)
    return TV_ERR_INVALID;
  if (batch < 1 || N < 1) return TV_ERR_INVALID;
  if (N > 1024) return TV_ERR_UNSUPPORTED;
  return device_status(tvk::launch_tree_root(root_token, ctx_len, batch, N, parent, token, depth,
                                             pos, score, anc_mask, n_nodes, stream));
}

size_t tv_tree_expand_workspace(int batch, int W, int V, int m) {
  if (!build_args_ok(batch, W, V, m, 0)) return 0;
  return tvk::build_plan(batch, W, V, m, 0).workspace;
}

tv_status tv_tree_expand(const void* node_logits, tv_dtype dt, int batch, int W, int V, int m,
                         float build_temp, const int32_t* ctx_len, const int32_t* frontier,
                         int N, int32_t* parent, int32_t* token, int32_t* depth, int32_t* pos,
                         double* score, uint64_t* anc_mask, int32_t* n_nodes,
                         int32_t* next_frontier, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!node_logits || !ctx_len || !frontier || !parent || !token || !depth || !pos || !score ||
      !anc_mask || !n_nodes || !next_frontier)
    return TV_ERR_INVALID;
  if (dt != TV_F32 && dt != TV_BF16) return TV_ERR_INVALID;
  if (!finite_pos(build_temp)) return TV_ERR_INVALID;
  if (batch < 1 || W < 1 || V < 1 || m < 1 || m > V || N < 1) return TV_ERR_INVALID;
  if (!build_args_ok(batch, W, V, m, 0) || N > 1024) return TV_ERR_UNSUPPORTED;
  const tvk::BuildPlan p = tvk::build_plan(batch, W, V, m, 0);
  if (p.C * m > 256 * tvk::kFinalizeE || p.rows > kMaxGridY) return TV_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.workspace) return TV_ERR_WORKSPACE;
  return device_status(tvk::launch_tree_expand(p, node_logits, dt == TV_BF16, batch, W, V, m,
                                               1.0f / build_temp, N, ctx_len, frontier, parent,
                                               token, depth, pos, score, anc_mask, n_nodes,
                                               next_frontier, workspace, stream));
}

tv_status tv_tree_ancestors(const int32_t* parent, const int32_t* n_nodes,
                            const int32_t* ctx_len, int batch, int N, int32_t* depth,
                            int32_t* pos, uint64_t* anc_mask, hipStream_t stream) {
  if (!parent || !n_nodes || !ctx_len || !depth || !pos || !anc_mask) return TV_ERR_INVALID;
  if (batch < 1 || N < 1) return TV_ERR_INVALID;
  if (N > 1024 || batch > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  return device_status(
      tvk::launch_ancestors(parent, n_nodes, ctx_len, batch, N, depth, pos, anc_mask, stream));
}

// ---------------------------------------------------------------------------
size_t tv_tree_attention_workspace(int batch, int N, int Hq, int Hkv, int D, int max_ctx,
                                   int splits) {
  if (!attn_args_ok(batch, N, Hq, Hkv, D, max_ctx, splits)) return 0;
  return tvk::attention_plan(batch, N, Hq, Hkv, D, max_ctx, splits).workspace;
}

static tv_status attention_impl(const void* q, const void* k_cache, const void* v_cache,
                                tv_dtype dt, const int32_t* ctx_len, const uint64_t* anc_mask,
                                const int32_t* n_nodes, const int32_t* pos, double rope_base,
                                int batch, int N, int Hq, int Hkv, int D, int cap, int max_ctx,
                                float scale, int splits, void* out, tv_dtype out_dt, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !ctx_len || !anc_mask || !n_nodes || !out)
    return TV_ERR_INVALID;
  if (pos && !rope_base_ok(rope_base)) return TV_ERR_INVALID;
  if (dt != TV_F32 && dt != TV_BF16) return TV_ERR_INVALID;
  if (out_dt != TV_F32 && out_dt != TV_BF16) return TV_ERR_INVALID;
  if (dt == TV_F32 && out_dt != TV_F32) return TV_ERR_UNSUPPORTED;
  if (batch < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_ctx < 0 || splits < 0 ||
      !finite_pos(scale))
    return TV_ERR_INVALID;
  if ((int64_t)max_ctx + N > (int64_t)cap) return TV_ERR_INVALID;
  if (!attn_args_ok(batch, N, Hq, Hkv, D, max_ctx, splits)) return TV_ERR_UNSUPPORTED;
  if ((int64_t)batch * Hkv > kMaxGridY) return TV_ERR_UNSUPPORTED;
  if ((int64_t)cap * D * 2 > 0x7FFFFFFF) return TV_ERR_UNSUPPORTED;  // one head's rows: 32-bit offsets
  const tvk::AttnPlan p = tvk::attention_plan(batch, N, Hq, Hkv, D, max_ctx, splits);
  if (dt == TV_BF16 && (!workspace || workspace_bytes < p.workspace)) return TV_ERR_WORKSPACE;
  return device_status(tvk::launch_attention(p, q, k_cache, v_cache, dt == TV_BF16, ctx_len,
                                             anc_mask, n_nodes, batch, N, Hq, Hkv, D, cap,
                                             max_ctx, scale, out, out_dt == TV_F32, lse, pos,
                                             pos ? std::log2(rope_base) : 0.0, workspace,
                                             stream));
}

tv_status tv_tree_attention_verify(const void* q, const void* k_cache, const void* v_cache,
                                   tv_dtype dt, const int32_t* ctx_len,
                                   const uint64_t* anc_mask, const int32_t* n_nodes,
                                   int batch, int N, int Hq, int Hkv, int D, int cap,
                                   int max_ctx, float scale, int splits, void* out,
                                   tv_dtype out_dt, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return attention_impl(q, k_cache, v_cache, dt, ctx_len, anc_mask, n_nodes, nullptr, 0.0, batch,
                        N, Hq, Hkv, D, cap, max_ctx, scale, splits, out, out_dt, lse, workspace,
                        workspace_bytes, stream);
}

tv_status tv_tree_attention_verify_rope(const void* q, const void* k_cache, const void* v_cache,
                                        tv_dtype dt, const int32_t* ctx_len,
                                        const uint64_t* anc_mask, const int32_t* n_nodes,
                                        const int32_t* pos, double rope_base, int batch, int N,
                                        int Hq, int Hkv, int D, int cap, int max_ctx, float scale,
                                        int splits, void* out, tv_dtype out_dt, float* lse,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  if (!pos) return TV_ERR_INVALID;
  return attention_impl(q, k_cache, v_cache, dt, ctx_len, anc_mask, n_nodes, pos, rope_base,
                        batch, N, Hq, Hkv, D, cap, max_ctx, scale, splits, out, out_dt, lse,
                        workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
size_t tv_tree_accept_workspace(int batch, int N, int K, int V, tv_accept_mode mode,
                                tv_proposal proposal) {
  if (!accept_args_ok(batch, N, V, 1)) return 0;
  const bool sampled = mode == TV_SAMPLED;
  const bool draft = sampled && proposal == TV_PROPOSAL_DRAFT;
  if (draft && K < 1) return 0;
  return tvk::accept_plan(batch, N, K, V, sampled, draft).workspace;
}

tv_status tv_tree_accept(const void* target_logits, const void* draft_logits, tv_dtype dt,
                         int batch, int N, int K, int V, const int32_t* parent,
                         const int32_t* token, const int32_t* depth, const int32_t* n_nodes,
                         tv_accept_mode mode, float temperature, tv_proposal proposal,
                         uint64_t seed, uint64_t round, int max_depth, int32_t* accept_len,
                         int32_t* accepted_nodes, int32_t* out_tokens, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !parent || !token || !depth || !n_nodes || !accept_len ||
      !accepted_nodes || !out_tokens)
    return TV_ERR_INVALID;
  if (dt != TV_F32 && dt != TV_BF16) return TV_ERR_INVALID;
  if (mode != TV_GREEDY && mode != TV_SAMPLED) return TV_ERR_INVALID;
  if (proposal != TV_PROPOSAL_POINT_MASS && proposal != TV_PROPOSAL_DRAFT)
    return TV_ERR_INVALID;
  const bool sampled = mode == TV_SAMPLED;
  const bool draft = sampled && proposal == TV_PROPOSAL_DRAFT;
  if (sampled && !finite_pos(temperature)) return TV_ERR_INVALID;
  if (draft && (!draft_logits || K < 1)) return TV_ERR_INVALID;
  if (draft && K > TV_MAX_POSITIONS) return TV_ERR_UNSUPPORTED;
  if (batch < 1 || N < 1 || V < 1 || max_depth < 1) return TV_ERR_INVALID;
  if (!accept_args_ok(batch, N, V, max_depth)) return TV_ERR_UNSUPPORTED;
  const tvk::AcceptPlan p = tvk::accept_plan(batch, N, K, V, sampled, draft);
  if (p.rows > kMaxGridY) return TV_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.workspace) return TV_ERR_WORKSPACE;
  const float inv_t = sampled ? 1.0f / temperature : 1.0f;
  return device_status(tvk::launch_accept(p, target_logits, draft ? draft_logits : nullptr,
                                          dt == TV_BF16, batch, N, K, V, parent, token, depth,
                                          n_nodes, sampled, inv_t, draft, seed, round,
                                          max_depth, accept_len, accepted_nodes, out_tokens,
                                          workspace, stream));
}

// ---------------------------------------------------------------------------
tv_status tv_tree_budget(const double* score, const int32_t* n_nodes, const double* cost,
                         int batch, int N, int ncost, int32_t* n_nodes_out, hipStream_t stream) {
  if (!score || !n_nodes || !cost || !n_nodes_out) return TV_ERR_INVALID;
  if (batch < 1 || N < 1 || ncost < N) return TV_ERR_INVALID;
  if (N > 1024 || batch > 0x7fffffff) return TV_ERR_UNSUPPORTED;
  return device_status(
      tvk::launch_tree_budget(score, n_nodes, cost, batch, N, n_nodes_out, stream));
}

// ---------------------------------------------------------------------------
static tv_status kv_commit_impl(void* k_cache, void* v_cache, tv_dtype dt, int batch, int Hkv,
                                int cap, int D, const int32_t* ctx_len,
                                const int32_t* accept_len, const int32_t* accepted_nodes,
                                int width, bool rope, double rope_base, int32_t* new_ctx_len,
                                hipStream_t stream) {
  if (!k_cache || !v_cache || !ctx_len || !accept_len || !accepted_nodes || !new_ctx_len)
    return TV_ERR_INVALID;
  if (dt != TV_F32 && dt != TV_BF16) return TV_ERR_INVALID;
  if (batch < 1 || Hkv < 1 || cap < 1 || width < 1) return TV_ERR_INVALID;
  if (rope && !rope_base_ok(rope_base)) return TV_ERR_INVALID;
  if ((D != 64 && D != 128) || width > tvk::kCommitMaxWidth || batch > 0x7fffffff)
    return TV_ERR_UNSUPPORTED;
  return device_status(tvk::launch_kv_commit(k_cache, v_cache, dt == TV_BF16 ? 2 : 4, batch, Hkv,
                                             cap, D, ctx_len, accept_len, accepted_nodes, width,
                                             new_ctx_len, rope, rope ? std::log2(rope_base) : 0.0,
                                             stream));
}

tv_status tv_kv_commit(void* k_cache, void* v_cache, tv_dtype dt, int batch, int Hkv, int cap,
                       int D, const int32_t* ctx_len, const int32_t* accept_len,
                       const int32_t* accepted_nodes, int width, int32_t* new_ctx_len,
                       hipStream_t stream) {
  return kv_commit_impl(k_cache, v_cache, dt, batch, Hkv, cap, D, ctx_len, accept_len,
                        accepted_nodes, width, false, 0.0, new_ctx_len, stream);
}

int tv_debug_set_spin_limit(int polls) { return tvk::set_rowstat_spin_limit(polls); }

tv_status tv_debug_weights(uint32_t first_bits, uint32_t count, float row_max, float inv_t,
                           int unit, uint64_t* out, hipStream_t stream) {
  if (!out || count < 1 || !std::isfinite(row_max) || !finite_pos(inv_t)) return TV_ERR_INVALID;
  if (unit && inv_t != 1.0f) return TV_ERR_INVALID;
  return device_status(
      tvk::launch_debug_weights(first_bits, count, row_max, inv_t, unit != 0, out, stream));
}

tv_status tv_debug_set_attention_events(hipEvent_t before, hipEvent_t between) {
  tvk::set_attention_events(before, between);
  return TV_OK;
}

tv_status tv_kv_commit_rope(void* k_cache, void* v_cache, tv_dtype dt, int batch, int Hkv,
                            int cap, int D, const int32_t* ctx_len, const int32_t* accept_len,
                            const int32_t* accepted_nodes, int width, double rope_base,
                            int32_t* new_ctx_len, hipStream_t stream) {
  return kv_commit_impl(k_cache, v_cache, dt, batch, Hkv, cap, D, ctx_len, accept_len,
                        accepted_nodes, width, true, rope_base, new_ctx_len, stream);
}

}  // extern "C"
