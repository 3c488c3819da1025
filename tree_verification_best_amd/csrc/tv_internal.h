// tv_internal.h -- host-side plans and kernel launchers of libtreeverify
// (shared between the API translation unit and the kernel files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>

#define TV_MAX_TOPK_ 64

namespace tvk {

// ---- build ----
constexpr int kBuildChunk = 8192;  // tokens per block in the draft-row passes
constexpr int kRankMax = 512;  // depth lists up to this size are ordered by rank counting
constexpr int kFinalizeE = 8;      // per-thread items when merging chunk candidates
constexpr size_t kMaxSelectLds = 160 * 1024 - 1024;  // the selection's dynamic LDS, at most

struct BuildPlan {
  int chunk, C;
  int64_t rows;
  int P;  // LDS room for the candidates of one depth (a power of two)
  size_t select_lds;
  size_t off_cval, off_cid, off_ftok, off_fq;
  size_t off_rowrec;  // per-row mass accumulator and arrival count (256-byte lines)
  size_t workspace;
};

BuildPlan build_plan(int batch, int K, int V, int topk, int budget);
hipError_t launch_build(const BuildPlan& p, const void* draft, bool bf16, int batch, int K,
                        int V, int topk, int budget, float inv_t, const int* root_token,
                        const int* ctx_len, int* parent, int* token, int* depth, int* pos,
                        double* score, uint64_t* anc, int* n_nodes, void* ws,
                        hipStream_t stream);
hipError_t launch_tree_expand(const BuildPlan& p, const void* logits, bool bf16, int batch, int W,
                              int V, int m, float inv_t, int N, const int* ctx_len,
                              const int* frontier, int* parent, int* token, int* depth, int* pos,
                              double* score, uint64_t* anc, int* n_nodes, int* next_frontier,
                              void* ws, hipStream_t stream);
hipError_t launch_tree_check(const int* parent, const int* depth, const int* n_nodes, int batch,
                             int N, int* status, hipStream_t stream);
hipError_t launch_tree_root(const int* root_token, const int* ctx_len, int batch, int N,
                            int* parent, int* token, int* depth, int* pos, double* score,
                            uint64_t* anc, int* n_nodes, hipStream_t stream);
hipError_t launch_tree_budget(const double* score, const int* n_nodes, const double* cost,
                              int batch, int N, int* n_out, hipStream_t stream);
hipError_t launch_ancestors(const int* parent, const int* n_nodes, const int* ctx_len,
                            int batch, int N, int* depth, int* pos, uint64_t* anc,
                            hipStream_t stream);

// ---- attention ----
struct AttnPlan {
  int rows_per_kv;  // G * N
  int row_blocks;   // ceil(rows_per_kv / 32)
  int waves;        // waves per workgroup
  int mtiles;       // workgroups along the rows of one KV head
  int splits;       // context splits (the tree keys get one more)
  int keys_per_split;
  size_t off_o, off_ml;
  size_t workspace;
};

AttnPlan attention_plan(int batch, int N, int Hq, int Hkv, int D, int max_ctx, int splits);
// Timing hook: events recorded just before the partial kernel and between
// the partial and combine kernels (nullptr: none).
void set_attention_events(hipEvent_t before, hipEvent_t between);
hipError_t launch_attention(const AttnPlan& p, const void* q, const void* k, const void* v,
                            bool bf16, const int* ctx_len, const uint64_t* anc,
                            const int* n_nodes, int batch, int N, int Hq, int Hkv, int D,
                            int cap, int max_ctx, float scale, void* out, bool out_f32,
                            float* lse, const int* pos, double log2_base, void* ws,
                            hipStream_t stream);

// ---- accept ----
constexpr int kAcceptChunk = 4096;  // tokens per block in the logits passes

struct AcceptPlan {
  int chunk, C;
  int64_t rows;  // batch * N target rows (+ batch * K draft rows in DRAFT mode)
  bool draft_rows;
  // chunk records, chunk-major ([C][rows]); the weight of each child's token
  // in its parent's row (and, DRAFT, in its drafter row) [batch][N]; DRAFT
  // residual chunk sums [batch][64] and the per-sequence hand-over record
  size_t off_cmax, off_carg, off_cz, off_wtg, off_wqg, off_rcz, off_pend;
  size_t off_slot;   // per-row slots of the chunk maxima, one-pass statistics (sampled)
  int slot_stride;   // slots per row (256-byte rows)
  size_t off_rowz, off_rowm;  // sampled: every row's mass Z and maximum, for the walk
  size_t off_gen;             // sampled: the row pass's slot generation
  size_t workspace;
};

AcceptPlan accept_plan(int batch, int N, int K, int V, bool sampled, bool draft);
int set_rowstat_spin_limit(int polls);  // < 0: the default; returns the previous limit
hipError_t launch_debug_weights(uint32_t first, uint32_t count, float m, float inv_t, bool unit,
                                uint64_t* out, hipStream_t stream);
hipError_t launch_accept(const AcceptPlan& p, const void* target, const void* draft,
                         bool bf16, int batch, int N, int K, int V, const int* parent,
                         const int* token, const int* depth, const int* n_nodes, bool sampled,
                         float inv_t, bool draft_proposal, uint64_t seed, uint64_t round,
                         int max_depth, int* accept_len, int* accepted_nodes, int* out_tokens,
                         void* ws, hipStream_t stream);

// ---- KV commit ----
constexpr int kCommitMaxWidth = 1024;
hipError_t launch_kv_commit(void* k_cache, void* v_cache, int elem_bytes, int batch, int Hkv,
                            int cap, int D, const int* ctx_len, const int* accept_len,
                            const int* accepted_nodes, int width, int* new_ctx_len,
                            bool rope, double log2_base, hipStream_t stream);

}  // namespace tvk
