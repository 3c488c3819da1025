/*
 * treeverify.h -- C ABI of libtreeverify.so: one tree-verification round of
 * speculative decoding on an AMD Instinct MI355X (gfx950).
 *
 * A round has three calls, in this order on one stream:
 *   tv_tree_build            draft marginals -> prefix-closed draft tree
 *   tv_tree_attention_verify tree-masked attention of the target over
 *                            context + tree (one layer)
 *   tv_tree_accept           acceptance walk -> accepted path + one token
 * plus:
 *   tv_tree_ancestors, tv_tree_check   trees that come from elsewhere
 *   tv_tree_root, tv_tree_expand       a layer-wise builder (root, then one
 *                                      call per drafting step)
 *   tv_tree_build_noalloc              tv_tree_build without a workspace
 *   tv_tree_budget                     cost-aware tree size
 *   tv_kv_commit                       keep the accepted path in the KV cache
 *   tv_tree_attention_verify_rope, tv_kv_commit_rope
 *                                      the same with the rotary embedding
 *                                      applied at the tree's position ids
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer owned by the caller, dense
 *     and row-major in the layout given in its comment.  The library
 *     allocates and frees nothing; scratch space is the caller's
 *     `workspace` of at least the size the matching *_workspace() returns
 *     (tv_tree_build_noalloc uses a static buffer of the library instead).
 *   - Calls are asynchronous on `stream`: they enqueue kernels and return
 *     without synchronising.  The library keeps no global mutable state, so
 *     calls from several host threads on different streams are safe
 *     (except overlapping tv_tree_build_noalloc calls on one GPU, which
 *     share that GPU's scratch buffer; for
 *     large budgets tv_tree_build raises its selection kernel's dynamic-LDS
 *     limit in the HIP runtime, an idempotent setting; the test hooks
 *     tv_debug_set_spin_limit and tv_debug_set_attention_events change
 *     process-wide settings).
 *   - Arguments are checked on the host before any launch; a bad argument
 *     returns TV_ERR_INVALID (or TV_ERR_UNSUPPORTED for a valid request this
 *     build does not serve) and launches nothing.  A launch failure
 *     reported by the HIP runtime returns TV_ERR_DEVICE.  Nothing throws
 *     across this boundary.
 *   - Device-side data (tree arrays, token ids, lengths) are preconditions;
 *     the kernels stay in bounds for any values, but results for values
 *     that break a stated precondition are unspecified.
 *   - Results are deterministic: the same inputs give the same bits.
 *
 * Numerics of the integer decisions (tree shape, accepted length, sampled
 * tokens), identical on every run:
 *   - A logit l of a row with maximum m at inverse temperature 1/T has the
 *     fixed-point weight W = rint(exp32(fl32(fl32(l - m) * fl32(1/T))) * 2^44),
 *     where exp32 is an fp32 Cody-Waite reduction (ln 2 split in two parts,
 *     the high part with 12 significand bits) followed by the degree-7
 *     Taylor polynomial of e^r in Horner form with fused multiply-adds, and
 *     is 0 below -32.  Row sums Z = sum W are exact 64-bit integers.
 *   - Draft probabilities are q = fp64(W) / fp64(Z); path scores are fp64
 *     products taken from the root down.
 *   - Random draws use Philox4x64-10 with key (seed, 0) and counter
 *     (round, sequence, node, slot).
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TV_OK = 0,
    TV_ERR_INVALID = 1,     /* bad pointer, size or combination of arguments */
    TV_ERR_UNSUPPORTED = 2, /* valid, but outside what this build serves      */
    TV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required     */
    TV_ERR_DEVICE = 4,      /* the HIP runtime reported a launch error        */
    TV_STATUS_RANGE_LO_ = INT32_MIN, TV_STATUS_RANGE_HI_ = INT32_MAX
} tv_status;

/* The *_RANGE_* members are not values of the interface: they give every
 * enum the range of int32, so that any int32 a caller passes (and the
 * library rejects) is a valid value of the type in C and in C++. */
typedef enum {
    TV_F32 = 0, TV_BF16 = 1,
    TV_DTYPE_RANGE_LO_ = INT32_MIN, TV_DTYPE_RANGE_HI_ = INT32_MAX
} tv_dtype;
typedef enum {
    TV_GREEDY = 0, TV_SAMPLED = 1,
    TV_MODE_RANGE_LO_ = INT32_MIN, TV_MODE_RANGE_HI_ = INT32_MAX
} tv_accept_mode;
typedef enum {
    TV_PROPOSAL_POINT_MASS = 0, TV_PROPOSAL_DRAFT = 1,
    TV_PROPOSAL_RANGE_LO_ = INT32_MIN, TV_PROPOSAL_RANGE_HI_ = INT32_MAX
} tv_proposal;

/* Limits of this build. */
#define TV_MAX_VOCAB (1 << 18)
#define TV_MAX_TOPK 64
#define TV_MAX_BUDGET 1023
#define TV_MAX_POSITIONS 64
/* Size of the static device scratch behind tv_tree_build_noalloc. */
#define TV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/* Human-readable name of a status code (static storage). */
const char *tv_status_string(tv_status s);

/* ABI version: major * 10000 + minor * 100 + patch. */
int tv_version(void);

/* Test hook: the number of polls a block of tv_tree_accept's sampled row
 * pass makes while waiting for the other blocks of its row before it finds
 * the row maximum by itself (< 0 restores the default, 48; larger values
 * are capped there).  0 sends nearly every block down that path, which
 * gives the same results.  Process-wide; returns the previous value. */
int tv_debug_set_spin_limit(int polls);

/* Test hook for timing: every later bf16 tv_tree_attention_verify(_rope)
 * call records `before` on its stream just before its first kernel (the
 * split partials) and `between` between that kernel and the second (their
 * combine), each when not null, so that with one more event recorded by the
 * caller after the call the two kernels are bracketed one by one.  null
 * (the default) records nothing.  Process-wide; the caller keeps the events
 * valid while they are set.  Returns TV_OK. */
tv_status tv_debug_set_attention_events(hipEvent_t before, hipEvent_t between);

/* Test hook: the fixed-point softmax weight that the builder and the
 * acceptance kernels give a logit (the primer's "acceptance and rejection":
 * the target and draft distributions as softmax weights; TAPS sec. 4.2: the
 * drafter's probabilities), for the `count` fp32 values whose bit patterns
 * are first_bits, first_bits + 1, ..., as logits of a row with maximum
 * row_max at inverse temperature inv_t.  unit != 0 selects the form the row
 * passes use when inv_t == 1 (then inv_t must be 1).  out: uint64 [count],
 * device.  TV_ERR_INVALID for a null out, count 0, a non-finite row_max or
 * inv_t <= 0. */
tv_status tv_debug_weights(uint32_t first_bits, uint32_t count, float row_max, float inv_t,
                           int unit, uint64_t *out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_build -- draft tree from per-position draft marginals.
 *
 * TAPS sec. 4.1: the drafter gives marginal logits for K future positions
 * in one pass; the top-`topk` tokens of each position form the candidate
 * tree (position j's candidates are the children of every depth j-1 node).
 * TAPS sec. 4.2 and TreeGraft sec. 3.1: each edge carries the drafter's
 * probability q of the child's token at its position; a node's reach
 * probability is the product of the edge probabilities from the root, and
 * the root (the verified prefix) has probability 1.  TAPS sec. 1 / 3.2: a
 * compact prefix-closed subtree that maximises the expected number of
 * accepted tokens under the node budget -- the `budget` nodes of largest
 * reach probability.
 *
 * Candidates of a position are its top-`topk` tokens by (logit desc, id asc),
 * ranked by (q desc, id asc); q uses temperature `build_temp`.  Nodes are
 * chosen in the total order (score desc, depth asc, parent earlier in this
 * order, rank asc) and written in that order: row 0 is the root, rows
 * 1..n-1 the chosen nodes, n = n_nodes[b] = 1 + min(budget, number of
 * candidate-tree nodes).  Every parent row precedes its children.
 *
 *   draft_logits  [batch][K][V], dtype dt (f32 or bf16); finite values, or
 *                 -inf with a finite row maximum.
 *   root_token    [batch] token of the root (the last verified token)
 *   ctx_len       [batch] context length L_b already in the KV cache
 *   parent, token, depth, pos   int32 [batch][budget+1]
 *                 parent row (-1 for the root), token id, depth (root 0),
 *                 position id L_b + depth (PTD sec. 3.1: a node's position
 *                 follows from the size of its ancestor set).
 *   score         double [batch][budget+1] reach probability (root 1.0)
 *   anc_mask      uint64 [batch][budget+1][ceil((budget+1)/64)]: bit j of
 *                 row i is set iff node j is i or an ancestor of i.
 *   n_nodes       int32 [batch]
 *   Rows past n_nodes: parent = token = depth = pos = -1, score 0, mask 0.
 * Limits: 1 <= K <= 64, 1 <= topk <= min(64, V), V <= 2^18, 0 <= budget <= 1023,
 *   build_temp > 0, K * topk <= 4096, ceil(V / 8192) * topk <= 2048, and the
 *   selection's lists within 159 KB of LDS (TV_ERR_UNSUPPORTED beyond): every
 *   budget up to 1023 with topk <= 16, up to 1013 with topk 32 and K 64, up
 *   to 869 with topk 64 and K 64.
 * ------------------------------------------------------------------------ */
size_t tv_tree_build_workspace(int batch, int K, int V, int topk, int budget);
tv_status tv_tree_build(const void *draft_logits, tv_dtype dt, int batch, int K, int V,
                        int topk, int budget, float build_temp, const int32_t *root_token,
                        const int32_t *ctx_len, int32_t *parent, int32_t *token,
                        int32_t *depth, int32_t *pos, double *score, uint64_t *anc_mask,
                        int32_t *n_nodes, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_build_noalloc -- tv_tree_build for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  Same arguments (less the workspace), results,
 * limits and status codes as tv_tree_build.
 *
 * The workspace is a static device buffer of TV_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.  A shape
 * whose tv_tree_build_workspace() exceeds it returns TV_ERR_UNSUPPORTED
 * before any device call.  The first call on a device looks up that device's
 * copy of the buffer (hipGetSymbolAddress; TV_ERR_DEVICE if that fails); no
 * call allocates or frees.  Every call on one GPU uses the same buffer and
 * leaves its contents behind (the kernels set what they read first), so
 * calls whose execution overlaps on one GPU -- from different streams or
 * host threads -- race; the caller orders them.
 * ------------------------------------------------------------------------ */
tv_status tv_tree_build_noalloc(const void *draft_logits, tv_dtype dt, int batch, int K, int V,
                                int topk, int budget, float build_temp,
                                const int32_t *root_token, const int32_t *ctx_len,
                                int32_t *parent, int32_t *token, int32_t *depth, int32_t *pos,
                                double *score, uint64_t *anc_mask, int32_t *n_nodes,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_ancestors -- depth, position ids and ancestor bit rows of trees
 * given as parent arrays (PTD sec. 3.1: pi(v) = {v} U pi(P(v))).
 *
 *   parent   int32 [batch][N]; parent[0] = -1, 0 <= parent[i] < i for
 *            1 <= i < n_nodes[b] (precondition).
 *   n_nodes  int32 [batch], 1 <= n_nodes[b] <= N.
 *   ctx_len  int32 [batch].
 *   depth, pos  int32 [batch][N];  anc_mask uint64 [batch][N][ceil(N/64)].
 *   Rows past n_nodes: depth = pos = -1, mask 0.
 * Limits: 1 <= N <= 1024.  No workspace.
 * ------------------------------------------------------------------------ */
tv_status tv_tree_ancestors(const int32_t *parent, const int32_t *n_nodes,
                            const int32_t *ctx_len, int batch, int N, int32_t *depth,
                            int32_t *pos, uint64_t *anc_mask, hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_check -- structural check of caller-supplied trees.
 *
 * The tree arrays of the other calls are preconditions (PTD sec. 3.1: every
 * node but the root has exactly one parent, so pi(v) = {v} U pi(P(v)) is
 * well defined; rows are stored parents first).  This call tests them on the
 * device, without synchronising, so that a caller can check trees from
 * elsewhere before verification:
 *   status[b] = 0  the tree is well formed;
 *             = 1  n_nodes[b] outside [1, N];
 *             = 2 + i  for the first row i that breaks a rule:
 *               parent[0] = -1, 0 <= parent[i] < i for 1 <= i < n_nodes[b],
 *               and, when depth is not NULL, depth[0] = 0 and
 *               depth[i] = depth[parent[i]] + 1.
 *   parent, depth int32 [batch][N] (depth may be NULL); n_nodes int32 [batch];
 *   status int32 [batch] (device).
 * ------------------------------------------------------------------------ */
tv_status tv_tree_check(const int32_t *parent, const int32_t *depth, const int32_t *n_nodes,
                        int batch, int N, int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_attention_verify -- one target attention layer over context +
 * tree in a single pass.
 *
 * Primer, "why the target can verify in parallel": the target reads the
 * original context followed by the draft tokens in one forward pass.  PTD
 * sec. 3.1: a tree node attends only to its ancestor set pi(v).  So node i of
 * sequence b, query head h, attends to the cached context keys [0, L_b) and
 * to the tree keys at cache rows L_b + j for every j in pi(i); GQA maps
 * query head h to KV head h / (Hq / Hkv).  out = softmax((q . k) * scale) v,
 * lse = natural log of the softmax normaliser (max included).
 *
 *   q        [batch][N][Hq][D]       dtype dt
 *   k_cache, v_cache [batch][Hkv][cap][D]  dtype dt; context rows [0, L_b),
 *            tree rows at L_b + i (the target layer writes them there).
 *   ctx_len  int32 [batch], 0 <= L_b <= max_ctx (precondition)
 *   anc_mask uint64 [batch][N][ceil(N/64)] as written by tv_tree_build
 *   n_nodes  int32 [batch], 1 <= n_nodes[b] <= N (precondition)
 *   out      [batch][N][Hq][D]       dtype out_dt: TV_F32 (the fp32 result of
 *            the accumulation) or, for bf16 inputs, TV_BF16 (rounded to
 *            nearest even; fp32 inputs need TV_F32)
 *   lse      float [batch][N][Hq], may be NULL
 *   splits   number of context splits (0 = automatic); partial results are
 *            merged with their log-sum-exp weights.
 *   Rows past n_nodes: out 0, lse -inf.
 * Limits: D in {64, 128}; Hq % Hkv == 0; N <= 1024; max_ctx + N <= cap;
 *         one head's cache rows (cap * D * 2 bytes) below 2 GiB (TV_ERR_UNSUPPORTED).
 * bf16: bf16 products on the matrix cores with fp32 accumulation and an
 * fp32 online softmax; the softmax weights enter the second product
 * rounded to bf16 while the normaliser sums them in fp32; each context
 * split's normalised partial result is kept in fp16 (|V| < 65504).  f32: fp32
 * throughout (vector ALU).
 * ------------------------------------------------------------------------ */
size_t tv_tree_attention_workspace(int batch, int N, int Hq, int Hkv, int D, int max_ctx,
                                   int splits);
tv_status tv_tree_attention_verify(const void *q, const void *k_cache, const void *v_cache,
                                   tv_dtype dt, const int32_t *ctx_len,
                                   const uint64_t *anc_mask, const int32_t *n_nodes,
                                   int batch, int N, int Hq, int Hkv, int D, int cap,
                                   int max_ctx, float scale, int splits, void *out,
                                   tv_dtype out_dt, float *lse, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_attention_verify_rope -- the same attention with the rotary
 * position embedding applied inside the kernel, at the tree's position ids.
 *
 * PTD sec. 3.1: a node's position encoding follows from the size of its
 * ancestor set, so node i sits at pos[b][i] = L_b + depth(i), the position it
 * would have in the plain sequence of the context and its root-to-node path.
 * The rotary embedding (not defined by the pages; the standard one with the
 * half-split pairing): dimension d < D/2 pairs with d + D/2 and the pair
 * turns by pos * rope_base^(-2d/D) radians.  Cache convention: context rows
 * [0, L_b) hold keys already rotated at their own positions (as
 * tv_kv_commit_rope leaves them); tree rows L_b + i hold keys as the target's
 * projection wrote them.  This call rotates every query row i and every tree
 * key row i at pos[b][i] as it loads them, then computes
 * tv_tree_attention_verify's result; q and the caches are not modified.
 *   pos        int32 [batch][N] position ids (tv_tree_build's pos)
 *   rope_base  finite, > 1 (e.g. 1e4, 1e6); other arguments as above.
 * Rotated bf16 values are rounded to bf16 (nearest even) before the matrix
 * products; angles are reduced in fp64 to [-1/2, 1/2] revolutions before the
 * hardware fp32 sine and cosine (abs error below 2e-7).
 * ------------------------------------------------------------------------ */
tv_status tv_tree_attention_verify_rope(const void *q, const void *k_cache, const void *v_cache,
                                        tv_dtype dt, const int32_t *ctx_len,
                                        const uint64_t *anc_mask, const int32_t *n_nodes,
                                        const int32_t *pos, double rope_base, int batch, int N,
                                        int Hq, int Hkv, int D, int cap, int max_ctx, float scale,
                                        int splits, void *out, tv_dtype out_dt, float *lse,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_accept -- the acceptance walk over one tree per sequence.
 *
 * Primer, "acceptance and rejection": starting at the root, greedy mode
 * follows the child whose token equals the target's argmax (lowest id on
 * ties; the first such child in row order) until none does, then emits the
 * target's argmax.  Sampled mode at temperature T:
 *   TV_PROPOSAL_POINT_MASS (trees of deterministic candidates, e.g. from
 *     tv_tree_build): at node u the children are tried in row order; child
 *     with token t is accepted with probability min(1, p_res(t) / 1), where
 *     p_res is the target's distribution at u with the tokens of the
 *     already rejected siblings removed and renormalised; if all are
 *     rejected (or u is a leaf) one token is drawn from p_res.  The emitted
 *     sequence has exactly the target's autoregressive law.
 *   TV_PROPOSAL_DRAFT (chains whose tokens were sampled from the drafter):
 *     child token t at depth d is accepted with probability min(1, p(t) /
 *     q_d(t)), q_d the drafter's distribution at position d (draft row d-1);
 *     at the first rejection one token is drawn from (p - q_d)+ normalised.
 *     A node with more than one child sets accept_len[b] = -1.
 * The round emits the accepted drafts and one more token.
 *
 * Draws: the acceptance of node c uses Philox word 0 of counter
 * (round, b, c, 0) under key (seed, 0); the final draw at node u uses words
 * 0 and 1 of counter (round, b, u, 0xFFFFFFFF) as a 128-bit uniform and an
 * exact integer inverse CDF over the weights.  POINT_MASS accepts iff
 * U * Z_res < W(t) * 2^64 (exact).  DRAFT accepts iff p > 0 and (p >= q
 * or (U >> 11) * 2^-53 < p / q) in fp64, and its residual weights are
 * rint(max(0, p - q) * 2^62).
 *
 *   target_logits [batch][N][V]   dtype dt; row i = the target's next-token
 *                                 logits after node i's prefix.
 *   draft_logits  [batch][K][V]   DRAFT only (else NULL); row j = position j+1.
 *   parent, token, depth  int32 [batch][N]; n_nodes int32 [batch].
 *   accept_len     int32 [batch]  accepted drafted tokens (or -1, see above)
 *   accepted_nodes int32 [batch][max_depth+1]: root row 0, then the rows of
 *                  the accepted nodes, then -1.
 *   out_tokens     int32 [batch][max_depth+1]: the accepted tokens, then
 *                  the emitted token, then -1.
 * A node at depth max_depth is treated as a leaf.  Tokens outside [0, V)
 * are never accepted.
 * Limits: V <= 2^18; N <= 1024; 1 <= max_depth <= 1023; temperature > 0 in
 * sampled mode; 1 <= K <= 64 with draft_logits in DRAFT mode.
 * Sampled mode reads every logit row once: the blocks that hold the chunks
 * of one row wait for each other to agree on the row's maximum before they
 * weigh their chunks.  The grid is sized within what the device holds at
 * once, and the wait is bounded (tens of microseconds): a block that waits
 * too long (other work holding the device) re-reads its row to find the
 * maximum itself, with the same result, only slower.
 * Workspace (sampled mode): zero-fill it once when it is allocated, and again
 * before reusing it for another (batch, N, K, V, mode, proposal).  The row
 * pass's hand-off words must be zero when a call starts; every call leaves
 * them zero, so calls and replays of captured calls need no clearing.
 * Greedy mode needs no particular contents.
 * ------------------------------------------------------------------------ */
size_t tv_tree_accept_workspace(int batch, int N, int K, int V, tv_accept_mode mode,
                                tv_proposal proposal);
tv_status tv_tree_accept(const void *target_logits, const void *draft_logits, tv_dtype dt,
                         int batch, int N, int K, int V, const int32_t *parent,
                         const int32_t *token, const int32_t *depth, const int32_t *n_nodes,
                         tv_accept_mode mode, float temperature, tv_proposal proposal,
                         uint64_t seed, uint64_t round, int max_depth, int32_t *accept_len,
                         int32_t *accepted_nodes, int32_t *out_tokens, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_root -- a tree of capacity N that holds only its root.
 *
 * TreeGraft sec. 3.1: the first drafting step expands the root alone (the
 * last verified token, score 1).  Row 0 gets parent -1, root_token[b], depth
 * 0, pos L_b = ctx_len[b], score 1.0 and ancestor bit 0; rows 1..N-1 get
 * -1 / 0 as rows past n_nodes do in tv_tree_build; n_nodes[b] = 1.
 *   parent, token, depth, pos int32 [batch][N]; score double [batch][N];
 *   anc_mask uint64 [batch][N][ceil(N/64)]; n_nodes int32 [batch]
 * Limits: 1 <= N <= 1024.
 * ------------------------------------------------------------------------ */
tv_status tv_tree_root(const int32_t *root_token, const int32_t *ctx_len, int batch, int N,
                       int32_t *parent, int32_t *token, int32_t *depth, int32_t *pos,
                       double *score, uint64_t *anc_mask, int32_t *n_nodes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_expand -- one drafting step of a layer-wise tree builder.
 *
 * TreeGraft sec. 3.1 (standard single-drafter expansion): each step takes
 * the frontier, the W best nodes added by the previous step by path score
 * (the root alone at the first step); the drafter's next-token distribution
 * at each frontier node gives its top-m tokens as children; an edge's score
 * is the drafter's probability of the child's token and a node's score the
 * product of the edge scores from the root.  The drafter runs outside this
 * library: node_logits holds its next-token logits at each frontier slot.
 *
 * Per sequence b with n0 = n_nodes[b]: the children of the valid frontier
 * slots (row in [0, n0)) are appended in slot order, then rank order
 * ((q desc, id asc), q = W / Z at build_temp as in tv_tree_build), at rows
 * n0, n0 + 1, ...; rows from N on are dropped.  A child c of parent f gets
 * parent f, its token, depth[f] + 1, pos = L_b + depth, score
 * fl64(score[f] * q) and anc_mask row anc[f] | bit c.  n_nodes[b] becomes
 * the new count and next_frontier[b] the W new rows of highest score (ties:
 * lower row first), padded with -1: it is the frontier of the next step.
 * A sequence with n0 outside [1, N] is left as it is (next_frontier all -1).
 *   node_logits   [batch][W][V], dtype dt (f32 or bf16); rows of empty
 *                 slots are read but unused
 *   ctx_len       [batch]
 *   frontier      int32 [batch][W] rows of the tree, -1 for an empty slot
 *   parent, token, depth, pos, score, anc_mask, n_nodes   a tree as written
 *                 by tv_tree_build (capacity N rows), updated in place
 *   next_frontier int32 [batch][W], may be the frontier array itself
 * Start from tv_tree_root's root-only tree and frontier {0, -1, ...};
 * repeat with the drafter's logits at next_frontier.
 * Limits: 1 <= W <= 64, 1 <= m <= min(64, V), V <= 2^18, W * m <= 4096,
 *   1 <= N <= 1024, build_temp > 0.
 * ------------------------------------------------------------------------ */
size_t tv_tree_expand_workspace(int batch, int W, int V, int m);
tv_status tv_tree_expand(const void *node_logits, tv_dtype dt, int batch, int W, int V, int m,
                         float build_temp, const int32_t *ctx_len, const int32_t *frontier,
                         int N, int32_t *parent, int32_t *token, int32_t *depth, int32_t *pos,
                         double *score, uint64_t *anc_mask, int32_t *n_nodes,
                         int32_t *next_frontier, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_tree_budget -- cost-aware size of the tree to verify.
 *
 * TAPS sec. 3.2 (key insight) and sec. 4.1 (third stage): verification should
 * not simply fill the budget; the selector keeps a compact prefix-closed
 * subtree that maximises the expected accepted tokens per unit of
 * verification cost.  The rows of a tree from tv_tree_build are in
 * best-first order, so its first n draft rows are the best prefix-closed
 * subtree of n nodes, and a round that verifies them emits 1 + S_n tokens in
 * expectation (S_n = s_1 + ... + s_n, the path scores, as reach
 * probabilities).  This call keeps
 *   n* = the smallest n in [0, n_nodes[b] - 1] maximising (1 + S_n) / cost[n]
 * (S_n summed left to right in fp64, one fp64 division) and sets
 * n_nodes_out[b] = n* + 1.  Rows past it need no change: attention and the
 * walk read only rows below n_nodes.
 *   score    double [batch][N] as written by tv_tree_build (row 0 the root)
 *   n_nodes  int32 [batch]; a value outside [1, N] is copied unchanged
 *   cost     double [ncost], ncost >= N: cost[n] > 0 is the measured cost of
 *            verifying a tree of n draft nodes (e.g. the attention time of
 *            a round at N = n + 1)
 *   n_nodes_out int32 [batch], may be the n_nodes array itself
 * Limits: N <= 1024.
 * ------------------------------------------------------------------------ */
tv_status tv_tree_budget(const double *score, const int32_t *n_nodes, const double *cost,
                         int batch, int N, int ncost, int32_t *n_nodes_out,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_kv_commit -- keep the accepted path in the target KV cache.
 *
 * Primer, "KV cache handling": after verification only the accepted tokens
 * stay in the target cache; the entries of the rejected candidates are
 * dropped (rolled back).  After a round, cache row L_b + i holds tree node i
 * (as tv_tree_attention_verify reads it); the committed sequence is the root
 * followed by the accepted drafts, accepted_nodes[b][0..accept_len[b]] as
 * written by tv_tree_accept.  This call moves row L_b + accepted_nodes[b][j]
 * to row L_b + j for j = 0..accept_len[b], in both caches and every KV head,
 * in place, and sets new_ctx_len[b] = L_b + accept_len[b] + 1.  Rows past the
 * new length are left as they are, free for the next round.
 *   k_cache, v_cache [batch][Hkv][cap][D]  dtype dt, modified in place
 *   ctx_len, accept_len     int32 [batch]
 *   accepted_nodes          int32 [batch][width]
 *   new_ctx_len             int32 [batch], may be the ctx_len array itself
 * Per sequence: accept_len < 0 (a refused tree) commits nothing and gives
 * new_ctx_len = L_b; a path that does not start at node 0, does not increase
 * strictly, does not fit in width, or reaches row cap or beyond (or L_b < 0)
 * is left uncommitted with new_ctx_len = -1.
 * Limits: D in {64, 128}; width <= 1024.
 * ------------------------------------------------------------------------ */
tv_status tv_kv_commit(void *k_cache, void *v_cache, tv_dtype dt, int batch, int Hkv, int cap,
                       int D, const int32_t *ctx_len, const int32_t *accept_len,
                       const int32_t *accepted_nodes, int width, int32_t *new_ctx_len,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * tv_kv_commit_rope -- tv_kv_commit for caches verified with
 * tv_tree_attention_verify_rope: the kept tree keys were not rotated yet, so
 * each kept K row j = 0..accept_len[b] (the root included) is turned at the
 * position of the row it lands on, L_b + j (its node's position id: the
 * path's j-th node has depth j), and rounded to the cache dtype (bf16:
 * nearest even).  V rows move as in tv_kv_commit.  After the call every row
 * below new_ctx_len holds a rotated key, as the next round expects.
 *   rope_base  finite, > 1, the value verification used; other arguments,
 *   checks and results as tv_kv_commit.
 * ------------------------------------------------------------------------ */
tv_status tv_kv_commit_rope(void *k_cache, void *v_cache, tv_dtype dt, int batch, int Hkv,
                            int cap, int D, const int32_t *ctx_len, const int32_t *accept_len,
                            const int32_t *accepted_nodes, int width, double rope_base,
                            int32_t *new_ctx_len, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
