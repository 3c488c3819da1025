/*
 * oracle.c -- plain, slow CPU oracle for one tree-verification round.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP product path
 * never calls it, and the two share no source, header, table or constant.
 *
 * Every function follows a passage of the pages it implements:
 *   TAPS (Target-Aware Prefix-tree Selection), sec. 4.1: per-position top-K
 *       candidate pool drawn from the diffusion drafter's marginals.
 *   TAPS sec. 4.2: edge acceptance q_cond(u->v) propagated into a path-level
 *       reach probability; sec. 1 / 3.2: greedy choice of a compact
 *       prefix-closed subtree that maximises expected accepted tokens under a
 *       verification budget.
 *   TreeGraft sec. 3.1: root r is the verified prefix, s(r) = 1 and
 *       s(v) = product of the edge scores on the path from r to v.
 *   PTD sec. 3.1 ("tree construction"): pi(v) = {v} U pi(P(v)); a node sees
 *       only its ancestors, and its position comes from |pi(v)|.
 *   Speculative-decoding primer (laumy.tech), "acceptance and rejection":
 *       greedy matching up to the first mismatch, then the target's token;
 *       sampled acceptance min(1, p/q); at the first rejection a draw from
 *       the normalised residual (p - q)+; a round emits the accepted prefix
 *       plus one corrected token.
 *
 * The pages fix no arithmetic.  Where a floating-point value decides an
 * integer (tree shape, accepted length, sampled token) this file takes the
 * decision in the precision the GPU kernels use:
 *   exp_spec   fp32 Cody-Waite range reduction + degree-7 Taylor polynomial;
 *   weights    W = rint(exp_spec(x) * 2^44) as u64, row sums exact in u64;
 *   q          fp64 W / fp64 Z;   path score s: fp64 products, root to leaf;
 *   draws      Philox4x64-10 (Salmon et al., SC'11) with a counter per draw;
 *   accept     exact 128-bit integer comparisons.
 * Built with -O2 -ffp-contract=off: every float operation below is a single
 * IEEE operation in the written order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;

#define TVO_OK 0
#define TVO_ERR 1

/* ------------------------------------------------------------------------- */
/* exp_spec: e^x for fp32 x <= 0.                                             */
/* Cody-Waite: x = n ln2 + r with n = rint(x log2 e), r reduced with a two-  */
/* part ln2 (the high part keeps 12 significand bits, so n * hi is exact for */
/* |n| < 2^12); e^r by its Taylor series to degree 7 in Horner form; result  */
/* 2^n * e^r.  Inputs below -32 (and NaN) give 0: their 2^44-scaled weight  */
/* would round to 0 anyway (e^-32 * 2^44 < 0.5 needs x < -31.2).            */
/* ------------------------------------------------------------------------- */
static float c_ln2_hi, c_ln2_lo, c_log2e;
static float c_taylor[8];
static int c_init = 0;

static void constants_init(void)
{
    if (c_init) return;
    const double ln2 = 0.693147180559945309417232121458176568;
    float hi = (float)ln2;
    uint32_t bits;
    memcpy(&bits, &hi, 4);
    bits &= 0xFFFFF000u; /* clear the low 12 significand bits */
    memcpy(&hi, &bits, 4);
    c_ln2_hi = hi;
    c_ln2_lo = (float)(ln2 - (double)hi);
    c_log2e = (float)1.442695040888963407359924681001892137;
    double fact = 1.0;
    for (int i = 0; i < 8; ++i) {
        if (i > 0) fact *= (double)i;
        c_taylor[i] = (float)(1.0 / fact);
    }
    c_init = 1;
}

float tvo_exp_spec(float x)
{
    constants_init();
    if (!(x >= -32.0f)) return 0.0f;
    float t = x * c_log2e;
    float n = rintf(t);
    float r = fmaf(-n, c_ln2_hi, x);
    r = fmaf(-n, c_ln2_lo, r);
    float p = c_taylor[7];
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, c_taylor[i]);
    return ldexpf(p, (int)n);
}

void tvo_exp_spec_n(const float *x, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = tvo_exp_spec(x[i]);
}

void tvo_constants(float *out4)
{
    constants_init();
    out4[0] = c_ln2_hi;
    out4[1] = c_ln2_lo;
    out4[2] = c_log2e;
    out4[3] = c_taylor[7];
}

/* Fixed-point softmax weight of one logit at inverse temperature inv_t,
 * relative to the row maximum m:  x = fl32(fl32(l - m) * inv_t),
 * W = rint(exp_spec(x) * 2^44).  W <= 2^44, so a row of up to 2^18 tokens
 * sums below 2^62 without overflow, in any order. */
uint64_t tvo_weight(float logit, float row_max, float inv_t)
{
    float d = logit - row_max;
    float x = d * inv_t;
    float e = tvo_exp_spec(x);
    float scaled = e * 17592186044416.0f; /* 2^44, exact power-of-two scaling */
    return (uint64_t)rintf(scaled);
}

/* Threads for the independent parts below -- the draft positions of
 * tvo_draft_candidates and the values of tvo_weight_range (1 = none).  Each
 * part is computed exactly as alone, so results do not depend on this. */
static int g_threads = 1;

int tvo_set_threads(int n)
{
    int prev = g_threads;
    g_threads = n < 1 ? 1 : n;
    return prev;
}

/* tvo_weight of every fp32 value whose bit pattern is first_bits + i,
 * 0 <= i < count, as the logit (a helper for exhaustive comparisons). */

void tvo_weight_range(uint32_t first_bits, int64_t count, float row_max_, float inv_t,
                      uint64_t *out)
{
#pragma omp parallel for schedule(static) num_threads(g_threads) if (g_threads > 1)
    for (int64_t i = 0; i < count; ++i) {
        uint32_t bits = first_bits + (uint32_t)i;
        float x;
        memcpy(&x, &bits, sizeof x);
        out[i] = tvo_weight(x, row_max_, inv_t);
    }
}

static float row_max(const float *row, int V)
{
    float m = row[0];
    for (int v = 1; v < V; ++v)
        if (row[v] > m) m = row[v];
    return m;
}

/* Softmax of one row in the weight domain: W[v] and Z = sum W. */
uint64_t tvo_row_weights(const float *row, int V, float inv_t, uint64_t *W)
{
    float m = row_max(row, V);
    uint64_t Z = 0;
    for (int v = 0; v < V; ++v) {
        uint64_t w = tvo_weight(row[v], m, inv_t);
        if (W) W[v] = w;
        Z += w;
    }
    return Z;
}

/* ------------------------------------------------------------------------- */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of the       */
/* Philox S-box on a 4 x 64-bit counter with a 2 x 64-bit key; the key is   */
/* bumped by the Weyl constants between rounds.                              */
/* ------------------------------------------------------------------------- */
static void mulhilo64(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo)
{
    u128 p = (u128)a * (u128)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void tvo_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(M0, c0, &hi0, &lo0);
        mulhilo64(M1, c2, &hi1, &lo1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* One draw of the acceptance walk: key = (seed, 0),
 * counter = (round, sequence, node, slot).  Each node owns two draws: the
 * uniform that decides its own acceptance (slot ACCEPT_SLOT) and the one
 * behind the final draw made at it (slot RESIDUAL_SLOT). */
static void draw(uint64_t seed, uint64_t round, uint64_t seq, uint64_t node, uint64_t slot,
                 uint64_t out[4])
{
    uint64_t ctr[4] = {round, seq, node, slot};
    uint64_t key[2] = {seed, 0};
    tvo_philox4x64_10(ctr, key, out);
}

#define ACCEPT_SLOT 0ULL
#define RESIDUAL_SLOT 0xFFFFFFFFULL

/* ------------------------------------------------------------------------- */
/* Per-position candidate pool (TAPS sec. 4.1) and the drafter's  */
/* probability of each candidate (the plain edge score of TAPS sec. 4.2).   */
/* ------------------------------------------------------------------------- */
typedef struct {
    float val;
    int32_t id;
    double q;
} cand_t;

static int cmp_logit_desc_id_asc(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->val > b->val) return -1;
    if (a->val < b->val) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

static int cmp_q_desc_id_asc(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->q > b->q) return -1;
    if (a->q < b->q) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

/* top-k of one row by (logit desc, id asc): sort the whole row, keep k. */
int tvo_topk(const float *row, int V, int k, int32_t *ids, float *vals)
{
    if (k < 1 || k > V) return TVO_ERR;
    cand_t *all = (cand_t *)malloc(sizeof(cand_t) * (size_t)V);
    if (!all) return TVO_ERR;
    for (int v = 0; v < V; ++v) {
        all[v].val = row[v];
        all[v].id = v;
        all[v].q = 0.0;
    }
    qsort(all, (size_t)V, sizeof(cand_t), cmp_logit_desc_id_asc);
    for (int i = 0; i < k; ++i) {
        ids[i] = all[i].id;
        if (vals) vals[i] = all[i].val;
    }
    free(all);
    return TVO_OK;
}

/* For each of the K positions: top-k tokens by logit, their drafter
 * probability q = W / Z at the build temperature, then re-sorted by
 * (q desc, id asc) -- rank r of a position is its index in this order. */
static int position_candidates(const float *row, int V, int k, float inv_t, int32_t *cand_tok,
                               double *cand_q, uint64_t *Z_out)
{
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)k);
    if (!ids || !c) { free(ids); free(c); return TVO_ERR; }
    tvo_topk(row, V, k, ids, NULL);
    float m = row_max(row, V);
    uint64_t Z = tvo_row_weights(row, V, inv_t, NULL);
    for (int i = 0; i < k; ++i) {
        uint64_t w = tvo_weight(row[ids[i]], m, inv_t);
        c[i].id = ids[i];
        c[i].val = row[ids[i]];
        c[i].q = (double)w / (double)Z;
    }
    qsort(c, (size_t)k, sizeof(cand_t), cmp_q_desc_id_asc);
    for (int i = 0; i < k; ++i) {
        cand_tok[i] = c[i].id;
        cand_q[i] = c[i].q;
    }
    if (Z_out) *Z_out = Z;
    free(ids);
    free(c);
    return TVO_OK;
}

int tvo_draft_candidates(const float *draft, int K, int V, int k, float build_temp,
                         int32_t *cand_tok, double *cand_q, uint64_t *Z_out)
{
    if (K < 1 || V < 1 || k < 1 || k > V || !(build_temp > 0.0f)) return TVO_ERR;
    float inv_t = 1.0f / build_temp;
    int rc = TVO_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads) if (g_threads > 1)
    for (int j = 0; j < K; ++j) {
        if (position_candidates(draft + (size_t)j * (size_t)V, V, k, inv_t,
                                cand_tok + (size_t)j * k, cand_q + (size_t)j * k,
                                Z_out ? Z_out + j : NULL)) {
#pragma omp atomic write
            rc = TVO_ERR;
        }
    }
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Selection order.                                                           */
/* A node of the virtual candidate tree at depth d has rank path            */
/* (r_1..r_d) and score s = fl64(...fl64(fl64(1*q_1(r_1))*q_2(r_2))...).      */
/* Total order (best first):                                                 */
/*   1. larger s;  2. smaller depth;                                          */
/*   3. earlier parent in this same order;  4. smaller sibling rank.          */
/* q <= 1 and rounding is monotone, so a child never beats its parent: every */
/* prefix of this order is a prefix-closed subtree, and the first B nodes    */
/* are the B largest path probabilities (the expected accepted tokens).     */
/* ------------------------------------------------------------------------- */
typedef struct {
    double s;
    int32_t depth;
    int32_t parent; /* output row of the parent (best-first) or position in
                       the parent's level order (exhaustive) */
    int32_t rank;
    int32_t token;
} node_t;

static int better(const node_t *a, const node_t *b)
{
    if (a->s != b->s) return a->s > b->s;
    if (a->depth != b->depth) return a->depth < b->depth;
    if (a->parent != b->parent) return a->parent < b->parent;
    return a->rank < b->rank;
}

/* --- textbook binary heap, best node on top --- */
typedef struct {
    node_t *a;
    int n, cap;
} heap_t;

static int heap_push(heap_t *h, node_t x)
{
    if (h->n == h->cap) {
        int nc = h->cap ? 2 * h->cap : 64;
        node_t *na = (node_t *)realloc(h->a, sizeof(node_t) * (size_t)nc);
        if (!na) return TVO_ERR;
        h->a = na;
        h->cap = nc;
    }
    int i = h->n++;
    h->a[i] = x;
    while (i > 0) {
        int p = (i - 1) / 2;
        if (!better(&h->a[i], &h->a[p])) break;
        node_t t = h->a[i]; h->a[i] = h->a[p]; h->a[p] = t;
        i = p;
    }
    return TVO_OK;
}

static node_t heap_pop(heap_t *h)
{
    node_t top = h->a[0];
    h->a[0] = h->a[--h->n];
    int i = 0;
    for (;;) {
        int l = 2 * i + 1, r = l + 1, b = i;
        if (l < h->n && better(&h->a[l], &h->a[b])) b = l;
        if (r < h->n && better(&h->a[r], &h->a[b])) b = r;
        if (b == i) break;
        node_t t = h->a[i]; h->a[i] = h->a[b]; h->a[b] = t;
        i = b;
    }
    return top;
}

static void write_root(int32_t root_token, int32_t *parent, int32_t *token, int32_t *depth,
                       double *score)
{
    parent[0] = -1;
    token[0] = root_token;
    depth[0] = 0;
    score[0] = 1.0;
}

/* Best-first selection: pop the best node, record it, push all k of its
 * children.  Rows are written in pop order; row 0 is the root. Returns the
 * number of rows written (root included), or -1 on error. */
int tvo_select_best_first(const int32_t *cand_tok, const double *cand_q, int K, int k,
                          int budget, int32_t root_token, int32_t *parent, int32_t *token,
                          int32_t *depth, double *score)
{
    if (K < 1 || k < 1 || budget < 0) return -1;
    write_root(root_token, parent, token, depth, score);
    heap_t h = {0, 0, 0};
    int n = 1;
    for (int r = 0; r < k; ++r) {
        node_t c = {1.0 * cand_q[r], 1, 0, r, cand_tok[r]};
        if (heap_push(&h, c)) { free(h.a); return -1; }
    }
    while (n < budget + 1 && h.n > 0) {
        node_t v = heap_pop(&h);
        parent[n] = v.parent;
        token[n] = v.token;
        depth[n] = v.depth;
        score[n] = v.s;
        if (v.depth < K) {
            const double *q = cand_q + (size_t)v.depth * k;
            const int32_t *t = cand_tok + (size_t)v.depth * k;
            for (int r = 0; r < k; ++r) {
                node_t c = {v.s * q[r], v.depth + 1, n, r, t[r]};
                if (heap_push(&h, c)) { free(h.a); return -1; }
            }
        }
        ++n;
    }
    free(h.a);
    return n;
}

/* Exhaustive selection (tiny inputs only): enumerate every node of the
 * virtual k-ary tree of depth K level by level, sort each level by the order
 * above (parent = position in the sorted previous level), merge all levels
 * by (s desc, depth asc, position asc) and keep the first `budget`. */
static int cmp_level(const void *pa, const void *pb)
{
    const node_t *a = (const node_t *)pa, *b = (const node_t *)pb;
    if (better(a, b)) return -1;
    if (better(b, a)) return 1;
    return 0;
}

typedef struct {
    double s;
    int32_t depth, pos;
} gkey_t;

static int cmp_global(const void *pa, const void *pb)
{
    const gkey_t *a = (const gkey_t *)pa, *b = (const gkey_t *)pb;
    if (a->s != b->s) return a->s > b->s ? -1 : 1;
    if (a->depth != b->depth) return a->depth < b->depth ? -1 : 1;
    return a->pos < b->pos ? -1 : (a->pos > b->pos);
}

int tvo_select_exhaustive(const int32_t *cand_tok, const double *cand_q, int K, int k,
                          int budget, int32_t root_token, int32_t *parent, int32_t *token,
                          int32_t *depth, double *score)
{
    if (K < 1 || k < 1 || budget < 0) return -1;
    /* level sizes k^d; refuse anything that is not tiny */
    int64_t total = 0, sz = 1;
    for (int d = 1; d <= K; ++d) {
        sz *= k;
        total += sz;
        if (total > 4000000) return -1;
    }
    node_t **lvl = (node_t **)calloc((size_t)K + 1, sizeof(node_t *));
    int64_t *lsz = (int64_t *)calloc((size_t)K + 1, sizeof(int64_t));
    lvl[0] = (node_t *)malloc(sizeof(node_t));
    lvl[0][0].s = 1.0; lvl[0][0].depth = 0; lvl[0][0].parent = -1; lvl[0][0].rank = 0;
    lvl[0][0].token = root_token;
    lsz[0] = 1;
    for (int d = 1; d <= K; ++d) {
        lsz[d] = lsz[d - 1] * k;
        lvl[d] = (node_t *)malloc(sizeof(node_t) * (size_t)lsz[d]);
        int64_t m = 0;
        for (int64_t p = 0; p < lsz[d - 1]; ++p)
            for (int r = 0; r < k; ++r) {
                node_t c;
                c.s = lvl[d - 1][p].s * cand_q[(size_t)(d - 1) * k + r];
                c.depth = d;
                c.parent = (int32_t)p; /* position of the parent in its sorted level */
                c.rank = r;
                c.token = cand_tok[(size_t)(d - 1) * k + r];
                lvl[d][m++] = c;
            }
        qsort(lvl[d], (size_t)lsz[d], sizeof(node_t), cmp_level);
    }
    gkey_t *all = (gkey_t *)malloc(sizeof(gkey_t) * (size_t)total);
    int64_t m = 0;
    for (int d = 1; d <= K; ++d)
        for (int64_t p = 0; p < lsz[d]; ++p) {
            all[m].s = lvl[d][p].s;
            all[m].depth = d;
            all[m].pos = (int32_t)p;
            ++m;
        }
    qsort(all, (size_t)total, sizeof(gkey_t), cmp_global);
    int64_t take = total < budget ? total : budget;
    /* output row of every selected (depth, pos); parents precede children */
    int32_t **row_of = (int32_t **)calloc((size_t)K + 1, sizeof(int32_t *));
    for (int d = 0; d <= K; ++d) {
        row_of[d] = (int32_t *)malloc(sizeof(int32_t) * (size_t)lsz[d]);
        for (int64_t p = 0; p < lsz[d]; ++p) row_of[d][p] = -1;
    }
    row_of[0][0] = 0;
    write_root(root_token, parent, token, depth, score);
    int n = 1, bad = 0;
    for (int64_t i = 0; i < take; ++i) {
        const node_t *v = &lvl[all[i].depth][all[i].pos];
        int32_t prow = row_of[all[i].depth - 1][v->parent];
        if (prow < 0) bad = 1; /* would mean the prefix was not closed */
        parent[n] = prow;
        token[n] = v->token;
        depth[n] = v->depth;
        score[n] = v->s;
        row_of[all[i].depth][all[i].pos] = n;
        ++n;
    }
    for (int d = 0; d <= K; ++d) { free(lvl[d]); free(row_of[d]); }
    free(lvl); free(lsz); free(row_of); free(all);
    return bad ? -1 : n;
}

/* ------------------------------------------------------------------------- */
/* Ancestor sets pi(i) = {i} U pi(parent(i)) as bit rows, and depth.    */
/* (PTD sec. 3.1.)  Requires parent[0] = -1 and parent[i] < i.               */
/* ------------------------------------------------------------------------- */
int tvo_ancestors(const int32_t *parent, int n, int words, uint64_t *anc, int32_t *depth)
{
    for (int i = 0; i < n; ++i) {
        uint64_t *row = anc + (size_t)i * words;
        memset(row, 0, sizeof(uint64_t) * (size_t)words);
        int p = parent[i];
        if (i == 0 || p < 0) {
            if (i != 0 && p != -1) return TVO_ERR;
            depth[i] = 0;
        } else {
            if (p >= i) return TVO_ERR;
            memcpy(row, anc + (size_t)p * words, sizeof(uint64_t) * (size_t)words);
            depth[i] = depth[p] + 1;
        }
        row[i / 64] |= 1ULL << (i % 64);
    }
    return TVO_OK;
}

/* Whole builder for a batch of sequences, in the boundary's layouts:
 * draft [b][K][V]; parent/token/depth/pos/score [b][budget+1];
 * anc [b][budget+1][ceil((budget+1)/64)]; n_nodes [b].
 * Rows past n_nodes: parent/token/depth/pos = -1, score 0, anc 0. */
int tvo_tree_build(const float *draft, int batch, int K, int V, int k, int budget,
                   float build_temp, const int32_t *root_token, const int32_t *ctx_len,
                   int32_t *parent, int32_t *token, int32_t *depth, int32_t *pos,
                   double *score, uint64_t *anc, int32_t *n_nodes)
{
    const int N = budget + 1;
    const int words = (N + 63) / 64;
    int32_t *ct = (int32_t *)malloc(sizeof(int32_t) * (size_t)K * k);
    double *cq = (double *)malloc(sizeof(double) * (size_t)K * k);
    int rc = TVO_OK;
    for (int b = 0; b < batch && rc == TVO_OK; ++b) {
        const float *d = draft + (size_t)b * K * V;
        int32_t *pa = parent + (size_t)b * N, *to = token + (size_t)b * N;
        int32_t *de = depth + (size_t)b * N, *po = pos + (size_t)b * N;
        double *sc = score + (size_t)b * N;
        uint64_t *an = anc + (size_t)b * N * words;
        if (tvo_draft_candidates(d, K, V, k, build_temp, ct, cq, NULL)) { rc = TVO_ERR; break; }
        int n = tvo_select_best_first(ct, cq, K, k, budget, root_token[b], pa, to, de, sc);
        if (n < 1) { rc = TVO_ERR; break; }
        for (int i = n; i < N; ++i) {
            pa[i] = -1; to[i] = -1; de[i] = -1; sc[i] = 0.0;
        }
        int32_t *dd = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
        memset(an, 0, sizeof(uint64_t) * (size_t)N * words);
        if (tvo_ancestors(pa, n, words, an, dd)) rc = TVO_ERR;
        free(dd);
        for (int i = 0; i < N; ++i) po[i] = i < n ? ctx_len[b] + de[i] : -1;
        n_nodes[b] = n;
    }
    free(ct);
    free(cq);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* The acceptance walk over one tree.                                       */
/* ------------------------------------------------------------------------- */
#define MODE_GREEDY 0
#define MODE_SAMPLED 1
#define PROPOSAL_POINT_MASS 0
#define PROPOSAL_DRAFT 1

static int argmax_row(const float *row, int V)
{
    int a = 0;
    for (int v = 1; v < V; ++v)
        if (row[v] > row[a]) a = v; /* strict: the lowest id wins ties */
    return a;
}

/* Exact inverse-CDF draw: the 128-bit uniform (hi, lo) picks
 * R = floor((hi 2^64 + lo) * Z / 2^128); the token is the smallest v with
 * sum_{v' <= v} w[v'] > R.  Requires Z = sum w > 0. */
static int inverse_cdf(const uint64_t *w, int V, uint64_t Z, uint64_t hi, uint64_t lo)
{
    u128 a = (u128)hi * Z + (((u128)lo * Z) >> 64);
    uint64_t R = (uint64_t)(a >> 64);
    uint64_t acc = 0;
    for (int v = 0; v < V; ++v) {
        acc += w[v];
        if (acc > R) return v;
    }
    return -1; /* unreachable when Z = sum w */
}

/* Children of u among rows [1, n), in row order. */
static int children_of(const int32_t *parent, int n, int u, int32_t *out)
{
    int c = 0;
    for (int i = 1; i < n; ++i)
        if (parent[i] == u) out[c++] = i;
    return c;
}

static int accept_one(const float *target, const float *draft, int N, int K, int V,
                      const int32_t *parent, const int32_t *token, const int32_t *depth, int n,
                      int mode, float temperature, int proposal, uint64_t seed, uint64_t round,
                      uint64_t seq, int max_depth, int32_t *accept_len, int32_t *acc_nodes,
                      int32_t *out_tokens)
{
    const int width = max_depth + 1;
    for (int i = 0; i < width; ++i) { acc_nodes[i] = -1; out_tokens[i] = -1; }
    *accept_len = -1;
    if (n < 1 || n > N) return TVO_ERR; /* needs a root and at most N rows */
    acc_nodes[0] = 0;
    int32_t *kids = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    uint64_t *W = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)V);
    uint64_t *Wq = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)V);
    uint8_t *excl = (uint8_t *)malloc((size_t)V);
    const float inv_t = mode == MODE_SAMPLED ? 1.0f / temperature : 1.0f;
    int u = 0, len = 0, bonus = -1, rc = TVO_OK;
    for (;;) {
        const float *row = target + (size_t)u * V;
        /* a node at depth max_depth is a leaf of the walk */
        int nk = len < max_depth ? children_of(parent, n, u, kids) : 0;
        if (mode == MODE_GREEDY) {
            int a = argmax_row(row, V);
            int next = -1;
            for (int i = 0; i < nk; ++i)
                if (token[kids[i]] == a) { next = kids[i]; break; }
            if (next < 0) { bonus = a; break; }
            acc_nodes[++len] = next;
            out_tokens[len - 1] = token[next];
            u = next;
            continue;
        }
        uint64_t Z = tvo_row_weights(row, V, inv_t, W);
        uint64_t rnd[4];
        if (proposal == PROPOSAL_POINT_MASS) {
            /* Candidate i is a point-mass proposal delta_t: accept with
             * min(1, p_res(t) / 1) = W_res[t] / Z_res; on rejection t leaves
             * the residual, which is p with the rejected tokens removed. */
            memset(excl, 0, (size_t)V);
            uint64_t Zres = Z;
            int next = -1;
            for (int i = 0; i < nk; ++i) {
                int t = token[kids[i]];
                uint64_t w = (t >= 0 && t < V && !excl[t]) ? W[t] : 0;
                draw(seed, round, seq, (uint64_t)kids[i], ACCEPT_SLOT, rnd);
                u128 lhs = (u128)rnd[0] * Zres;         /* U * Z_res        */
                u128 rhs = (u128)w << 64;               /* W[t] * 2^64      */
                if (lhs < rhs) { next = kids[i]; break; }
                if (t >= 0 && t < V && !excl[t]) { excl[t] = 1; Zres -= w; }
            }
            if (next >= 0) {
                acc_nodes[++len] = next;
                out_tokens[len - 1] = token[next];
                u = next;
                continue;
            }
            for (int v = 0; v < V; ++v) Wq[v] = excl[v] ? 0 : W[v];
            draw(seed, round, seq, (uint64_t)u, RESIDUAL_SLOT, rnd);
            bonus = inverse_cdf(Wq, V, Zres, rnd[0], rnd[1]);
            break;
        }
        /* DRAFT proposal: the child's token was drawn from the drafter's q at
         * its position; chain trees only. */
        if (nk > 1) { rc = TVO_ERR; break; }
        if (nk == 0) {
            draw(seed, round, seq, (uint64_t)u, RESIDUAL_SLOT, rnd);
            bonus = inverse_cdf(W, V, Z, rnd[0], rnd[1]);
            break;
        }
        int c = kids[0];
        int t = token[c];
        int d = depth[c];
        if (d < 1 || d > K || !draft) { rc = TVO_ERR; break; }
        const float *qrow = draft + (size_t)(d - 1) * V;
        uint64_t Zq = tvo_row_weights(qrow, V, inv_t, Wq);
        double pt = (t >= 0 && t < V) ? (double)W[t] / (double)Z : 0.0;
        double qt = (t >= 0 && t < V) ? (double)Wq[t] / (double)Zq : 0.0;
        draw(seed, round, seq, (uint64_t)c, ACCEPT_SLOT, rnd);
        double u53 = (double)(rnd[0] >> 11) * 0x1p-53;
        /* min(1, p/q): p = 0 (including a token outside the vocabulary)
         * gives probability 0, whatever q is */
        int accept = pt > 0.0 && ((pt >= qt) || (u53 < pt / qt));
        if (accept) {
            acc_nodes[++len] = c;
            out_tokens[len - 1] = t;
            u = c;
            continue;
        }
        /* residual (p - q)+ in fp64, scaled to integers by 2^62 */
        uint64_t ZR = 0;
        for (int v = 0; v < V; ++v) {
            double p = (double)W[v] / (double)Z;
            double q = (double)Wq[v] / (double)Zq;
            double r = p - q;
            uint64_t R = r > 0.0 ? (uint64_t)rint(r * 0x1p62) : 0;
            Wq[v] = R;
            ZR += R;
        }
        draw(seed, round, seq, (uint64_t)u, RESIDUAL_SLOT, rnd);
        if (ZR > 0)
            bonus = inverse_cdf(Wq, V, ZR, rnd[0], rnd[1]);
        else /* p == q to rounding: fall back to the target row itself */
            bonus = inverse_cdf(W, V, Z, rnd[0], rnd[1]);
        break;
    }
    if (rc == TVO_OK) {
        *accept_len = len;
        out_tokens[len] = bonus;
    } else {
        *accept_len = -1;
    }
    free(kids); free(W); free(Wq); free(excl);
    return rc;
}

/* Acceptance for a batch: target [b][N][V]; draft [b][K][V] (DRAFT only);
 * parent/token/depth [b][N]; n_nodes [b]; accept_len [b];
 * accepted_nodes / out_tokens [b][max_depth + 1].
 * Sequence b uses Philox counters (round, b, node, slot): node c's
 * acceptance uses (round, b, c, 0), the final draw at node u uses
 * (round, b, u, 0xFFFFFFFF). */
int tvo_tree_accept(const float *target, const float *draft, int batch, int N, int K, int V,
                    const int32_t *parent, const int32_t *token, const int32_t *depth,
                    const int32_t *n_nodes, int mode, float temperature, int proposal,
                    uint64_t seed, uint64_t round, int max_depth, int32_t *accept_len,
                    int32_t *accepted_nodes, int32_t *out_tokens)
{
    int rc = TVO_OK;
    const int width = max_depth + 1;
    for (int b = 0; b < batch; ++b) {
        const float *dr = draft ? draft + (size_t)b * K * V : NULL;
        int r = accept_one(target + (size_t)b * N * V, dr, N, K, V, parent + (size_t)b * N,
                           token + (size_t)b * N, depth + (size_t)b * N, n_nodes[b], mode,
                           temperature, proposal, seed, round, (uint64_t)b, max_depth,
                           accept_len + b, accepted_nodes + (size_t)b * width,
                           out_tokens + (size_t)b * width);
        if (r) rc = r;
    }
    return rc;
}
