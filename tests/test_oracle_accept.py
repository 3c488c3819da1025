"""Pins of the oracle's acceptance walk.

(iv) greedy: the emitted tokens equal token-by-token argmax decoding of a
     synthetic target model f(path), and accept_len is the longest tree path
     that matches that decoding (primer: greedy acceptance keeps drafts while
     the target agrees, then substitutes the target's token).
(v)  sampled: the emitted token is distributed as the target's p
     (chi-square over 10^6 trials), the acceptance rate of a draft drawn from
     q is sum_v min(p, q) (primer: alpha = min(1, p/q) and the residual
     (p - q)+), and for a tree of deterministic candidates the law of the
     first two emitted tokens equals autoregressive sampling of f.
Plus the primer's own worked example (tests/golden/primer_chain_example.json).
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

ALPHA = 1e-3
TRIALS = 1_000_000


# --------------------------------------------------------------------------
# synthetic target model f(path): per-depth base rows plus a path-hash term
# --------------------------------------------------------------------------
class PathModel:
    def __init__(self, V, max_depth, seed, sigma=2.0, eta=1.0):
        r = np.random.default_rng(seed)
        self.V = V
        self.base = (r.standard_normal((max_depth + 2, V)) * sigma).astype(np.float32)
        self.eta = eta
        self.seed = seed

    def row(self, path):
        h = np.random.default_rng([self.seed, 7919] + [int(t) + 1 for t in path])
        eps = h.standard_normal(self.V).astype(np.float32)
        return (self.base[len(path) - 1] + np.float32(self.eta) * eps).astype(np.float32)

    def greedy_decode(self, root, steps):
        path, out = [root], []
        for _ in range(steps):
            a = int(np.argmax(self.row(path)))    # numpy argmax: lowest id on ties
            out.append(a)
            path.append(a)
        return out


def _paths(parent, token, n):
    paths = [[int(token[0])]]
    for i in range(1, n):
        paths.append(paths[parent[i]] + [int(token[i])])
    return paths


def _target_rows(model, parent, token, n, N):
    t = np.zeros((N, model.V), np.float32)
    for i, p in enumerate(_paths(parent, token, n)):
        t[i] = model.row(p)
    return t


def _random_tree_unique(r, n, V, max_children=3):
    parent = np.full(n, -1, np.int32)
    token = np.zeros(n, np.int32)
    token[0] = r.integers(0, V)
    kids = {0: []}
    for i in range(1, n):
        ok = [p for p in range(i) if len(kids[p]) < max_children]
        p = ok[r.integers(0, len(ok))]
        free = [t for t in range(V) if t not in [token[c] for c in kids[p]]]
        parent[i] = p
        token[i] = free[r.integers(0, len(free))]
        kids[p].append(i)
        kids[i] = []
    depth = np.zeros(n, np.int32)
    for i in range(1, n):
        depth[i] = depth[parent[i]] + 1
    return parent, token, depth


def _longest_match(parent, token, n, ar):
    best = 0
    for i, p in enumerate(_paths(parent, token, n)):
        d = len(p) - 1
        if d > 0 and p[1:] == ar[:d]:
            best = max(best, d)
    return best


@pytest.mark.parametrize("seed", range(8))
def test_greedy_equals_argmax_decoding_random_tree(orc, seed):
    r = np.random.default_rng(seed)
    V, n = 12, 30
    parent, token, depth = _random_tree_unique(r, n, V)
    model = PathModel(V, int(depth.max()) + 1, seed=seed, sigma=1.0, eta=0.5)
    # plant: make the tree follow the model's own argmax along one branch
    ar = model.greedy_decode(int(token[0]), int(depth.max()) + 1)
    u = 0
    for a in ar:
        kids = [c for c in range(1, n) if parent[c] == u]
        if not kids:
            break
        c = kids[r.integers(0, len(kids))]
        if a in [token[x] for x in kids if x != c]:
            break
        token[c] = a
        u = c
        if r.random() < 0.2:
            break
    target = _target_rows(model, parent, token, n, n)
    res = orc.tree_accept(target[None], parent[None], token[None], depth[None], np.array([n]),
                          mode=orc.GREEDY, max_depth=int(depth.max()))
    L = int(res["accept_len"][0])
    assert L == _longest_match(parent, token, n, ar)
    assert list(res["out_tokens"][0, :L + 1]) == ar[:L + 1]
    assert np.all(res["out_tokens"][0, L + 1:] == -1)
    nodes = res["accepted_nodes"][0]
    assert nodes[0] == 0 and np.all(nodes[L + 1:] == -1)
    for j in range(1, L + 1):
        assert parent[nodes[j]] == nodes[j - 1]


def test_greedy_on_built_tree(orc):
    """The oracle's own builder from drafter marginals close to f, then (iv)."""
    V, K, k, B = 40, 5, 3, 30
    model = PathModel(V, K + 1, seed=99, sigma=2.0, eta=0.3)
    root = 5
    ar = model.greedy_decode(root, K + 1)
    r = np.random.default_rng(1)
    draft = np.stack([model.row([root] + ar[:j]) + r.standard_normal(V).astype(np.float32)
                      for j in range(K)])
    tree = orc.tree_build(draft[None], k, B, np.array([root], np.int32), np.array([0], np.int32))
    n = int(tree["n_nodes"][0])
    parent, token, depth = tree["parent"][0], tree["token"][0], tree["depth"][0]
    target = _target_rows(model, parent, token, n, B + 1)
    res = orc.tree_accept(target[None], parent[None], token[None], depth[None],
                          tree["n_nodes"], mode=orc.GREEDY, max_depth=K)
    L = int(res["accept_len"][0])
    assert L == _longest_match(parent, token, n, ar)
    assert list(res["out_tokens"][0, :L + 1]) == ar[:L + 1]


def test_primer_worked_example(orc):
    path = os.path.join(os.path.dirname(__file__), "golden", "primer_chain_example.json")
    ex = json.load(open(path))
    t = np.array(ex["target_logits"], np.float32)[None]
    n = len(ex["parent"])
    res = orc.tree_accept(t, np.array([ex["parent"]]), np.array([ex["token"]]),
                          np.array([ex["depth"]]), np.array([n]), mode=orc.GREEDY, max_depth=3)
    L = ex["expected_accept_len"]
    assert res["accept_len"][0] == L
    assert list(res["out_tokens"][0, :L + 1]) == ex["expected_out_tokens"]
    assert list(res["accepted_nodes"][0, :L + 1]) == ex["expected_accepted_nodes"]


def test_greedy_root_only_and_depth_cut(orc):
    r = np.random.default_rng(3)
    V = 9
    t = r.standard_normal((1, 6, V)).astype(np.float32)
    res = orc.tree_accept(t, np.array([[-1, 0, 0, 0, 0, 0]]), np.zeros((1, 6), np.int32),
                          np.zeros((1, 6), np.int32), np.array([1]), mode=orc.GREEDY, max_depth=5)
    assert res["accept_len"][0] == 0 and res["out_tokens"][0, 0] == int(np.argmax(t[0, 0]))
    # a chain that the target always agrees with, cut at max_depth = 3
    parent = np.arange(-1, 5, dtype=np.int32)
    token = np.zeros(6, np.int32)
    for i in range(1, 6):
        token[i] = int(np.argmax(t[0, i - 1]))
    res = orc.tree_accept(t, parent[None], token[None], np.arange(6, dtype=np.int32)[None],
                          np.array([6]), mode=orc.GREEDY, max_depth=3)
    assert res["accept_len"][0] == 3
    assert res["out_tokens"][0, 3] == int(np.argmax(t[0, 3]))


# --------------------------------------------------------------------------
# sampled acceptance
# --------------------------------------------------------------------------
def _softmax(x):
    x = x.astype(np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _chisq_pvalue(counts, probs):
    counts = np.asarray(counts, np.float64)
    exp = probs * counts.sum()
    keep = exp >= 5
    c, e = counts[keep], exp[keep]
    rest_c, rest_e = counts[~keep].sum(), exp[~keep].sum()
    if rest_e > 0:
        c = np.append(c, rest_c)
        e = np.append(e, rest_e)
    return stats.chisquare(c, e * c.sum() / e.sum()).pvalue


def _draft_chain_trials(orc, p_logits, q_logits, root_tok, y, T=1.0, seed=11):
    V = p_logits.shape[0]
    b = y.shape[0]
    target = np.broadcast_to(np.stack([p_logits, p_logits]), (b, 2, V))
    draft = np.broadcast_to(q_logits[None], (b, 1, V))
    parent = np.broadcast_to(np.array([-1, 0], np.int32), (b, 2))
    token = np.stack([np.full(b, root_tok, np.int32), y.astype(np.int32)], axis=1)
    depth = np.broadcast_to(np.array([0, 1], np.int32), (b, 2))
    return orc.tree_accept(target, parent, token, depth, np.full(b, 2, np.int32),
                           mode=orc.SAMPLED, temperature=T, proposal=orc.DRAFT, seed=seed,
                           round=3, max_depth=1, draft=draft)


def test_draft_proposal_preserves_target_and_rate(orc):
    r = np.random.default_rng(21)
    V = 8
    p_l = (r.standard_normal(V) * 1.5).astype(np.float32)
    q_l = (p_l + r.standard_normal(V)).astype(np.float32)
    p, q = _softmax(p_l), _softmax(q_l)
    y = r.choice(V, size=TRIALS, p=q)
    res = _draft_chain_trials(orc, p_l, q_l, 0, y)
    first = res["out_tokens"][:, 0]
    assert _chisq_pvalue(np.bincount(first, minlength=V), p) > ALPHA
    acc = (res["accept_len"] == 1).mean()
    closed = np.minimum(p, q).sum()
    sd = np.sqrt(closed * (1 - closed) / TRIALS)
    assert abs(acc - closed) < 5 * sd


def test_draft_proposal_at_other_temperature(orc):
    r = np.random.default_rng(22)
    V, T = 8, 0.7
    p_l = (r.standard_normal(V) * 1.5).astype(np.float32)
    q_l = (p_l + r.standard_normal(V)).astype(np.float32)
    p, q = _softmax(p_l / T), _softmax(q_l / T)
    y = r.choice(V, size=TRIALS // 2, p=q)
    res = _draft_chain_trials(orc, p_l, q_l, 0, y, T=T)
    assert _chisq_pvalue(np.bincount(res["out_tokens"][:, 0], minlength=V), p) > ALPHA


def test_negative_control_draft_rule_on_deterministic_child(orc):
    """min(1, p/q) with q the drafter's marginal is NOT lossless when the
    child is the drafter's deterministic top-1 instead of a draw from q."""
    r = np.random.default_rng(23)
    V = 8
    p_l = (r.standard_normal(V) * 1.5).astype(np.float32)
    q_l = (p_l + r.standard_normal(V)).astype(np.float32)
    p = _softmax(p_l)
    y = np.full(TRIALS // 4, int(np.argmax(q_l)))
    res = _draft_chain_trials(orc, p_l, q_l, 0, y)
    assert _chisq_pvalue(np.bincount(res["out_tokens"][:, 0], minlength=V), p) < 1e-12


def _point_mass_trials(orc, parent, token, depth, target, trials, seed=5, T=1.0):
    n = parent.shape[0]
    V = target.shape[1]
    return orc.tree_accept(np.broadcast_to(target, (trials, n, V)),
                           np.broadcast_to(parent, (trials, n)),
                           np.broadcast_to(token, (trials, n)),
                           np.broadcast_to(depth, (trials, n)), np.full(trials, n, np.int32),
                           mode=orc.SAMPLED, temperature=T, proposal=orc.POINT_MASS,
                           seed=seed, round=0, max_depth=int(depth.max()) + 1)


def _reach_probabilities(parent, token, P):
    """Pr(walk reaches v) = product over the path of p_parent(token)."""
    n = parent.shape[0]
    reach = np.zeros(n)
    reach[0] = 1.0
    for i in range(1, n):
        reach[i] = reach[parent[i]] * P[parent[i]][token[i]]
    return reach


@pytest.mark.parametrize("seed", [0, 1])
def test_point_mass_tree_preserves_target(orc, seed):
    r = np.random.default_rng(30 + seed)
    V, n = 8, 10
    parent, token, depth = _random_tree_unique(r, n, V, max_children=3)
    target = (r.standard_normal((n, V)) * 1.5).astype(np.float32)
    P = [_softmax(target[i]) for i in range(n)]
    res = _point_mass_trials(orc, parent, token, depth, target, TRIALS, seed=seed)
    out = res["out_tokens"]
    L = res["accept_len"]
    # first emitted token ~ p at the root
    assert _chisq_pvalue(np.bincount(out[:, 0], minlength=V), P[0]) > ALPHA
    # joint law of (first token, second token if the first was a child):
    # AR sampling of the model gives p_root(a) p_child(a)(b)
    kids = {int(token[c]): c for c in range(1, n) if parent[c] == 0}
    probs, cats = [], {}
    for a in range(V):
        if a in kids:
            for bb in range(V):
                cats[(a, bb)] = len(probs)
                probs.append(P[0][a] * P[kids[a]][bb])
        else:
            cats[(a, None)] = len(probs)
            probs.append(P[0][a])
    counts = np.zeros(len(probs))
    for a in range(V):
        sel = out[:, 0] == a
        if a in kids:
            counts[[cats[(a, bb)] for bb in range(V)]] += np.bincount(out[sel, 1], minlength=V)
        else:
            counts[cats[(a, None)]] += sel.sum()
    assert _chisq_pvalue(counts, np.array(probs)) > ALPHA
    # acceptance at the root: sum of the children's target probabilities
    closed = sum(P[0][t] for t in kids)
    sd = np.sqrt(closed * (1 - closed) / TRIALS)
    assert abs((L >= 1).mean() - closed) < 5 * sd
    # mean accepted length: sum over drafted nodes of their reach probability
    reach = _reach_probabilities(parent, token, P)
    mean_closed = reach[1:].sum()
    assert abs(L.mean() - mean_closed) < 5 * L.std() / np.sqrt(TRIALS)


def test_point_mass_duplicate_siblings_and_leaf(orc):
    r = np.random.default_rng(40)
    V = 8
    parent = np.array([-1, 0, 0, 0], np.int32)
    token = np.array([0, 2, 2, 5], np.int32)       # a repeated candidate token
    depth = np.array([0, 1, 1, 1], np.int32)
    target = (r.standard_normal((4, V)) * 1.5).astype(np.float32)
    p = _softmax(target[0])
    res = _point_mass_trials(orc, parent, token, depth, target, TRIALS // 2)
    assert _chisq_pvalue(np.bincount(res["out_tokens"][:, 0], minlength=V), p) > ALPHA
    # the second copy of token 2 is never taken
    assert not np.any(res["accepted_nodes"][:, 1] == 2)
    # a bare root (leaf): the bonus token is a draw from p
    res = _point_mass_trials(orc, parent[:1], token[:1], depth[:1], target[:1], TRIALS // 2)
    assert np.all(res["accept_len"] == 0)
    assert _chisq_pvalue(np.bincount(res["out_tokens"][:, 0], minlength=V), p) > ALPHA


def test_draft_proposal_rejects_branching_tree(orc):
    r = np.random.default_rng(41)
    t = r.standard_normal((1, 3, 8)).astype(np.float32)
    res = orc.tree_accept(t, np.array([[-1, 0, 0]]), np.array([[0, 1, 2]]),
                          np.array([[0, 1, 1]]), np.array([3]), mode=orc.SAMPLED,
                          proposal=orc.DRAFT, max_depth=1, draft=t[:, :1])
    assert res["accept_len"][0] == -1


def test_draft_proposal_zero_target_mass_never_accepted(orc):
    """min(1, p/q) is 0 where p is 0: a child whose token the target gives no
    mass (a -inf logit, or a token outside the vocabulary) is rejected on
    every draw, even where q is 0 too; where q is 0 and p is not, the child
    is accepted on every draw."""
    V, b = 8, 400
    p_l = np.linspace(-1.0, 1.0, V).astype(np.float32)
    q_l = p_l.copy()
    p_l[3] = -np.inf          # p(3) = 0, q(3) > 0
    p_l[5] = q_l[5] = -np.inf  # p(5) = q(5) = 0
    q_l[6] = -np.inf          # q(6) = 0 < p(6)
    for y, expect in ((3, 0), (5, 0), (-2, 0), (V + 1, 0), (6, 1)):
        res = _draft_chain_trials(orc, p_l, q_l, 0, np.full(b, y))
        assert np.all(res["accept_len"] == expect), (y, expect)
        if expect == 0:  # the residual never emits a token of zero target mass
            first = res["out_tokens"][:, 0]
            assert np.all((first >= 0) & (first < V) & (first != 3) & (first != 5))


def test_draws_are_keyed_by_the_deciding_node(orc):
    """Pin of the draw layout, written from the Philox words alone: child c
    of the root is accepted iff U_c * Z_res < W(t_c) * 2^64 with U_c = word 0
    of counter (round, b, c, 0) under key (seed, 0), Z_res the root's mass
    minus the tokens already rejected; after both children are rejected the
    emitted token is the smallest v whose running residual mass exceeds
    floor(U * Z_res / 2^128), U = words 0, 1 of (round, b, 0, 0xFFFFFFFF)."""
    r = np.random.default_rng(44)
    V, b, rnd = 12, 3, 7
    row = (r.standard_normal(V) * 0.8).astype(np.float32)
    W, Z = orc.row_weights(row)
    W = [int(w) for w in W]
    t1, t2 = 4, 9
    target = np.broadcast_to(row, (b, 3, V))
    parent = np.broadcast_to(np.array([-1, 0, 0], np.int32), (b, 3))
    token = np.broadcast_to(np.array([0, t1, t2], np.int32), (b, 3))
    depth = np.broadcast_to(np.array([0, 1, 1], np.int32), (b, 3))
    seen = set()
    for seed in range(60):
        res = orc.tree_accept(target, parent, token, depth, np.full(b, 3, np.int32),
                              mode=orc.SAMPLED, seed=seed, round=rnd, max_depth=1)
        for s in range(b):
            key = [seed, 0]
            u1 = int(orc.philox([rnd, s, 1, 0], key)[0])
            u2 = int(orc.philox([rnd, s, 2, 0], key)[0])
            if u1 * Z < W[t1] << 64:
                want = (1, t1)
            elif u2 * (Z - W[t1]) < W[t2] << 64:
                want = (1, t2)
            else:
                f = orc.philox([rnd, s, 0, 0xFFFFFFFF], key)
                U = (int(f[0]) << 64) | int(f[1])
                zres = Z - W[t1] - W[t2]
                R = (U * zres) >> 128
                run, tok = 0, None
                for v in range(V):
                    run += 0 if v in (t1, t2) else W[v]
                    if run > R:
                        tok = v
                        break
                want = (0, tok)
            got = (int(res["accept_len"][s]), int(res["out_tokens"][s, 0]))
            assert got == want, (seed, s, got, want)
            seen.add(want[0] if want[0] == 0 else want[1])
    assert seen == {0, t1, t2}  # every branch of the rule was exercised


def test_sampled_is_replayable(orc):
    """Same (seed, round) -> same draws; another round -> other draws."""
    r = np.random.default_rng(42)
    V, n = 50, 12
    parent, token, depth = _random_tree_unique(r, n, V)
    target = r.standard_normal((8, n, V)).astype(np.float32)
    args = (target, np.broadcast_to(parent, (8, n)), np.broadcast_to(token, (8, n)),
            np.broadcast_to(depth, (8, n)), np.full(8, n))
    a = orc.tree_accept(*args, mode=orc.SAMPLED, seed=9, round=4, max_depth=12)
    b = orc.tree_accept(*args, mode=orc.SAMPLED, seed=9, round=4, max_depth=12)
    c = orc.tree_accept(*args, mode=orc.SAMPLED, seed=9, round=5, max_depth=12)
    assert all(np.array_equal(a[f], b[f]) for f in a)
    assert not np.array_equal(a["out_tokens"], c["out_tokens"])
