"""Pins of the oracle's tree builder.

* top-k against numpy's lexsort (a library sort).
* best-first selection equals the exhaustive top-B of every path of the
  candidate tree (TAPS sec. 4.2 / 4.1: path reach probability, compact
  prefix-closed subtree under a budget), with and without score ties.
* for tiny trees, the selected subtree has the largest sum of path
  probabilities -- the expected number of accepted tokens -- among ALL
  prefix-closed subtrees of the same size (brute force).
* path scores are the products of the candidates' probabilities along the
  path (TreeGraft sec. 3.1), and the root's score is 1.
* ancestor bit rows: pi(v) = {v} U pi(P(v)) (PTD sec. 3.1).
"""
import itertools

import numpy as np
import pytest

import workloads


def test_topk_matches_lexsort(orc):
    r = np.random.default_rng(3)
    for V, k in [(1000, 4), (5000, 16), (64, 64), (7, 1)]:
        row = (r.standard_normal(V) * 2).astype(np.float32)
        row[r.integers(0, V, size=V // 5)] = row[0]           # plenty of ties
        ids, vals = orc.topk(row, k)
        order = np.lexsort((np.arange(V), -row.astype(np.float64)))
        assert np.array_equal(ids, order[:k])
        assert np.array_equal(vals, row[order[:k]])


def test_candidates_sorted_and_probabilities(orc):
    r = np.random.default_rng(4)
    draft = (r.standard_normal((5, 300)) * 2).astype(np.float32)
    tok, q, Z = orc.draft_candidates(draft, 6)
    for j in range(5):
        # same token set as the top-6 by logit
        ids, _ = orc.topk(draft[j], 6)
        assert set(tok[j]) == set(ids)
        # ordered by (q desc, id asc)
        key = list(zip(-q[j], tok[j]))
        assert key == sorted(key)
        # q is the softmax probability of the token (within fp32 error budget)
        x = draft[j].astype(np.float64)
        p = np.exp(x - x.max()) / np.exp(x - x.max()).sum()
        assert np.allclose(q[j], p[tok[j]], rtol=1e-5)


def _random_candidates(r, K, k, ties=False):
    if ties:
        levels = np.array([0.5, 0.25, 0.125, 0.0625, 0.03125])
        q = levels[r.integers(0, len(levels), size=(K, k))]
        q = -np.sort(-q, axis=1)
    else:
        q = r.dirichlet(np.ones(k * 3), size=K)[:, :k]
        q = -np.sort(-q, axis=1)
    tok = r.integers(0, 1000, size=(K, k)).astype(np.int32)
    return tok, q


@pytest.mark.parametrize("K,k,B", [(4, 4, 16), (3, 2, 6), (3, 3, 39), (5, 2, 20),
                                   (2, 5, 30), (4, 3, 200), (1, 4, 3), (3, 1, 2)])
@pytest.mark.parametrize("ties", [False, True])
def test_best_first_equals_exhaustive(orc, K, k, B, ties):
    r = np.random.default_rng(K * 100 + k * 10 + B + (7 if ties else 0))
    for _ in range(5):
        tok, q = _random_candidates(r, K, k, ties)
        a = orc.select_best_first(tok, q, B, root_token=7)
        b = orc.select_exhaustive(tok, q, B, root_token=7)
        for f in ("parent", "token", "depth", "score"):
            assert np.array_equal(a[f], b[f]), f
        total = sum(k ** d for d in range(1, K + 1))
        assert a["n"] == min(B, total) + 1


def _all_paths(K, k):
    for d in range(1, K + 1):
        for path in itertools.product(range(k), repeat=d):
            yield path


def _path_score(q, path):
    s = 1.0
    for j, r in enumerate(path):
        s = s * q[j, r]
    return s


def test_selection_is_top_b_by_path_probability(orc):
    r = np.random.default_rng(5)
    K, k, B = 4, 3, 25
    tok, q = _random_candidates(r, K, k)
    sel = orc.select_best_first(tok, q, B)
    scores = sorted((_path_score(q, p) for p in _all_paths(K, k)), reverse=True)
    assert np.allclose(sel["score"][1:], scores[:B], rtol=1e-15, atol=0)
    assert sel["score"][0] == 1.0
    # every node's score is its parent's score times its own candidate q
    for i in range(1, sel["n"]):
        p = sel["parent"][i]
        d = sel["depth"][i]
        j = list(tok[d - 1]).index(sel["token"][i])
        assert sel["score"][i] == sel["score"][p] * q[d - 1, j]


def _prefix_closed_subsets(K, k, size):
    nodes = list(_all_paths(K, k))
    for comb in itertools.combinations(nodes, size):
        s = set(comb)
        if all(len(p) == 1 or p[:-1] in s for p in comb):
            yield comb


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6])
def test_selection_maximises_expected_accepted_tokens(orc, B):
    """Brute force over every prefix-closed subtree of size B (K=3, k=2)."""
    r = np.random.default_rng(50 + B)
    K, k = 3, 2
    for _ in range(4):
        tok, q = _random_candidates(r, K, k)
        sel = orc.select_best_first(tok, q, B)
        ours = float(np.sum(sel["score"][1:]))
        best = max(sum(_path_score(q, p) for p in sub) for sub in _prefix_closed_subsets(K, k, B))
        assert ours >= best - 1e-12


def _check_prefix_closed(parent, depth, n):
    assert parent[0] == -1 and depth[0] == 0
    for i in range(1, n):
        assert 0 <= parent[i] < i
        assert depth[i] == depth[parent[i]] + 1


def test_tree_build_batch_layout(orc):
    cfg = dict(workloads.CONFIGS["tiny"])
    draft, _ = workloads.logits(cfg, 2, cfg["B"] + 1)
    ctx = np.array([128, 77], np.int32)
    out = orc.tree_build(draft, cfg["k"], cfg["B"], np.array([3, 4], np.int32), ctx)
    N = cfg["B"] + 1
    for b in range(2):
        n = out["n_nodes"][b]
        assert n == N
        _check_prefix_closed(out["parent"][b], out["depth"][b], n)
        assert np.all(out["pos"][b, :n] == ctx[b] + out["depth"][b, :n])
        assert np.all(np.diff(out["score"][b, 1:n]) <= 0)        # best-first order
        tok, q, _ = orc.draft_candidates(draft[b], cfg["k"])
        ref = orc.select_exhaustive(tok, q, cfg["B"], root_token=3 + b)
        assert np.array_equal(out["parent"][b, :n], ref["parent"])
        assert np.array_equal(out["token"][b, :n], ref["token"])


def test_tree_build_small_candidate_tree(orc):
    """A budget above the size of the whole candidate tree emits all of it."""
    r = np.random.default_rng(6)
    draft = r.standard_normal((1, 2, 50)).astype(np.float32)
    out = orc.tree_build(draft, 3, 20, np.array([0], np.int32), np.array([5], np.int32))
    n = out["n_nodes"][0]
    assert n == 1 + 3 + 9
    assert np.all(out["parent"][0, n:] == -1) and np.all(out["anc"][0, n:] == 0)


def test_ancestor_rows(orc):
    r = np.random.default_rng(7)
    for n in (1, 2, 17, 65, 130):
        parent = np.full(n, -1, np.int32)
        for i in range(1, n):
            parent[i] = r.integers(0, i)
        anc, depth = orc.ancestors(parent)
        for i in range(n):
            bits = {j for j in range(n) if (int(anc[i, j // 64]) >> (j % 64)) & 1}
            chain, v = set(), i
            while v >= 0:
                chain.add(v)
                v = parent[v] if v > 0 else -1
            assert bits == chain
            assert depth[i] == len(chain) - 1
    # a chain: row i holds bits 0..i
    parent = np.arange(-1, 99, dtype=np.int32)
    anc, depth = orc.ancestors(parent)
    for i in range(100):
        full = (1 << (i + 1)) - 1
        got = int(anc[i, 0]) | (int(anc[i, 1]) << 64)
        assert got == full and depth[i] == i
    with pytest.raises(ValueError):
        orc.ancestors(np.array([-1, 2, 0], np.int32))
