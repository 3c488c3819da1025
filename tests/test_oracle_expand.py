"""Pins of the layer-wise frontier expansion (oracle/expand.py)."""
import numpy as np
import pytest

import oracle


def _softmax64(x, T=1.0):
    z = np.asarray(x, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


# q is the build's fixed-point softmax: an fp32 exponential of an fp32
# argument |x - m| / T <= 32, so each probability carries a relative error of
# a few 1e-6 against the exact softmax
EDGE_RTOL = 2e-5


def test_width_one_branch_one_is_greedy_decoding():
    """W = 1, m = 1: the tree is the chain of argmax tokens, and each score is
    the product of the chosen tokens' softmax probabilities (fp64 softmax)."""
    r = np.random.default_rng(1)
    b, N, V, steps = 3, 12, 50, 8
    t = oracle.tree_root(b, N, np.arange(b), np.full(b, 7))
    frontier = np.zeros((b, 1), np.int32)
    rows = []
    for k in range(steps):
        logits = (r.standard_normal((b, 1, V)) * 2).astype(np.float32)
        rows.append(logits)
        t, frontier = oracle.tree_expand(logits, 1, frontier, t, np.full(b, 7))
    for s in range(b):
        assert int(t["n_nodes"][s]) == steps + 1
        prod = 1.0
        for k in range(steps):
            node = k + 1
            assert t["parent"][s, node] == k and t["depth"][s, node] == k + 1
            tk = int(np.argmax(rows[k][s, 0]))
            assert t["token"][s, node] == tk
            prod *= _softmax64(rows[k][s, 0])[tk]
            assert abs(t["score"][s, node] - prod) <= EDGE_RTOL * (k + 1) * prod
            assert t["pos"][s, node] == 7 + k + 1


def test_full_expansion_scores_sum_to_one():
    """m = V from the root: the children's scores are a probability vector."""
    r = np.random.default_rng(2)
    V = 40
    t = oracle.tree_root(1, V + 1, [0], [0])
    logits = (r.standard_normal((1, 1, V)) * 3).astype(np.float32)
    t, _ = oracle.tree_expand(logits, V, np.zeros((1, 1), np.int32), t, [0], build_temp=0.8)
    assert abs(t["score"][0, 1:].sum() - 1.0) < 1e-12
    np.testing.assert_allclose(t["score"][0, 1:], np.sort(_softmax64(logits[0, 0], 0.8))[::-1],
                               rtol=EDGE_RTOL, atol=1e-15)


@pytest.mark.parametrize("W,m", [(3, 2), (4, 3), (2, 5)])
def test_structure_frontier_and_capacity(W, m):
    r = np.random.default_rng(W * 10 + m)
    b, N, V = 4, 30, 60
    ctx = np.array([5, 0, 11, 3])
    t = oracle.tree_root(b, N, np.zeros(b, np.int32), ctx)
    frontier = np.full((b, W), -1, np.int32)
    frontier[:, 0] = 0
    for step in range(6):
        logits = (r.standard_normal((b, W, V)) * 1.5).astype(np.float32)
        prev = t
        t, nxt = oracle.tree_expand(logits, m, frontier, t, ctx)
        for s in range(b):
            n0, n1 = int(prev["n_nodes"][s]), int(t["n_nodes"][s])
            live = [f for f in frontier[s] if 0 <= f < n0]
            assert n1 == min(N, n0 + len(live) * m)
            new = list(range(n0, n1))
            # the frontier is the W best new rows by (score desc, row asc)
            best = sorted(new, key=lambda v: (-t["score"][s, v], v))[:W]
            assert list(nxt[s][:len(best)]) == best and (nxt[s][len(best):] == -1).all()
            # each new row hangs under a frontier node, edge score in (0, 1]
            for v in new:
                p = int(t["parent"][s, v])
                assert p in live
                e = t["score"][s, v] / t["score"][s, p]
                assert 0.0 < e <= 1.0 + 1e-12
        frontier = nxt
    # ancestors and depths agree with the independent ancestor routine
    for s in range(b):
        n = int(t["n_nodes"][s])
        anc, depth = oracle.ancestors(t["parent"][s, :n], words=(N + 63) // 64)
        np.testing.assert_array_equal(t["anc"][s, :n], anc)
        np.testing.assert_array_equal(t["depth"][s, :n], depth)
        np.testing.assert_array_equal(t["pos"][s, :n], ctx[s] + depth)


def test_children_are_each_slots_top_m_in_slot_then_rank_order():
    """Brute force per frontier slot: its children sit at consecutive rows in
    slot order; their tokens are the m largest logits of the slot's row
    (ties: lower id), in order; each edge score score(child)/score(parent)
    is the fp64 softmax probability of the child's token."""
    r = np.random.default_rng(11)
    b, W, m, N, V, T = 3, 4, 5, 64, 80, 0.7
    ctx = np.array([2, 9, 0])
    t = oracle.tree_root(b, N, np.zeros(b, np.int32), ctx)
    frontier = np.full((b, W), -1, np.int32)
    frontier[:, 0] = 0
    logits = (r.standard_normal((b, W, V)) * 2).astype(np.float32)
    t, frontier = oracle.tree_expand(logits, m, frontier, t, ctx, build_temp=T)
    frontier[1, 2] = -1                  # an empty slot in the middle
    logits = np.round(r.standard_normal((b, W, V)) * 2).astype(np.float32)  # many ties
    prev = t
    t, _ = oracle.tree_expand(logits, m, frontier, t, ctx, build_temp=T)
    for s in range(b):
        row = int(prev["n_nodes"][s])
        for w in range(W):
            f = int(frontier[s, w])
            if f < 0:
                continue
            order = sorted(range(V), key=lambda i: (-float(logits[s, w, i]), i))[:m]
            p = _softmax64(logits[s, w], T)
            for rk, tok in enumerate(order):
                assert t["parent"][s, row] == f and t["token"][s, row] == tok, (s, w, rk)
                e = t["score"][s, row] / t["score"][s, f]
                assert abs(e - p[tok]) <= EDGE_RTOL * p[tok]
                row += 1
        assert row == int(t["n_nodes"][s])
