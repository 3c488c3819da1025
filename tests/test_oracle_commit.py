"""Pins of the KV commit oracle (oracle/commit.py).

The commit is checked against what it is for, not against its own formula:
after the commit, plain causal attention of an accepted node's query over
the committed cache prefix must equal the tree-masked attention that node
received during verification (the node saw the context plus its ancestors,
which are exactly the committed rows, in order)."""
import numpy as np
import pytest

import oracle


def _tree(r, n, max_children=3):
    parent = np.full(n, -1, np.int32)
    kids = np.zeros(n, np.int64)
    for i in range(1, n):
        ok = [p for p in range(i) if kids[p] < max_children]
        p = ok[r.integers(0, len(ok))]
        parent[i] = p
        kids[p] += 1
    return parent


def _path_to(parent, u):
    path = [u]
    while parent[path[-1]] >= 0:
        path.append(int(parent[path[-1]]))
    return path[::-1]


def _plain_attention(q, k, v, nkeys, scale):
    """q [Hq][D]; k, v [Hkv][cap][D]: softmax over keys [0, nkeys) in fp64."""
    Hq, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    out = np.empty((Hq, D))
    for h in range(Hq):
        kk = k[h // G, :nkeys].astype(np.float64)
        s = kk @ q[h].astype(np.float64) * scale
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ v[h // G, :nkeys].astype(np.float64)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_committed_prefix_reproduces_tree_attention(seed):
    r = np.random.default_rng(seed)
    b, n, L, Hq, Hkv, D = 1, 24, 37, 4, 2, 16
    cap = L + n + 5
    parent = _tree(r, n)
    anc = oracle.ancestors(parent)[0][None]
    q = r.standard_normal((b, n, Hq, D)).astype(np.float32)
    k = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    v = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    scale = 1.0 / np.sqrt(D)
    tree_out, _ = oracle.tree_attention(q, k, v, np.array([L], np.int32), anc,
                                        np.array([n], np.int32), scale)
    for u in r.choice(np.arange(1, n), size=6, replace=False):
        path = _path_to(parent, int(u))
        a = len(path) - 1
        width = a + 3
        acc = np.full((b, width), -1, np.int32)
        acc[0, :a + 1] = path
        k2, v2, new = oracle.kv_commit(k, v, np.array([L]), np.array([a]), acc)
        assert int(new[0]) == L + a + 1
        for j, node in enumerate(path):  # every node on the path, not only u
            got = _plain_attention(q[0, node], k2[0], v2[0], L + j + 1, scale)
            np.testing.assert_allclose(got, tree_out[0, node], rtol=1e-9, atol=1e-9)
        # rows before L and past the committed range are untouched
        np.testing.assert_array_equal(k2[0, :, :L], k[0, :, :L])
        np.testing.assert_array_equal(v2[0, :, L + a + 1:], v[0, :, L + a + 1:])


def test_special_cases():
    r = np.random.default_rng(9)
    b, Hkv, cap, D, L = 4, 2, 30, 8, 5
    k = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    v = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    acc = np.full((b, 6), -1, np.int32)
    acc[0, :1] = [0]                   # root only: nothing moves
    acc[1, :4] = [0, 1, 2, 3]          # a chain accepted in full: identity
    acc[2, :3] = [0, 2, 2]             # not strictly increasing: refused
    acc[3, :3] = [0, 4, cap]           # past the cache: refused
    alen = np.array([0, 3, 2, 2], np.int32)
    k2, v2, new = oracle.kv_commit(k, v, np.full(b, L), alen, acc)
    np.testing.assert_array_equal(new, [L + 1, L + 4, -1, -1])
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)
    # a walk that refused its tree (accept_len -1) commits nothing
    _, _, new = oracle.kv_commit(k, v, np.full(b, L), np.full(b, -1), acc)
    np.testing.assert_array_equal(new, np.full(b, L))


def test_out_of_range_lengths_commit_nothing():
    """accept_len past the width (also INT32_MAX) and a negative context
    length: nothing moves, new length -1."""
    r = np.random.default_rng(10)
    b, Hkv, cap, D = 3, 2, 30, 8
    k = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    v = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    acc = np.tile(np.arange(6, dtype=np.int32), (b, 1))
    alen = np.array([6, 2**31 - 1, 3], np.int32)
    ctx = np.array([4, 4, -3], np.int32)
    k2, v2, new = oracle.kv_commit(k, v, ctx, alen, acc)
    np.testing.assert_array_equal(new, [-1, -1, -1])
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)
