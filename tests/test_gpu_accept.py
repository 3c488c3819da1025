"""GPU parity of tv_tree_accept with the oracle: bit-exact accept_len,
accepted_nodes and out_tokens for the same (seed, round) draws."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import assert_accept_equal, bf16_dev, dev

pytestmark = pytest.mark.gpu


def _random_trees(r, b, N, V, max_children=4, ns=None):
    parent = np.full((b, N), -1, np.int32)
    token = r.integers(0, V, size=(b, N)).astype(np.int32)
    depth = np.zeros((b, N), np.int32)
    for s in range(b):
        kids = np.zeros(N, np.int64)
        for i in range(1, N):
            ok = [p for p in range(i) if kids[p] < max_children]
            p = ok[r.integers(0, len(ok))]
            parent[s, i] = p
            depth[s, i] = depth[s, p] + 1
            kids[p] += 1
    n = np.full(b, N, np.int32) if ns is None else np.asarray(ns, np.int32)
    return parent, token, depth, n


def _both(target, parent, token, depth, n, *, mode, dtype="f32", draft=None, **kw):
    if dtype == "bf16":
        target = workloads.round_bf16(target)
        draft = workloads.round_bf16(draft) if draft is not None else None
        put = bf16_dev
    else:
        put = dev
    g = tv.tv_tree_accept(put(target), dev(parent), dev(token), dev(depth), dev(n), mode=mode,
                          draft_logits=put(draft) if draft is not None else None, **kw)
    torch.cuda.synchronize()
    o = oracle.tree_accept(target, parent, token, depth, n, mode=mode, draft=draft, **kw)
    return g, o


CASES = [
    # name, b, N, V, sigma, plant, max_children, dtype
    ("tiny", 1, 17, 1000, 2.0, 4.0, 4, "f32"),
    ("batch", 8, 33, 5000, 3.0, 9.0, 4, "f32"),
    ("bf16", 4, 33, 4097, 3.0, 9.0, 3, "bf16"),
    ("wide", 2, 200, 3000, 1.0, 2.5, 64, "f32"),
    ("vocab-1", 2, 9, 1, 1.0, 0.0, 4, "f32"),
    ("full-vocab", 2, 65, 151936, 3.0, 12.0, 8, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", ["greedy", "sampled"])
def test_accept_random_trees(case, mode):
    name, b, N, V, sig, plant, mc, dt = case
    r = np.random.default_rng(zlib.crc32(name.encode()))
    parent, token, depth, n = _random_trees(r, b, N, V, mc, ns=[N] + [max(1, N - 3 * s) for s in range(1, b)])
    target = (r.standard_normal((b, N, V)) * sig).astype(np.float32)
    target = workloads.plant(target, parent, token, n, plant)
    md = int(depth.max()) + 1
    kw = dict(max_depth=md)
    if mode == "greedy":
        g, o = _both(target, parent, token, depth, n, mode=oracle.GREEDY, dtype=dt, **kw)
        assert_accept_equal(g, o, name)
    else:
        for T, rnd in ((1.0, 0), (0.7, 5), (1.6, 9)):
            g, o = _both(target, parent, token, depth, n, mode=oracle.SAMPLED, dtype=dt,
                         temperature=T, seed=1234, round=rnd, **kw)
            assert_accept_equal(g, o, f"{name} T={T}")


def test_accept_depth_cut_and_root_only():
    r = np.random.default_rng(2)
    b, N, V = 3, 12, 50
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (b, 1))
    depth = np.tile(np.arange(N, dtype=np.int32), (b, 1))
    target = r.standard_normal((b, N, V)).astype(np.float32)
    token = np.zeros((b, N), np.int32)
    for s in range(b):
        for i in range(1, N):
            token[s, i] = int(np.argmax(target[s, i - 1]))
    n = np.array([N, 1, 7], np.int32)
    for md in (1, 4, 11, 15):
        g, o = _both(target, parent, token, depth, n, mode=oracle.GREEDY, max_depth=md)
        assert_accept_equal(g, o, f"greedy md={md}")
        g, o = _both(target, parent, token, depth, n, mode=oracle.SAMPLED, max_depth=md,
                     seed=77, round=md)
        assert_accept_equal(g, o, f"sampled md={md}")


def test_accept_duplicate_and_invalid_tokens():
    r = np.random.default_rng(3)
    b, V = 64, 10
    parent = np.tile(np.array([-1, 0, 0, 0, 0, 1], np.int32), (b, 1))
    depth = np.tile(np.array([0, 1, 1, 1, 1, 2], np.int32), (b, 1))
    token = np.tile(np.array([0, 3, 3, -4, 99, 2], np.int32), (b, 1))
    target = (r.standard_normal((b, 6, V)) * 1.5).astype(np.float32)
    n = np.full(b, 6, np.int32)
    g, o = _both(target, parent, token, depth, n, mode=oracle.SAMPLED, max_depth=3, seed=5)
    assert_accept_equal(g, o, "dup")
    g, o = _both(target, parent, token, depth, n, mode=oracle.GREEDY, max_depth=3)
    assert_accept_equal(g, o, "dup greedy")


@pytest.mark.parametrize("V", [8, 3000, 151936])
def test_accept_draft_proposal_chain(V):
    """DRAFT proposal on chains whose tokens were drawn from the drafter."""
    r = np.random.default_rng(V)
    b, K = 16, 6
    N = K + 1
    base = (r.standard_normal((b, K + 1, V)) * 2).astype(np.float32)
    target = base + (0.3 * r.standard_normal((b, N, V))).astype(np.float32)
    draft = base[:, :K] + r.standard_normal((b, K, V)).astype(np.float32)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (b, 1))
    depth = np.tile(np.arange(N, dtype=np.int32), (b, 1))
    token = np.zeros((b, N), np.int32)
    for s in range(b):
        for j in range(K):
            q = np.exp(draft[s, j] - draft[s, j].max())
            token[s, j + 1] = r.choice(V, p=q / q.sum())
    n = np.array([N - (s % 3) for s in range(b)], np.int32)
    g, o = _both(target, parent, token, depth, n, mode=oracle.SAMPLED, draft=draft,
                 proposal=oracle.DRAFT, seed=99, round=1, max_depth=K)
    assert_accept_equal(g, o, "draft")
    # a branching tree is refused per sequence
    parent2 = parent.copy()
    parent2[0, 2] = 0
    g, o = _both(target, parent2, token, depth, n, mode=oracle.SAMPLED, draft=draft,
                 proposal=oracle.DRAFT, seed=99, round=1, max_depth=K)
    assert_accept_equal(g, o, "draft branching")
    assert int(g["accept_len"][0]) == -1


def test_accept_replayable():
    r = np.random.default_rng(4)
    parent, token, depth, n = _random_trees(r, 4, 40, 2000)
    t = dev((r.standard_normal((4, 40, 2000)) * 2).astype(np.float32))
    args = (t, dev(parent), dev(token), dev(depth), dev(n))
    a = tv.tv_tree_accept(*args, mode=tv.TV_SAMPLED, seed=3, round=8, max_depth=40)
    b = tv.tv_tree_accept(*args, mode=tv.TV_SAMPLED, seed=3, round=8, max_depth=40)
    torch.cuda.synchronize()
    for f in a:
        assert torch.equal(a[f], b[f])
