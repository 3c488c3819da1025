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
    # 130 rows x 38 chunks: more blocks than the device holds, so the sampled
    # row pass runs pipelined over bf16 rows
    ("full-vocab-bf16", 2, 65, 151936, 3.0, 12.0, 8, "bf16"),
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


@pytest.mark.parametrize("mode", ["greedy", "sampled"])
def test_accept_wide_star_and_full_rows(mode):
    """A root with 150 children (three groups of wave lanes, tokens repeated
    across groups) and a 1024-row tree (most final draws derived on demand)."""
    r = np.random.default_rng(51)
    V = 700
    # star: root + 150 children, then one grandchild under each of 5 children
    N1 = 156
    parent = np.full((3, N1), 0, np.int32)
    parent[:, 0] = -1
    parent[:, 151:] = np.arange(1, 6)
    depth = np.where(np.arange(N1) == 0, 0, np.where(np.arange(N1) > 150, 2, 1))
    depth = np.tile(depth.astype(np.int32), (3, 1))
    token = r.integers(0, 40, size=(3, N1)).astype(np.int32)  # many repeats
    token[1, 70] = token[1, 3]
    target = (r.standard_normal((3, N1, V)) * 1.2).astype(np.float32)
    target[:, 0, :40] += 3.0  # the children's tokens carry most of the root's mass
    n = np.array([N1, N1, 100], np.int32)
    m = oracle.GREEDY if mode == "greedy" else oracle.SAMPLED
    for rnd in range(4):
        g, o = _both(target, parent, token, depth, n, mode=m, max_depth=3, seed=21, round=rnd)
        assert_accept_equal(g, o, f"star round {rnd}")
    # 1024 rows
    N2 = 1024
    parent, token, depth, n = _random_trees(r, 2, N2, 300, max_children=3, ns=[N2, 777])
    target = (r.standard_normal((2, N2, 300)) * 1.5).astype(np.float32)
    target = workloads.plant(target, parent, token, n, 6.0)
    for rnd in range(3):
        g, o = _both(target, parent, token, depth, n, mode=m, max_depth=int(depth.max()) + 1,
                     seed=8, round=rnd)
        assert_accept_equal(g, o, f"1024 rows round {rnd}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_accept_draft_proposal_edge_tokens(dtype):
    """DRAFT chains with tokens of zero target mass, tokens outside the
    vocabulary, a bad depth on an unvisited and on a visited node, and the
    largest drafter depth (K = 64)."""
    r = np.random.default_rng(61)
    b, K, V = 24, 64, 5000
    N = K + 1
    target = (r.standard_normal((b, N, V)) * 1.0).astype(np.float32)
    draft = (target[:, :K] + 0.2 * r.standard_normal((b, K, V))).astype(np.float32)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (b, 1))
    depth = np.tile(np.arange(N, dtype=np.int32), (b, 1))
    token = np.zeros((b, N), np.int32)
    for s in range(b):
        for j in range(K):
            token[s, j + 1] = int(np.argmax(draft[s, j]))  # likely accepted for a while
    target[0, 0, token[0, 1]] = -np.inf    # p = 0 at the first child
    token[1, 1] = -3                      # outside the vocabulary
    token[2, 1] = V + 7
    token[3, 2] = token[3, 1]
    target[3, 1, token[3, 2]] = -np.inf
    depth[4, 3] = 0                       # bad depth, visited only if 2 levels accept
    depth[5, 1] = K + 5                   # bad depth on the first child
    n = np.array([N - (s % 5) for s in range(b)], np.int32)
    for rnd in range(3):
        g, o = _both(target, parent, token, depth, n, mode=oracle.SAMPLED, dtype=dtype,
                     draft=draft, proposal=oracle.DRAFT, seed=13, round=rnd, max_depth=K)
        assert_accept_equal(g, o, f"draft edges round {rnd}")
    assert int(g["accept_len"][5]) == -1
    assert int(g["accept_len"][1]) == 0 and int(g["accept_len"][2]) == 0


def test_accept_draft_proposal_limits():
    t = torch.zeros((1, 2, 16), device="cuda")
    d = torch.zeros((1, 65, 16), device="cuda")
    i = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    n = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(tv.TreeVerifyError):
        tv.tv_tree_accept(t, i, i, i, n, mode=tv.TV_SAMPLED, max_depth=1,
                          proposal=tv.TV_PROPOSAL_DRAFT, draft_logits=d)


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


@pytest.mark.parametrize("proposal", ["point_mass", "draft"])
def test_accept_sampled_workspace_reuse(proposal):
    """One zero-filled workspace serves consecutive sampled calls of one shape:
    each call leaves the row pass's hand-off words zero for the next (no
    clearing launch).  Every call matches the oracle."""
    r = np.random.default_rng(31)
    V = 151936
    if proposal == "point_mass":
        b, N, K = 2, 65, 16
        prop = tv.TV_PROPOSAL_POINT_MASS
    else:
        b, K = 2, 5
        N = K + 1
        prop = tv.TV_PROPOSAL_DRAFT
    ws = torch.zeros(tv.accept_workspace(b, N, K, V, tv.TV_SAMPLED, prop), dtype=torch.uint8,
                     device="cuda")
    for call in range(4):
        if proposal == "point_mass":
            parent, token, depth, n = _random_trees(r, b, N, V, 8, ns=[N, 30 + call])
            target = workloads.plant((r.standard_normal((b, N, V)) * 3).astype(np.float32),
                                     parent, token, n, 12.0)
            draft, kw = None, dict(max_depth=int(depth.max()) + 1)
        else:
            base = (r.standard_normal((b, N, V)) * 2).astype(np.float32)
            target = base + (0.3 * r.standard_normal((b, N, V))).astype(np.float32)
            draft = base[:, :K] + r.standard_normal((b, K, V)).astype(np.float32)
            parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (b, 1))
            depth = np.tile(np.arange(N, dtype=np.int32), (b, 1))
            token = r.integers(0, V, size=(b, N)).astype(np.int32)
            for s_ in range(b):
                for j in range(K):
                    token[s_, j + 1] = int(np.argmax(draft[s_, j]))
            n = np.full(b, N, np.int32)
            kw = dict(max_depth=K, proposal=oracle.DRAFT)
        g = tv.tv_tree_accept(dev(target), dev(parent), dev(token), dev(depth), dev(n),
                              mode=tv.TV_SAMPLED, draft_logits=dev(draft) if draft is not None
                              else None, temperature=1.0, seed=99, round=call, workspace=ws,
                              **kw)
        torch.cuda.synchronize()
        o = oracle.tree_accept(target, parent, token, depth, n, mode=oracle.SAMPLED,
                               draft=draft, temperature=1.0, seed=99, round=call, **kw)
        assert_accept_equal(g, o, f"{proposal} call {call}")


@pytest.mark.parametrize("proposal", ["point_mass", "draft"])
def test_accept_row_pass_fallback(proposal):
    """The sampled row pass with its wait bound at 0 polls: nearly every block
    finds its row's maximum by reading the whole row itself.  The results are
    those of the oracle (and of the default bound)."""
    r = np.random.default_rng(11)
    V = 151936
    if proposal == "point_mass":
        b, N = 2, 65
        parent, token, depth, n = _random_trees(r, b, N, V, 8, ns=[N, 40])
        target = workloads.plant((r.standard_normal((b, N, V)) * 3).astype(np.float32),
                                 parent, token, n, 12.0)
        draft, kw = None, dict(max_depth=int(depth.max()) + 1)
    else:
        b, K = 3, 6
        N = K + 1
        base = (r.standard_normal((b, N, V)) * 2).astype(np.float32)
        target = base + (0.3 * r.standard_normal((b, N, V))).astype(np.float32)
        draft = base[:, :K] + r.standard_normal((b, K, V)).astype(np.float32)
        parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (b, 1))
        depth = np.tile(np.arange(N, dtype=np.int32), (b, 1))
        token = r.integers(0, V, size=(b, N)).astype(np.int32)
        for s in range(b):
            for j in range(K):
                token[s, j + 1] = int(np.argmax(draft[s, j]))
        n = np.full(b, N, np.int32)
        kw = dict(max_depth=K, proposal=oracle.DRAFT)
    old = tv.lib().tv_debug_set_spin_limit(0)
    try:
        for T, rnd in ((1.0, 1), (0.8, 2)):
            g, o = _both(target, parent, token, depth, n, mode=oracle.SAMPLED, draft=draft,
                         temperature=T, seed=4321, round=rnd, **kw)
            assert_accept_equal(g, o, f"{proposal} fallback T={T}")
    finally:
        tv.lib().tv_debug_set_spin_limit(old)


def test_accept_concurrent_streams():
    """Sampled walks of the full-vocabulary shape on four streams at once, each
    with its own workspace: together their row-pass grids exceed what the
    device holds at once, so blocks may wait in vain and take the fallback.
    Every stream's result is the oracle's."""
    r = np.random.default_rng(12)
    b, N, V = 1, 65, 151936
    parent, token, depth, n = _random_trees(r, b, N, V, 8)
    target = workloads.plant((r.standard_normal((b, N, V)) * 3).astype(np.float32),
                             parent, token, n, 12.0)
    args = (dev(target), dev(parent), dev(token), dev(depth), dev(n))
    kw = dict(mode=tv.TV_SAMPLED, seed=77, max_depth=int(depth.max()) + 1)
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    import time
    t0 = time.perf_counter()
    outs = []
    for i, st in enumerate(streams):
        with torch.cuda.stream(st):
            outs.append(tv.tv_tree_accept(*args, round=i, **kw))
    torch.cuda.synchronize()
    print(f"four concurrent sampled calls: {1e3 * (time.perf_counter() - t0):.2f} ms", flush=True)
    for i, g in enumerate(outs):
        o = oracle.tree_accept(target, parent, token, depth, n, mode=oracle.SAMPLED,
                               seed=77, round=i, max_depth=kw["max_depth"])
        assert_accept_equal(g, o, f"stream {i}")
