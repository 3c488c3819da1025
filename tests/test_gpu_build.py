"""GPU parity of tv_tree_build and tv_tree_ancestors with the oracle: bit-exact
tree topology, tokens, depths, positions, score bits and ancestor rows."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import assert_tree_equal, bf16_dev, dev, host

pytestmark = pytest.mark.gpu


def _run(draft32, k, B, roots, ctx, dtype="f32", temp=1.0):
    if dtype == "bf16":
        draft32 = workloads.round_bf16(draft32)
        d = bf16_dev(draft32)
    else:
        d = dev(draft32)
    g = tv.tv_tree_build(d, k, B, dev(roots), dev(ctx), build_temp=temp)
    torch.cuda.synchronize()
    o = oracle.tree_build(draft32, k, B, roots, ctx, build_temp=temp)
    return g, o


CASES = [
    # name, batch, K, V, k, B, sigma, dtype
    ("tiny", 1, 4, 1000, 4, 16, 2.0, "f32"),
    ("tiny-b3", 3, 4, 1000, 4, 16, 2.0, "f32"),
    ("small-bf16", 2, 6, 5000, 8, 64, 3.0, "bf16"),
    ("ragged-V", 1, 5, 8195, 5, 40, 3.0, "f32"),
    ("k1-chain", 1, 9, 300, 1, 20, 2.0, "f32"),
    ("k64", 1, 3, 20000, 64, 200, 3.0, "f32"),
    ("deep", 1, 40, 700, 2, 300, 0.5, "f32"),
    ("peaked", 1, 12, 900, 3, 60, 12.0, "f32"),
    ("budget-512", 1, 30, 500, 2, 512, 0.7, "f32"),
    ("mid-bf16", 2, 8, 4000, 16, 256, 3.0, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_build_random(case):
    name, b, K, V, k, B, sig, dt = case
    r = np.random.default_rng(zlib.crc32(name.encode()))
    draft = (r.standard_normal((b, K, V)) * sig).astype(np.float32)
    roots = r.integers(0, V, size=b).astype(np.int32)
    ctx = r.integers(0, 5000, size=b).astype(np.int32)
    g, o = _run(draft, k, B, roots, ctx, dt)
    for s in range(b):
        assert_tree_equal(g, o, s)


def test_build_ties():
    """Equal logits inside and across positions: the tie orders decide."""
    r = np.random.default_rng(5)
    K, V, k, B = 5, 600, 6, 120
    levels = np.array([0.0, -0.5, -1.0, -3.0], np.float32)
    draft = levels[r.integers(0, 4, size=(2, K, V))]
    draft[1, 2] = 0.0                                  # a whole flat row
    g, o = _run(draft, k, B, np.array([1, 2], np.int32), np.array([10, 20], np.int32))
    for s in range(2):
        assert_tree_equal(g, o, s)


def test_build_signed_zero_ties():
    """+0 and -0 are equal logits: their order falls to the token ids."""
    r = np.random.default_rng(15)
    K, V, k, B = 4, 9000, 8, 60
    draft = np.where(r.random((1, K, V)) < 0.5, np.float32(0.0), np.float32(-0.0))
    draft = draft.astype(np.float32)
    draft[0, :, ::7] = -1.0
    g, o = _run(draft, k, B, np.array([3], np.int32), np.array([5], np.int32))
    assert_tree_equal(g, o, 0)


def test_build_nan_logits_finish():
    """NaN logits are outside the contract (finite, or -inf with a finite
    row maximum), so the tree they give is unspecified; the call must still
    finish, with the node count within the budget and the root in row 0."""
    r = np.random.default_rng(16)
    K, V, k, B = 6, 20000, 8, 64
    draft = (r.standard_normal((2, K, V)) * 3).astype(np.float32)
    draft[0, 1, r.integers(0, V, 40)] = np.nan
    draft[1, :, 5] = np.nan
    g = tv.tv_tree_build(dev(draft), k, B, dev(np.array([1, 2], np.int32)),
                         dev(np.array([10, 20], np.int32)))
    torch.cuda.synchronize()
    parent, depth, nn = host(g["parent"]), host(g["depth"]), host(g["n_nodes"])
    for s in range(2):
        assert 1 <= int(nn[s]) <= B + 1
        assert parent[s, 0] == -1 and depth[s, 0] == 0


def test_build_neg_inf_and_small_tree():
    r = np.random.default_rng(6)
    K, V, k = 3, 50, 3
    draft = r.standard_normal((1, K, V)).astype(np.float32)
    draft[0, 1, 10:] = -np.inf
    for B in (0, 1, 5, 39, 100):       # 3 + 9 + 27 = 39 candidate nodes
        g, o = _run(draft, k, B, np.array([0], np.int32), np.array([7], np.int32))
        assert_tree_equal(g, o, 0)


def test_build_temperature():
    r = np.random.default_rng(7)
    draft = (r.standard_normal((1, 6, 3000)) * 3).astype(np.float32)
    for temp in (0.5, 2.0):
        g, o = _run(draft, 6, 50, np.array([3], np.int32), np.array([0], np.int32), temp=temp)
        assert_tree_equal(g, o, 0)


@pytest.mark.parametrize("cfg", ["4b", "8b", "long"])
def test_build_full_size(cfg):
    c = workloads.CONFIGS[cfg]
    draft, _ = workloads.logits(c, 1, 1)
    roots = workloads.root_tokens(c, 1)
    ctx = workloads.context_lengths(c, 1)
    g, o = _run(draft, c["k"], c["B"], roots, ctx, c["dtype"])
    assert_tree_equal(g, o, 0)


def test_build_repeatable():
    r = np.random.default_rng(8)
    d = dev((r.standard_normal((2, 8, 20000)) * 3).astype(np.float32))
    args = (8, 100, dev(np.array([1, 2], np.int32)), dev(np.array([5, 6], np.int32)))
    a = tv.tv_tree_build(d, *args)
    b = tv.tv_tree_build(d, *args)
    torch.cuda.synchronize()
    for f in a:
        assert torch.equal(a[f], b[f]), f


@pytest.mark.parametrize("N", [1, 33, 130, 1024])
def test_ancestors(N):
    r = np.random.default_rng(N)
    b = 3
    parent = np.full((b, N), -1, np.int32)
    n_nodes = np.array([N, max(1, N // 2), max(1, N - 3)], np.int32)
    for s in range(b):
        for i in range(1, N):
            parent[s, i] = r.integers(max(0, i - 5), i) if s == 2 else r.integers(0, i)
    ctx = np.array([0, 100, 4096], np.int32)
    g = tv.tv_tree_ancestors(dev(parent), dev(n_nodes), dev(ctx))
    torch.cuda.synchronize()
    W = (N + 63) // 64
    for s in range(b):
        n = int(n_nodes[s])
        anc, depth = oracle.ancestors(parent[s, :n], words=W)
        assert np.array_equal(host(g["depth"])[s, :n], depth)
        assert np.all(host(g["depth"])[s, n:] == -1)
        assert np.array_equal(host(g["pos"])[s, :n], ctx[s] + depth)
        ga = host(g["anc"])[s].view(np.uint64)
        assert np.array_equal(ga[:n], anc)
        assert np.all(ga[n:] == 0)


def test_build_workspace_reuse_and_many_rows():
    """One workspace serves consecutive builds of one shape, whatever the
    previous call left in it; 12 sequences x 16 positions of the full
    vocabulary (228 draft rows' chunks per kernel launch)."""
    c = workloads.CONFIGS["4b"]
    b, K, V, k, B = 12, 16, c["V"], 8, 64
    ws = torch.empty(tv.tree_build_workspace(b, K, V, k, B), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    for call in range(3):
        r = np.random.default_rng(100 + call)
        draft = (r.standard_normal((b, K, V)) * 3).astype(np.float32)
        roots = r.integers(0, V, size=b).astype(np.int32)
        ctx = r.integers(0, 5000, size=b).astype(np.int32)
        g = tv.tv_tree_build(dev(draft), k, B, dev(roots), dev(ctx), workspace=ws)
        torch.cuda.synchronize()
        o = oracle.tree_build(draft, k, B, roots, ctx)
        for s_ in range(b):
            assert_tree_equal(g, o, s_)
