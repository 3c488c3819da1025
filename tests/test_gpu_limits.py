"""Parity at the limits the C ABI accepts: budget 1023 (1024 rows), and
K * topk = 4096 with the largest budget that fits, at vocabulary 2^18; a
1023-deep accepted path and a commit of 1024 rows; the widest layer-wise
step (W * m = 4096)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import (assert_accept_equal, assert_tree_equal, bf16_dev, dev, host, ATOL,
                      RTOL_NORM)

pytestmark = pytest.mark.gpu

VMAX = 1 << 18


@pytest.mark.parametrize("K,k,B", [(64, 16, 1023), (64, 64, 869)])
def test_build_at_the_limits(K, k, B):
    """The largest budgets whose selection lists fit the workgroup's LDS
    (beyond 64 KB), at the largest vocabulary."""
    r = np.random.default_rng(1)
    b = 1
    # a peaked base row shared by the positions keeps the candidate tree deep
    base = r.standard_normal(VMAX).astype(np.float32) * 3
    draft = (base + r.standard_normal((b, K, VMAX)).astype(np.float32) * 0.5).astype(np.float32)
    roots = np.array([7], np.int32)
    ctx = np.array([100], np.int32)
    g = tv.tv_tree_build(dev(draft), k, B, dev(roots), dev(ctx))
    torch.cuda.synchronize()
    o = oracle.tree_build(draft, k, B, roots, ctx)
    assert int(o["n_nodes"][0]) == B + 1
    assert_tree_equal(g, o, 0)


def test_attention_1024_rows():
    r = np.random.default_rng(2)
    c = workloads.CONFIGS["4b"]
    b, N, Hq, Hkv, D, L = 1, 1024, 32, 8, 128, 1500
    cap = L + N
    q, k, v = workloads.qkv(c, b, N, cap, salt=4)
    parent = np.concatenate([[-1], r.integers(np.maximum(0, np.arange(1, N) - 40),
                                              np.arange(1, N))]).astype(np.int32)
    anc = oracle.ancestors(parent)[0][None]
    ctx = np.array([L], np.int32)
    nn = np.array([N], np.int32)
    out, lse = tv.tv_tree_attention_verify(bf16_dev(q), bf16_dev(k), bf16_dev(v), dev(ctx),
                                           dev(anc.view(np.int64)), dev(nn), L)
    torch.cuda.synchronize()
    go, gl = host(out), host(lse)
    rows = [(0, i) for i in (0, 1, 511, 640, 1022, 1023)]
    for (s, i), (ro, rl) in oracle.tree_attention_rows(q, k, v, ctx, anc, nn, rows).items():
        d = go[s, i] - ro
        assert np.abs(d).max() <= ATOL and np.linalg.norm(d) / np.linalg.norm(ro) <= RTOL_NORM
        assert np.abs(gl[s, i] - rl).max() <= 1e-2


def test_deepest_walk_and_commit():
    """A 1024-node chain whose target prefers every next token: the walk
    accepts all 1023 drafts (max_depth 1023) over a 2^18 vocabulary, greedy
    and sampled; the commit then moves 1024 rows (width 1024)."""
    r = np.random.default_rng(3)
    N = 1024
    parent = np.arange(-1, N - 1, dtype=np.int32)[None]
    depth = np.arange(N, dtype=np.int32)[None]
    token = r.integers(0, VMAX, size=(1, N)).astype(np.int32)
    n = np.array([N], np.int32)
    target = np.empty((1, N, VMAX), np.float32)
    for i in range(N):
        target[0, i] = r.standard_normal(VMAX).astype(np.float32)
    target = workloads.plant(target, parent, token, n, 40.0)
    tg = dev(target)
    for mode, T in ((oracle.GREEDY, 1.0), (oracle.SAMPLED, 1.0)):
        kw = dict(temperature=T, seed=5, round=1, max_depth=N - 1)
        g = tv.tv_tree_accept(tg, dev(parent), dev(token), dev(depth), dev(n), mode=mode, **kw)
        torch.cuda.synchronize()
        o = oracle.tree_accept(target, parent, token, depth, n, mode=mode, **kw)
        assert_accept_equal(g, o, f"mode {mode}")
        assert int(o["accept_len"][0]) == N - 1
    del tg, target
    # commit the whole chain: rows L .. L + 1023 are already in place, so
    # move a sparse 1024-row path of a wider tree instead
    Hkv, D, L = 2, 64, 30
    cap = L + 2 * N
    kc = r.standard_normal((1, Hkv, cap, D)).astype(np.float32)
    vc = r.standard_normal((1, Hkv, cap, D)).astype(np.float32)
    path = np.concatenate([[0], np.sort(r.choice(np.arange(1, 2 * N), size=N - 1,
                                                 replace=False))]).astype(np.int32)[None]
    alen = np.array([N - 1], np.int32)
    ko, vo, no = oracle.kv_commit(kc, vc, np.array([L]), alen, path)
    kg, vg = dev(kc), dev(vc)
    new = tv.tv_kv_commit(kg, vg, dev(np.array([L], np.int32)), dev(alen), dev(path))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(new), no)
    assert np.array_equal(host(kg), ko) and np.array_equal(host(vg), vo)


def test_widest_expansion_step():
    r = np.random.default_rng(4)
    b, W, m, N, V = 2, 64, 64, 1024, 3000
    ctx = np.array([9, 0], np.int32)
    roots = np.array([1, 2], np.int32)
    o = oracle.tree_root(b, N, roots, ctx)
    g = tv.tv_tree_root(dev(roots), dev(ctx), N)
    f_o = np.full((b, W), -1, np.int32)
    f_o[:, 0] = 0
    f_g = dev(f_o)
    for step in range(3):  # 1 + 64 + 4096 children: the third step fills the tree
        logits = (r.standard_normal((b, W, V)) * 2).astype(np.float32)
        o, f_o = oracle.tree_expand(logits, m, f_o, o, ctx)
        f_g = tv.tv_tree_expand(dev(logits), m, f_g, g, dev(ctx))
        torch.cuda.synchronize()
        for s in range(b):
            assert_tree_equal(g, o, s)
        np.testing.assert_array_equal(host(f_g), f_o)
    assert (o["n_nodes"] == N).all()
