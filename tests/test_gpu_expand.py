"""GPU parity of tv_tree_root / tv_tree_expand with the oracle (bit-exact:
rows, tokens, depths, positions, fp64 score bits, ancestor rows, node counts
and the next frontier)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import assert_tree_equal, bf16_dev, dev, host

pytestmark = pytest.mark.gpu

def _check(g, o, nxt_g, nxt_o, label):
    torch.cuda.synchronize()
    for s in range(o["parent"].shape[0]):
        try:
            assert_tree_equal(g, o, s)
        except AssertionError as e:
            raise AssertionError(f"{label} seq {s}: {e}") from None
    np.testing.assert_array_equal(host(nxt_g), nxt_o, err_msg=label)


def test_root_matches_oracle():
    b = 5
    for N in (1, 64, 65, 1024):
        root = np.arange(b, dtype=np.int32) * 7
        ctx = np.array([0, 3, 100, 4096, 77], np.int32)
        g = tv.tv_tree_root(dev(root), dev(ctx), N)
        o = oracle.tree_root(b, N, root, ctx)
        torch.cuda.synchronize()
        for s in range(b):
            assert_tree_equal(g, o, s)


@pytest.mark.parametrize("W,m,N,V,bf16", [
    (1, 1, 12, 50, False),        # greedy chain
    (3, 2, 30, 60, False),
    (4, 3, 65, 9000, True),       # two vocabulary chunks, anc rows of two words
    (8, 8, 257, 20000, True),     # capacity reached mid-step
    (64, 1, 130, 300, False),     # the widest frontier
    (2, 64, 200, 70, False),      # the largest m
])
def test_expand_steps_match_oracle(W, m, N, V, bf16):
    r = np.random.default_rng(W * 1000 + m * 10 + N)
    b = 4
    ctx = np.array([5, 0, 11, 4096], np.int32)[:b]
    root = r.integers(0, V, size=b).astype(np.int32)
    o = oracle.tree_root(b, N, root, ctx)
    g = tv.tv_tree_root(dev(root), dev(ctx), N)
    f_o = np.full((b, W), -1, np.int32)
    f_o[:, 0] = 0
    f_g = dev(f_o)
    for step in range(7):
        logits = (r.standard_normal((b, W, V)) * 2.5).astype(np.float32)
        if bf16:
            logits = workloads.round_bf16(logits)
        if step == 2:
            logits[1, :, : V // 2] = -np.inf       # -inf logits with a finite maximum
            logits[2, 0, :] = 0.0                   # a flat row: ties broken by id
        x = bf16_dev(logits) if bf16 else dev(logits)
        o, nxt_o = oracle.tree_expand(logits, m, f_o, o, ctx)
        nxt_g = tv.tv_tree_expand(x, m, f_g, g, dev(ctx))
        _check(g, o, nxt_g, nxt_o, f"step {step}")
        f_o, f_g = nxt_o, nxt_g


def test_expand_odd_frontiers_in_place():
    """Empty, out-of-range and repeated frontier slots; a sequence that is not
    a tree (n_nodes 0 / N+1) is left alone; next_frontier aliases frontier."""
    r = np.random.default_rng(7)
    b, W, m, N, V = 6, 5, 3, 40, 500
    ctx = np.arange(b, dtype=np.int32) * 10
    root = np.arange(b, dtype=np.int32)
    o = oracle.tree_root(b, N, root, ctx)
    g = tv.tv_tree_root(dev(root), dev(ctx), N)
    f_o = np.full((b, W), -1, np.int32)
    f_o[:, 0] = 0
    logits = (r.standard_normal((b, W, V)) * 2).astype(np.float32)
    o, f_o = oracle.tree_expand(logits, m, f_o, o, ctx)
    f_g = dev(np.where(np.arange(W) == 0, 0, -1).astype(np.int32)[None].repeat(b, 0))
    tv.tv_tree_expand(dev(logits), m, f_g, g, dev(ctx), next_frontier=f_g)
    _check(g, o, f_g, f_o, "first step")
    front = f_o.copy()
    front[0] = [1, -1, 2, 1, 99]          # a repeat, an empty slot, a row past n_nodes
    front[1] = [-1, -1, -1, -1, -1]       # nothing to expand
    front[2] = [-5, 3, 0, 2, 1]           # a negative row; the root again
    nn = o["n_nodes"].copy()
    nn[3], nn[4] = 0, N + 1               # not trees
    o["n_nodes"] = nn
    g["n_nodes"] = dev(nn)
    logits = (r.standard_normal((b, W, V)) * 2).astype(np.float32)
    o2, nxt_o = oracle.tree_expand(logits, m, front, o, ctx)
    fg = dev(front)
    tv.tv_tree_expand(dev(logits), m, fg, g, dev(ctx), next_frontier=fg)
    _check(g, o2, fg, nxt_o, "second step")


def test_expand_full_vocabulary_layerwise_build():
    """A layer-wise build at the 8B drafting shape: V = 151936 bf16 logits,
    W = 8, m = 8, capacity 257 (budget 256), drafting until full."""
    cfg = workloads.CONFIGS["8b"]
    N, W, m, b = cfg["B"] + 1, 8, 8, 2
    ctx = workloads.context_lengths(cfg, b)
    root = workloads.root_tokens(cfg, b)
    o = oracle.tree_root(b, N, root, ctx)
    g = tv.tv_tree_root(dev(root), dev(ctx), N)
    f_o = np.full((b, W), -1, np.int32)
    f_o[:, 0] = 0
    f_g = dev(f_o)
    for step, logits in enumerate(workloads.expand_logits(cfg, b, W, 6)):
        o, f_o = oracle.tree_expand(logits, m, f_o, o, ctx)
        f_g = tv.tv_tree_expand(bf16_dev(logits), m, f_g, g, dev(ctx))
        _check(g, o, f_g, f_o, f"step {step}")
    assert (o["n_nodes"] == N).all()
