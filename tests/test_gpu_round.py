"""One whole verification round on the GPU (build -> attention -> accept) on
the tiny workload and the 4B-class workload, each step against the oracle on
the same seeded inputs; plus the statistical law of the GPU's sampled walk."""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import (assert_accept_equal, assert_attention_close, assert_tree_equal, bf16_dev,
                      dev)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", ["tiny", "4b"])
def test_round(cfg):
    c = workloads.CONFIGS[cfg]
    b, N = c["batch"], c["B"] + 1
    draft, target = workloads.logits(c, b, N)
    roots = workloads.root_tokens(c, b)
    ctx = workloads.context_lengths(c, b)
    cap = int(ctx.max()) + N
    q, k, v = workloads.qkv(c, b, N, cap)
    bf = c["dtype"] == "bf16"
    put = bf16_dev if bf else dev
    if bf:
        draft, target = workloads.round_bf16(draft), workloads.round_bf16(target)
    # build
    tree = tv.tv_tree_build(put(draft), c["k"], c["B"], dev(roots), dev(ctx))
    torch.cuda.synchronize()
    otree = oracle.tree_build(draft, c["k"], c["B"], roots, ctx)
    for s in range(b):
        assert_tree_equal(tree, otree, s)
    # attention over the GPU's tree
    out, lse = tv.tv_tree_attention_verify(put(q), put(k), put(v), dev(ctx), tree["anc"],
                                           tree["n_nodes"], int(ctx.max()))
    torch.cuda.synchronize()
    if cfg == "tiny":
        ro, rl = oracle.tree_attention(q, k, v, ctx, otree["anc"], otree["n_nodes"])
        assert_attention_close(out, lse, ro, rl, otree["n_nodes"], cfg)
    else:
        rows = [(0, i) for i in (0, 1, 7, 32, 64)]
        ref = oracle.tree_attention_rows(q, k, v, ctx, otree["anc"], otree["n_nodes"], rows)
        g = out.float().cpu().numpy()
        gl = lse.cpu().numpy()
        for (s, i), (ro, rl) in ref.items():
            d = g[s, i] - ro
            assert np.abs(d).max() <= 1e-2, i
            assert np.linalg.norm(d) / np.linalg.norm(ro) <= 2e-2, i
            assert np.abs(gl[s, i] - rl).max() <= 1e-2, i
    # accept, every temperature of the workload
    for T in c["temperatures"]:
        mode = oracle.GREEDY if T == 0 else oracle.SAMPLED
        g = tv.tv_tree_accept(put(target), tree["parent"], tree["token"], tree["depth"],
                              tree["n_nodes"], mode=mode, temperature=max(T, 1e-3), seed=1234,
                              round=0, max_depth=c["K"])
        torch.cuda.synchronize()
        o = oracle.tree_accept(target, otree["parent"], otree["token"], otree["depth"],
                               otree["n_nodes"], mode=mode, temperature=max(T, 1e-3), seed=1234,
                               round=0, max_depth=c["K"])
        assert_accept_equal(g, o, f"{cfg} T={T}")


def test_gpu_sampled_walk_preserves_target():
    """Chi-square of the GPU's first emitted token against p at the root over
    10^6 walks on one tree of deterministic candidates (POINT_MASS)."""
    r = np.random.default_rng(12)
    V, n = 8, 6
    parent = np.array([-1, 0, 0, 0, 1, 1], np.int32)
    token = np.array([0, 2, 5, 7, 1, 2], np.int32)
    depth = np.array([0, 1, 1, 1, 2, 2], np.int32)
    target = (r.standard_normal((n, V)) * 1.5).astype(np.float32)
    p = np.exp(target[0].astype(np.float64) - target[0].max())
    p /= p.sum()
    per_call = 8000   # rows = 6 * 8000 < 65535
    tgt = dev(np.broadcast_to(target, (per_call, n, V)).copy())
    args = [dev(np.broadcast_to(a, (per_call, n)).copy()) for a in (parent, token, depth)]
    nn = dev(np.full(per_call, n, np.int32))
    counts = np.zeros(V)
    acc = 0
    calls = 125
    for rnd in range(calls):
        res = tv.tv_tree_accept(tgt, *args, nn, mode=tv.TV_SAMPLED, seed=42, round=rnd,
                                max_depth=3)
        first = res["out_tokens"][:, 0].cpu().numpy()
        counts += np.bincount(first, minlength=V)
        acc += int((res["accept_len"] >= 1).sum().item())
    total = per_call * calls
    assert stats.chisquare(counts, p * total).pvalue > 1e-3
    closed = p[[2, 5, 7]].sum()
    assert abs(acc / total - closed) < 5 * np.sqrt(closed * (1 - closed) / total)
