"""One verification round at the full sizes of the 8B, long-context and batched
workloads, on the inputs and in the launch configuration bench.py uses: the
tree (built, or a random tree through tv_tree_ancestors) and the accept walk
bit-exact against the oracle for every sequence; attention checked on sampled
(sequence, node) rows against the oracle's row-by-row fp64 attention."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import ATOL, RTOL_NORM, assert_accept_equal, assert_tree_equal, bf16_dev, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", ["8b", "long", "batched"])
def test_round_full_size(cfg):
    c = workloads.CONFIGS[cfg]
    b, N, K = c["batch"], c["B"] + 1, c["K"]
    draft, target = workloads.logits(c, b, N)
    roots = workloads.root_tokens(c, b)
    ctx = workloads.context_lengths(c, b)
    cap = int(ctx.max()) + N
    print(f"{cfg}: b={b} N={N} ctx={ctx.min()}..{ctx.max()}", flush=True)
    if c["build"]:
        tree = tv.tv_tree_build(dev(draft), c["k"], c["B"], dev(roots), dev(ctx))
        torch.cuda.synchronize()
        otree = oracle.tree_build(draft, c["k"], c["B"], roots, ctx)
        for s in range(b):
            assert_tree_equal(tree, otree, s)
        parent, token, depth, nn = (otree["parent"], otree["token"], otree["depth"],
                                    otree["n_nodes"])
        anc = otree["anc"]
    else:
        parent, token, _ = workloads.random_trees(c, b, N, max_depth=K,
                                                  max_children=c.get("max_children", 4))
        nn = np.full(b, N, np.int32)
        target = workloads.plant(target, parent, token, nn, 9.0)
        g = tv.tv_tree_ancestors(dev(parent), dev(nn), dev(ctx))
        torch.cuda.synchronize()
        W = (N + 63) // 64
        anc = np.zeros((b, N, W), np.uint64)
        depth = np.zeros((b, N), np.int32)
        for s in range(b):
            anc[s], depth[s] = oracle.ancestors(parent[s], words=W)
        np.testing.assert_array_equal(host(g["anc"]).view(np.uint64), anc)
        np.testing.assert_array_equal(host(g["depth"]), depth)
        np.testing.assert_array_equal(host(g["pos"]), ctx[:, None] + depth)
        tree = dict(parent=dev(parent), token=dev(token), depth=g["depth"], anc=g["anc"],
                    n_nodes=dev(nn))
    # attention in the automatic split configuration, sampled rows
    q, k, v = workloads.qkv(c, b, N, cap)
    out, lse = tv.tv_tree_attention_verify(bf16_dev(q), bf16_dev(k), bf16_dev(v), dev(ctx),
                                           tree["anc"], tree["n_nodes"], int(ctx.max()))
    torch.cuda.synchronize()
    go, gl = host(out), host(lse)
    rows = []
    for s in sorted({0, b // 2, b - 1}):
        n = int(nn[s])
        rows += [(s, i) for i in sorted({0, 1, n // 2, n - 1})]
    ref = oracle.tree_attention_rows(q, k, v, ctx, anc, nn, rows)
    for (s, i), (ro, rl) in ref.items():
        d = go[s, i] - ro
        assert np.abs(d).max() <= ATOL, (s, i)
        assert np.linalg.norm(d) / np.linalg.norm(ro) <= RTOL_NORM, (s, i)
        assert np.abs(gl[s, i] - rl).max() <= 1e-2, (s, i)
    # the walk at every temperature of the workload
    for T in c["temperatures"]:
        mode = oracle.GREEDY if T == 0 else oracle.SAMPLED
        kw = dict(temperature=max(T, 1e-3), seed=1234, round=3, max_depth=K)
        g = tv.tv_tree_accept(dev(target), tree["parent"], tree["token"], tree["depth"],
                              tree["n_nodes"], mode=mode, **kw)
        torch.cuda.synchronize()
        o = oracle.tree_accept(target, parent, token, depth, nn, mode=mode, **kw)
        assert_accept_equal(g, o, f"{cfg} T={T}")
