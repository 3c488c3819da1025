"""GPU parity of tv_kv_commit with the oracle: the caches after the commit
and the new context lengths are bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import bf16_dev, dev, host

pytestmark = pytest.mark.gpu


def _paths(r, b, width, cap, ctx):
    """Accepted paths of random trees, plus the special cases."""
    alen = np.zeros(b, np.int32)
    acc = np.full((b, width), -1, np.int32)
    for s in range(b):
        room = cap - int(ctx[s])
        a = int(r.integers(0, min(width, room)))
        nodes = np.sort(r.choice(np.arange(1, room), size=a, replace=False)) if a else []
        acc[s, 0] = 0
        acc[s, 1:a + 1] = nodes
        alen[s] = a
    alen[0] = 0                              # the root alone
    alen[1] = -1                             # a refused tree
    if b > 5:
        alen[4] = width                      # one past the width
        alen[5] = 2**31 - 1                  # any value: no overflow
    if b > 3:
        acc[2, 1:3] = [5, 5]                 # not strictly increasing
        alen[2] = max(alen[2], 2)
        acc[3, alen[3]] = cap                # past the cache
        alen[3] = max(alen[3], 1)
        acc[3, alen[3]] = cap - int(ctx[3])
    return alen, acc


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_commit_matches_oracle(dtype, D):
    r = np.random.default_rng(D + (1 if dtype == "bf16" else 0))
    b, Hkv, cap, width = 7, 3, 160, 40
    ctx = r.integers(0, 100, size=b).astype(np.int32)
    ctx[6] = -4                              # a negative context length
    k = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    v = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    if dtype == "bf16":
        k, v = workloads.round_bf16(k), workloads.round_bf16(v)
        kg, vg = bf16_dev(k), bf16_dev(v)
    else:
        kg, vg = dev(k), dev(v)
    alen, acc = _paths(r, b, width, cap, ctx)
    ko, vo, no = oracle.kv_commit(k, v, ctx, alen, acc)
    new = tv.tv_kv_commit(kg, vg, dev(ctx), dev(alen), dev(acc))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(new), no)
    assert np.array_equal(host(kg), ko) and np.array_equal(host(vg), vo)


def test_commit_after_a_round_in_place():
    """A full-size round (4B layer shape): build, accept, then commit with
    the context lengths updated in place."""
    cfg = workloads.CONFIGS["4b"]
    r = np.random.default_rng(5)
    b, Hkv, D, K, B = 2, cfg["Hkv"], cfg["D"], cfg["K"], cfg["B"]
    N = B + 1
    ctx = np.array([4096, 1000], np.int32)
    cap = 4096 + N
    draft, target = workloads.logits(cfg, b, N)
    tree = tv.tv_tree_build(dev(draft), cfg["k"], B, dev(np.zeros(b, np.int32)), dev(ctx))
    par, tok, nn = host(tree["parent"]), host(tree["token"]), host(tree["n_nodes"])
    target = workloads.plant(target, par, tok, nn, 12.0)
    acc = tv.tv_tree_accept(dev(target), tree["parent"], tree["token"], tree["depth"],
                            tree["n_nodes"], mode=tv.TV_SAMPLED, seed=3, round=1, max_depth=K)
    k = workloads.round_bf16(r.standard_normal((b, Hkv, cap, D)).astype(np.float32))
    v = workloads.round_bf16(r.standard_normal((b, Hkv, cap, D)).astype(np.float32))
    kg, vg = bf16_dev(k), bf16_dev(v)
    alen, nodes = host(acc["accept_len"]), host(acc["accepted_nodes"])
    assert alen.max() >= 2  # the planted target accepts a path
    ko, vo, no = oracle.kv_commit(k, v, ctx, alen, nodes)
    ctx_g = dev(ctx)
    tv.tv_kv_commit(kg, vg, ctx_g, acc["accept_len"], acc["accepted_nodes"], new_ctx_len=ctx_g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ctx_g), no)
    assert np.array_equal(host(kg), ko) and np.array_equal(host(vg), vo)
