"""tv_tree_build_noalloc (the library's static scratch, no workspace) against
tv_tree_build (a caller workspace): identical tree arrays, bit for bit, on two
calls in a row, the second with a smaller input than the first, so that the
scratch holds the first call's leftovers when the second runs."""
import numpy as np
import pytest
import torch

import tree_verification_best_amd as tv
import workloads
from gpu_util import bf16_dev, dev

pytestmark = pytest.mark.gpu

NAMES = ("parent", "token", "depth", "pos", "score", "anc", "n_nodes")


def _inputs(seed, b, K, V, sigma, dtype):
    r = np.random.default_rng(seed)
    draft = (r.standard_normal((b, K, V)) * sigma).astype(np.float32)
    roots = dev(r.integers(0, V, size=b).astype(np.int32))
    ctx = dev(r.integers(0, 8000, size=b).astype(np.int32))
    if dtype == "bf16":
        return bf16_dev(workloads.round_bf16(draft)), roots, ctx
    return dev(draft), roots, ctx


def _compare(d, k, B, roots, ctx, temp):
    want = tv.tv_tree_build(d, k, B, roots, ctx, build_temp=temp)
    got = tv.tv_tree_build_noalloc(d, k, B, roots, ctx, build_temp=temp)
    torch.cuda.synchronize()
    for name in NAMES:
        assert torch.equal(got[name], want[name]), name
    return got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_call(dtype):
    # batched verification shape (16 sequences, K=16, top-4, B=32), then a small tree
    big = _inputs(11, 16, 16, 151936, 3.0, dtype)
    print("noalloc call 1: b=16 K=16 V=151936 k=4 B=32", dtype, flush=True)
    g1 = _compare(*big[:1], 4, 32, *big[1:], 1.0)
    assert int(g1["n_nodes"].min()) == 33
    small = _inputs(12, 1, 4, 1000, 2.0, dtype)
    print("noalloc call 2: b=1 K=4 V=1000 k=4 B=16", dtype, flush=True)
    g2 = _compare(*small[:1], 4, 16, *small[1:], 0.7)
    assert int(g2["n_nodes"][0]) == 17


def test_noalloc_large_budget_then_smaller():
    # 32K-context shape (K=32, top-16, B=512: dynamic LDS beyond 64 KB), then the 4B shape
    a = _inputs(21, 1, 32, 151936, 3.0, "f32")
    print("noalloc call 1: b=1 K=32 V=151936 k=16 B=512", flush=True)
    _compare(*a[:1], 16, 512, *a[1:], 1.0)
    c = workloads.CONFIGS["4b"]
    draft, _ = workloads.logits(c, 1, c["B"] + 1)
    roots = dev(workloads.root_tokens(c, 1))
    ctx = dev(np.array([c["L"]], np.int32))
    print("noalloc call 2: 4B shape K=16 k=8 B=64", flush=True)
    g = _compare(dev(draft), c["k"], c["B"], roots, ctx, 1.0)
    assert int(g["n_nodes"][0]) == c["B"] + 1
