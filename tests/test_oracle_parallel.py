"""The oracle's all-core mode (oracle.set_threads): the builder's draft
positions on OpenMP threads and the attention's (sequence, node) rows on
worker processes give exactly the single-thread results."""
import numpy as np

import workloads


def test_parallel_oracle_matches_serial(orc):
    r = np.random.default_rng(17)
    b, K, V, k, B = 2, 6, 3000, 4, 40
    N = B + 1
    draft = (r.standard_normal((b, K, V)) * 3).astype(np.float32)
    roots = r.integers(0, V, size=b).astype(np.int32)
    ctx = np.array([300, 170], np.int32)
    q = r.standard_normal((b, N, 4, 64)).astype(np.float32)
    kc = r.standard_normal((b, 2, 300 + N, 64)).astype(np.float32)
    vc = r.standard_normal((b, 2, 300 + N, 64)).astype(np.float32)
    prev = orc.set_threads(1)
    try:
        t1 = orc.tree_build(draft, k, B, roots, ctx)
        a1 = orc.tree_attention(q, kc, vc, ctx, t1["anc"], t1["n_nodes"])
        orc.set_threads(3)
        t3 = orc.tree_build(draft, k, B, roots, ctx)
        a3 = orc.tree_attention(q, kc, vc, ctx, t3["anc"], t3["n_nodes"])
    finally:
        orc.set_threads(prev)
    for name in t1:
        assert np.array_equal(t1[name], t3[name]), name
    assert np.array_equal(a1[0], a3[0]) and np.array_equal(a1[1], a3[1])
    assert int(t1["n_nodes"].min()) == N


def test_parallel_candidates_match_serial(orc):
    c = workloads.CONFIGS["4b"]
    draft, _ = workloads.logits(dict(c, name="4b"), 1, 2)
    prev = orc.set_threads(1)
    try:
        one = orc.draft_candidates(draft[0], c["k"])
        orc.set_threads(5)
        many = orc.draft_candidates(draft[0], c["k"])
    finally:
        orc.set_threads(prev)
    for x, y in zip(one, many):
        assert np.array_equal(x, y)
