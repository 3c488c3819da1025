"""Pins of the cost-aware tree size (oracle/budget.py).

The objective's numerator is pinned by what it claims: when the target's
next-token distribution after every node equals the drafter's marginal at
that depth (the edge scores are then the true acceptance probabilities), the
mean number of tokens a sampled round emits is 1 + sum of the tree's path
scores.  The choice itself is checked by brute force over all sizes and
against a cost that makes one size optimal in closed form."""
import numpy as np
import pytest

import oracle


def _tree_and_target(seed, K=4, k=3, B=10, V=12):
    r = np.random.default_rng(seed)
    draft = (r.standard_normal((1, K, V)) * 1.2).astype(np.float32)
    t = oracle.tree_build(draft, k, B, np.array([0], np.int32), np.array([0], np.int32))
    n = int(t["n_nodes"][0])
    # node u's target row = the drafter's marginal at depth(u) + 1
    target = np.zeros((1, n, V), np.float32)
    for u in range(n):
        d = int(t["depth"][0, u])
        target[0, u] = draft[0, d] if d < K else draft[0, K - 1]
    return t, target, n, K


@pytest.mark.parametrize("seed", [1, 2])
def test_expected_emitted_tokens_is_one_plus_score_sum(seed):
    t, target, n, K = _tree_and_target(seed)
    trials = 40000
    b = 400
    total = 0.0
    sq = 0.0
    for rnd in range(trials // b):
        res = oracle.tree_accept(np.broadcast_to(target, (b,) + target.shape[1:]),
                                 np.broadcast_to(t["parent"][:, :n], (b, n)),
                                 np.broadcast_to(t["token"][:, :n], (b, n)),
                                 np.broadcast_to(t["depth"][:, :n], (b, n)),
                                 np.full(b, n, np.int32), mode=oracle.SAMPLED, seed=seed,
                                 round=rnd, max_depth=K)
        e = res["accept_len"].astype(np.float64) + 1.0
        total += e.sum()
        sq += (e * e).sum()
    mean = total / trials
    sd = np.sqrt(max(sq / trials - mean * mean, 1e-12) / trials)
    expect = 1.0 + t["score"][0, 1:n].sum()
    assert abs(mean - expect) < 5 * sd + 1e-9, (mean, expect, sd)


def test_choice_brute_force_and_closed_form():
    r = np.random.default_rng(3)
    b, N = 6, 40
    score = np.zeros((b, N))
    score[:, 0] = 1.0
    score[:, 1:] = -np.sort(-r.uniform(0.01, 1.0, size=(b, N - 1)), axis=1)
    n_nodes = np.array([40, 1, 2, 17, 40, 33], np.int32)
    cost = 1.0 + 0.05 * np.arange(N) + 0.002 * np.arange(N) ** 2
    got = oracle.tree_budget(score, n_nodes, cost)
    for s in range(b):
        n = int(n_nodes[s])
        ratios = [(1.0 + score[s, 1:m + 1].sum()) / cost[m] for m in range(n)]
        best = int(np.argmax(ratios))
        assert got[s] == best + 1
    # a flat cost keeps every node; a cost that jumps after m nodes keeps m
    assert list(oracle.tree_budget(score, n_nodes, np.ones(N))) == list(n_nodes)
    step = np.where(np.arange(N) <= 5, 1.0, 100.0)
    assert list(oracle.tree_budget(score, np.full(b, N), step)) == [6] * b
