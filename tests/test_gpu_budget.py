"""GPU parity of tv_tree_budget with the oracle (bit-exact node counts)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [2, 65, 257, 1024])
def test_budget_matches_oracle(N):
    r = np.random.default_rng(N)
    b = 9
    score = np.zeros((b, N))
    score[:, 0] = 1.0
    score[:, 1:] = -np.sort(-r.uniform(1e-4, 1.0, size=(b, N - 1)) ** 3, axis=1)
    score[1, 1:] = 0.25  # equal scores: ties between ratios
    n_nodes = r.integers(1, N + 1, size=b).astype(np.int32)
    n_nodes[0] = N
    n_nodes[2] = 1
    if b > 4:
        n_nodes[3] = 0        # outside [1, N]: copied unchanged
        n_nodes[4] = N + 1
    cost = 1.0 + 0.02 * np.arange(N) + 1e-4 * np.arange(N) ** 2
    cost[N // 2:] += 0.5      # a step in the measured cost
    want = oracle.tree_budget(score, np.clip(n_nodes, 1, N), cost)
    want[3], want[4] = n_nodes[3], n_nodes[4]
    got = host(tv.tv_tree_budget(dev(score), dev(n_nodes), dev(cost)))
    np.testing.assert_array_equal(got, want)
    # flat cost: every node is kept; in place
    nn = dev(np.clip(n_nodes, 1, N))
    tv.tv_tree_budget(dev(score), nn, dev(np.ones(N)), n_nodes_out=nn)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(nn), np.clip(n_nodes, 1, N))


def test_budget_on_built_trees():
    cfg = workloads.CONFIGS["8b"]
    b, B = 3, cfg["B"]
    draft, _ = workloads.logits(cfg, b, 2)
    tree = tv.tv_tree_build(dev(draft), cfg["k"], B, dev(np.zeros(b, np.int32)),
                            dev(np.full(b, 100, np.int32)))
    N = B + 1
    cost = 30.0 + 0.19 * np.arange(N)  # affine: a fixed cost plus a per-node cost
    got = host(tv.tv_tree_budget(tree["score"], tree["n_nodes"], dev(cost)))
    want = oracle.tree_budget(host(tree["score"]), host(tree["n_nodes"]), cost)
    np.testing.assert_array_equal(got, want)
    assert (got >= 1).all() and (got <= host(tree["n_nodes"])).all()
