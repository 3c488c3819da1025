"""GPU parity of tv_tree_check with oracle.tree_check (bit-exact codes)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
from gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [1, 33, 300, 1024])
def test_check_matches_oracle(N):
    r = np.random.default_rng(N)
    b = 24
    parent = np.full((b, N), -1, np.int32)
    depth = np.zeros((b, N), np.int32)
    for s in range(b):
        for i in range(1, N):
            parent[s, i] = int(r.integers(max(0, i - 8), i))
            depth[s, i] = depth[s, parent[s, i]] + 1
    n = r.integers(1, N + 1, size=b).astype(np.int32)
    n[0] = N
    n[1] = 0 if N > 1 else 2          # out of range
    for s in range(2, b):             # faults at random rows, some past n_nodes
        if s % 3 == 0 or N == 1:
            continue
        i = int(r.integers(0, N))
        if s % 3 == 1:
            parent[s, i] = i if i > 0 else 3
        else:
            depth[s, i] += 2
    for with_depth in (False, True):
        want = oracle.tree_check(parent, n, depth if with_depth else None)
        got = tv.tv_tree_check(dev(parent), dev(n), dev(depth) if with_depth else None)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(got), want)
