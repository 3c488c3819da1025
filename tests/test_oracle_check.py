"""Pins of the structural tree check (oracle.tree_check).

Against the C ancestor routine, which refuses malformed parent arrays below
the root on its own terms (an independent implementation), and against
hand-made violations, the root's rules included."""
import numpy as np

import oracle
import workloads


def test_check_agrees_with_ancestor_routine():
    r = np.random.default_rng(1)
    N = 20
    for trial in range(300):
        parent = np.array([-1] + [int(r.integers(0, i)) for i in range(1, N)], np.int32)
        if trial % 2:  # plant a fault below the root: a self, forward, negative or
            # early parent (the C routine takes row 0 as the root whatever its
            # parent and a later -1 as a second root, so neither is planted)
            i = int(r.integers(1, N))
            parent[i] = int(r.choice([i, min(N - 1, i + 1 + int(r.integers(0, 3))), -3, 5]))
        code = oracle.tree_check(parent[None], np.array([N]))[0]
        try:
            oracle.ancestors(parent)
            refused = False
        except ValueError:
            refused = True
        assert (code != 0) == refused, (parent, code)


def test_check_codes():
    c = workloads.CONFIGS["batched"]
    parent, _, depth = workloads.random_trees(c, 3, 33, max_depth=16, max_children=4)
    n = np.full(3, 33, np.int32)
    np.testing.assert_array_equal(oracle.tree_check(parent, n, depth), [0, 0, 0])
    p2, d2 = parent.copy(), depth.copy()
    p2[0, 7] = 9            # a parent after the node
    d2[1, 12] += 1          # a depth that does not follow the parent's
    p2[2, 0] = 0            # the root with a parent
    np.testing.assert_array_equal(oracle.tree_check(p2, n, d2), [2 + 7, 2 + 12, 2])
    np.testing.assert_array_equal(oracle.tree_check(p2, n), [2 + 7, 0, 2])
    np.testing.assert_array_equal(oracle.tree_check(parent, np.array([0, 34, 1])), [1, 1, 0])
    # rows past n_nodes are not looked at
    p3 = parent.copy()
    p3[:, 20:] = 99
    np.testing.assert_array_equal(oracle.tree_check(p3, np.array([20, 20, 21])), [0, 0, 22])
