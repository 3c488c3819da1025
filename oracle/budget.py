"""Cost-aware choice of the tree size (test infrastructure only).

TAPS sec. 3.2 (key insight) and sec. 4.1 (third stage): verification should
be cost-aware rather than fill the budget -- the selector keeps a compact
prefix-closed subtree that maximises the expected number of accepted tokens
per unit of verification cost.  A best-first prefix of n nodes is the best
prefix-closed subtree of size n (each node's path score is at most its
parent's), so only the size is chosen: with the path scores s_1 >= s_2 >= ...
of the built tree (row 0 is the root), the round emits 1 + sum_{i<=n} s_i
tokens in expectation when the scores are the true reach probabilities, and

    n* = the smallest n in [0, n_nodes - 1] maximising r_n = (1 + S_n) / c[n],

where S_n is the left-to-right fp64 sum s_1 + ... + s_n, r_n is one fp64
division, and c[n] > 0 is the caller's measured cost of verifying a tree of
n draft nodes.  The new node count is n* + 1.
"""
import numpy as np


def tree_budget(score, n_nodes, cost):
    """score [b][N] f64, n_nodes [b], cost [>= max n_nodes] f64 -> n_nodes' [b]."""
    score = np.asarray(score, np.float64)
    cost = np.asarray(cost, np.float64)
    out = np.empty(len(n_nodes), np.int32)
    for s, n in enumerate(n_nodes):
        n = int(n)
        S = 0.0
        best_n, best_r = 0, (1.0 + S) / cost[0]
        for i in range(1, n):
            S = S + float(score[s, i])
            r = (1.0 + S) / cost[i]
            if r > best_r:
                best_n, best_r = i, r
        out[s] = best_n + 1
    return out
