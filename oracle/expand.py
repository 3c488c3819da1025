"""One drafting step of a layer-wise tree builder (test infrastructure only).

TreeGraft sec. 3.1, "standard single-drafter expansion": at drafting step k
the candidate pool is the set of nodes added at the previous step (the root
at the first step); the frontier is the W of them with the highest path
score s(v), Top_W(C_k, s); the drafter runs on the prefix ending at each
frontier node and the top-m tokens of that next-token distribution become its
children; the edge score p(u) is the drafter's probability of u's token and
s(v) is the product of the edge scores on the path from the root (s(root) = 1).

Here the drafter's outputs are given: node_logits[b][w] is the next-token
logits row for frontier slot w.  Probabilities follow the build's fixed-point
softmax (q = W(t) / Z at the build temperature) and the top-m order is
(q desc, id asc).  Children are appended in frontier-slot order, then rank
order, at rows n_nodes, n_nodes + 1, ...; rows past the tree's capacity N are
dropped.  Each child gets depth(parent) + 1, pos = L + depth, its ancestor
row (the parent's plus itself) and s = fl64(s(parent) * q).  The next frontier
is the W new children with the highest s (ties: the lower row), padded
with -1.  A frontier slot holding -1 or a row outside [0, n_nodes) is empty;
a sequence whose n_nodes is outside [1, N] is left as it is.
"""
import numpy as np

from . import draft_candidates


def tree_expand(node_logits, m, frontier, tree, ctx_len, build_temp=1.0):
    """node_logits [b][W][V]; frontier [b][W]; tree: dict of parent, token,
    depth, pos (int32 [b][N]), score (f64 [b][N]), anc (u64 [b][N][words]),
    n_nodes (int32 [b]).  Returns (new tree dict, next_frontier [b][W])."""
    t = {f: np.array(v, copy=True) for f, v in tree.items()}
    b, W = frontier.shape
    N = t["parent"].shape[1]
    nxt = np.full((b, W), -1, np.int32)
    for s in range(b):
        n0 = int(t["n_nodes"][s])
        if n0 < 1 or n0 > N:  # not a tree: left as it is
            continue
        tok, q, _ = draft_candidates(node_logits[s], m, build_temp)
        row = n0
        new = []
        for w in range(W):
            f = int(frontier[s, w])
            if f < 0 or f >= n0:
                continue
            for r in range(m):
                if row >= N:
                    break
                t["parent"][s, row] = f
                t["token"][s, row] = tok[w, r]
                t["depth"][s, row] = t["depth"][s, f] + 1
                t["pos"][s, row] = int(ctx_len[s]) + t["depth"][s, row]
                t["score"][s, row] = float(t["score"][s, f]) * float(q[w, r])
                t["anc"][s, row] = t["anc"][s, f]
                t["anc"][s, row, row // 64] |= np.uint64(1) << np.uint64(row % 64)
                new.append(row)
                row += 1
        t["n_nodes"][s] = row
        order = sorted(new, key=lambda v: (-float(t["score"][s, v]), v))[:W]
        nxt[s, :len(order)] = order
    return t, nxt


def tree_root(b, N, root_token, ctx_len):
    """A batch of trees holding only their roots (row 0)."""
    words = (N + 63) // 64
    t = dict(parent=np.full((b, N), -1, np.int32), token=np.full((b, N), -1, np.int32),
             depth=np.full((b, N), -1, np.int32), pos=np.full((b, N), -1, np.int32),
             score=np.zeros((b, N), np.float64), anc=np.zeros((b, N, words), np.uint64),
             n_nodes=np.ones(b, np.int32))
    t["token"][:, 0] = root_token
    t["depth"][:, 0] = 0
    t["pos"][:, 0] = ctx_len
    t["score"][:, 0] = 1.0
    t["anc"][:, 0, 0] = 1
    return t
