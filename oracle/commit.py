"""KV commit after a verification round, in numpy (test infrastructure only).

Primer, "KV cache handling": the target cache keeps only the accepted tokens;
the entries of the rejected candidates are dropped.  After a round, tree row
L_b + i of the cache holds node i; the committed sequence is the root followed
by the accepted drafts, accepted_nodes[b][0..accept_len[b]].  The commit
places row L_b + accepted_nodes[b][j] at row L_b + j, for j = 0..accept_len[b],
in both caches and every KV head, and the new context length is
L_b + accept_len[b] + 1.  Rows past it are free for the next round.

A sequence with accept_len[b] < 0 (a walk that refused the tree) is left as
is, new length L_b.  A path that does not start at node 0, is not strictly
increasing, does not fit in the width, or reaches past the cache (or a
negative L_b) is left as is, new length -1.

Layouts: k, v [b][Hkv][cap][D]; ctx_len, accept_len [b];
accepted_nodes [b][width].
"""
import numpy as np


def valid_path(path, L, cap):
    return (len(path) >= 1 and path[0] == 0 and all(path[j] < path[j + 1]
            for j in range(len(path) - 1)) and L >= 0 and L + path[-1] < cap)


def kv_commit(k, v, ctx_len, accept_len, accepted_nodes):
    """Returns (k', v', new_ctx_len); the inputs are not modified."""
    k = np.array(k, copy=True)
    v = np.array(v, copy=True)
    b, _, cap, _ = k.shape
    width = accepted_nodes.shape[1]
    new = np.empty(b, np.int32)
    for s in range(b):
        L, a = int(ctx_len[s]), int(accept_len[s])
        if a < 0:
            new[s] = L
            continue
        path = [int(x) for x in accepted_nodes[s][:a + 1]] if a + 1 <= width else []
        if not valid_path(path, L, cap):
            new[s] = -1
            continue
        src = [L + p for p in path]
        # fancy indexing reads every source row before any row is written
        k[s, :, L:L + a + 1, :] = k[s][:, src, :]
        v[s, :, L:L + a + 1, :] = v[s][:, src, :]
        new[s] = L + a + 1
    return k, v, new
