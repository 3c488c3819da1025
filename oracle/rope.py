"""Rotary position embedding on the tree's position ids (test infrastructure only).

PTD sec. 3.1: a node's position encoding follows from the size of its
observable prefix pi(v), so tree node i sits at position pos[b][i] =
L_b + depth(i) (the root at L_b), the position it would have in a plain
sequence made of the context and its root-to-node path.  The pages do not
define the rotary embedding itself; this is the standard one (RoFormer) with
the half-split pairing of the Qwen / LLaMA family: dimension i < D/2 pairs
with dimension i + D/2 and the pair turns by the angle pos * base^(-2i/D).

The cache convention: context rows [0, L_b) were rotated at their own
positions when they were committed; the tree rows L_b + i hold keys as the
target's projection wrote them, not yet rotated.  So verification rotates
the queries and the tree keys at pos, and the commit that keeps the accepted
path rotates each kept key at the position of the row it lands on.

Everything is fp64 from the exact input values.
"""
import numpy as np

from .attention import tree_attention, tree_attention_rows
from .commit import kv_commit


def inv_freq(D, base):
    """Angle per unit of position of pair i, i < D/2: base^(-2i/D)."""
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


def rope(x, pos, base):
    """x [..., D]; pos integer array broadcastable to x[..., 0]."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, np.float64)[..., None] * inv_freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def _rotated_inputs(q, k, ctx_len, n_nodes, pos, base, seqs):
    q = np.asarray(q, np.float64).copy()
    k = np.asarray(k, np.float64).copy()
    for s in seqs:
        L, n = int(ctx_len[s]), int(n_nodes[s])
        p = np.asarray(pos[s][:n])
        q[s, :n] = rope(q[s, :n], p[:, None], base)          # every query head
        k[s, :, L:L + n] = rope(k[s, :, L:L + n], p[None, :], base)  # every KV head
    return q, k


def tree_attention_rope(q, k, v, ctx_len, anc, n_nodes, pos, base, scale=None):
    """tree_attention after rotating the queries and the tree keys at pos."""
    b = np.asarray(q).shape[0]
    qr, kr = _rotated_inputs(q, k, ctx_len, n_nodes, pos, base, range(b))
    return tree_attention(qr, kr, v, ctx_len, anc, n_nodes, scale)


def tree_attention_rope_rows(q, k, v, ctx_len, anc, n_nodes, pos, base, rows, scale=None):
    """Only the listed (sequence, node) pairs, as tree_attention_rows."""
    seqs = sorted({s for s, _ in rows})
    qr, kr = _rotated_inputs(q, k, ctx_len, n_nodes, pos, base, seqs)
    return tree_attention_rows(qr, kr, v, ctx_len, anc, n_nodes, rows, scale)


def kv_commit_rope(k, v, ctx_len, accept_len, accepted_nodes, base):
    """kv_commit, then each kept key row L_b + j turned at position L_b + j.
    Returns (k' in fp64, v', new_ctx_len)."""
    k2, v2, new = kv_commit(k, v, ctx_len, accept_len, accepted_nodes)
    k2 = np.asarray(k2, np.float64)
    for s in range(k2.shape[0]):
        L, a = int(ctx_len[s]), int(accept_len[s])
        if a < 0 or int(new[s]) != L + a + 1:
            continue
        k2[s, :, L:L + a + 1] = rope(k2[s, :, L:L + a + 1], np.arange(L, L + a + 1)[None, :],
                                     base)
    return k2, v2, new
