"""Tree-masked attention in fp64 (test infrastructure only).

PTD sec. 3.1 (tree construction): a node v sees only pi(v) = {v} U pi(P(v));
the primer ("why target verification can run in parallel"): the target reads
the original context plus the draft tokens in one pass.  So node i of
sequence b attends to every cached context key [0, L_b) and to the tree keys
stored at cache rows L_b + j for every j in pi(i).  GQA: query head h reads
KV head h // (Hq / Hkv).  Softmax of (q . k) * scale, weighted sum of v,
computed in fp64 from the exact input values, with no blocking or split.

Layouts: q [b][N][Hq][D]; k, v [b][Hkv][cap][D]; anc [b][N][words] (u64 bit
rows, bit j of row i set iff j in pi(i)); ctx_len [b]; n_nodes [b].
Rows i >= n_nodes[b] are padding: output 0, lse -inf.
"""
import numpy as np


def _visible(anc_row, n):
    idx = [j for j in range(n) if (int(anc_row[j // 64]) >> (j % 64)) & 1]
    return np.asarray(idx, dtype=np.int64)


def _one(qrow, kb, vb, L, tree_idx, scale):
    """qrow [Hq][D]; kb, vb [Hkv][cap][D] -> (out [Hq][D], lse [Hq])."""
    Hq, D = qrow.shape
    Hkv = kb.shape[0]
    G = Hq // Hkv
    keys = np.concatenate([np.arange(L, dtype=np.int64), L + tree_idx])
    K = kb[:, keys, :].astype(np.float64)            # [Hkv][nk][D]
    V = vb[:, keys, :].astype(np.float64)
    Q = qrow.astype(np.float64).reshape(Hkv, G, D)    # [Hkv][G][D]
    s = np.matmul(Q, K.transpose(0, 2, 1)) * scale    # [Hkv][G][nk]
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    out = np.matmul(e, V) / z                          # [Hkv][G][D]
    lse = (m + np.log(z))[..., 0]
    return out.reshape(Hq, D), lse.reshape(Hq)


def tree_attention(q, k, v, ctx_len, anc, n_nodes, scale=None):
    q = np.asarray(q)
    b, N, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((b, N, Hq, D), np.float64)
    lse = np.full((b, N, Hq), -np.inf, np.float64)
    for s in range(b):
        L = int(ctx_len[s])
        n = int(n_nodes[s])
        for i in range(n):
            o, l = _one(q[s, i], k[s], v[s], L, _visible(anc[s, i], n), scale)
            out[s, i] = o
            lse[s, i] = l
    return out, lse


def tree_attention_rows(q, k, v, ctx_len, anc, n_nodes, rows, scale=None):
    """Only the listed (sequence, node) pairs: returns {(s, i): (out [Hq][D], lse [Hq])}."""
    q = np.asarray(q)
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    res = {}
    for (s, i) in rows:
        n = int(n_nodes[s])
        res[(s, i)] = _one(q[s, i], k[s], v[s], int(ctx_len[s]), _visible(anc[s, i], n), scale)
    return res
