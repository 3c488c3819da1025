"""Pins of the oracle's tree attention against torch's scaled_dot_product_attention
(CPU, fp64) -- an independent library routine.

(i)  A chain tree under the tree mask equals causal attention over
     [context; chain] (primer: "why target verification can run in
     parallel" -- each draft position sees the context and the drafts left
     of it).
(ii) Every node equals plain, unmasked attention over the context plus its
     own root-to-node path gathered into a separate sequence (PTD sec. 3.1:
     a node sees only pi(v)).
Special cases: a star tree, an empty context, GQA head grouping.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _sdpa(q, k, v, mask=None):
    """q [Hq][n][D], k/v [Hq][m][D] float64 tensors."""
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask)


def _expand_kv(kb, G):
    # kb [Hkv][m][D] -> [Hq][m][D], query head h reads kv head h // G
    return kb.repeat_interleave(G, dim=0)


def _make(r, b, N, Hq, Hkv, D, cap):
    q = r.standard_normal((b, N, Hq, D))
    k = r.standard_normal((b, Hkv, cap, D))
    v = r.standard_normal((b, Hkv, cap, D))
    return q, k, v


@pytest.mark.parametrize("L,n,Hq,Hkv", [(37, 9, 4, 2), (0, 5, 2, 2), (64, 70, 8, 2)])
def test_chain_equals_causal(orc, L, n, Hq, Hkv):
    r = np.random.default_rng(L + n)
    D = 16
    cap = L + n + 3
    q, k, v = _make(r, 1, n, Hq, Hkv, D, cap)
    parent = np.arange(-1, n - 1, dtype=np.int32)
    anc, _ = orc.ancestors(parent)
    out, lse = orc.tree_attention(q, k, v, np.array([L]), anc[None], np.array([n]))
    G = Hq // Hkv
    Q = torch.from_numpy(q[0].transpose(1, 0, 2).copy())                   # [Hq][n][D]
    Kt = _expand_kv(torch.from_numpy(k[0, :, :L + n]), G)
    Vt = _expand_kv(torch.from_numpy(v[0, :, :L + n]), G)
    mask = torch.ones(n, L + n, dtype=torch.bool)
    mask[:, L:] = torch.tril(torch.ones(n, n, dtype=torch.bool))
    ref = _sdpa(Q, Kt, Vt, mask).numpy().transpose(1, 0, 2)
    assert np.allclose(out[0], ref, atol=1e-12, rtol=1e-12)
    # lse: log-sum-exp of the visible scores
    s = np.einsum("hnd,hmd->hnm", Q.numpy(), Kt.numpy()) / np.sqrt(D)
    s = np.where(mask.numpy()[None], s, -np.inf)
    ref_lse = np.log(np.exp(s).sum(-1)).transpose(1, 0)
    assert np.allclose(lse[0], ref_lse, atol=1e-12)


def _random_parent(r, n):
    parent = np.full(n, -1, np.int32)
    for i in range(1, n):
        parent[i] = r.integers(0, i)
    return parent


@pytest.mark.parametrize("shape", ["random", "star"])
@pytest.mark.parametrize("L", [0, 50])
def test_node_equals_attention_over_its_path(orc, shape, L):
    r = np.random.default_rng(11 + L)
    n, Hq, Hkv, D = 23, 4, 1, 8
    cap = L + n
    q, k, v = _make(r, 2, n, Hq, Hkv, D, cap)
    parents = []
    for b in range(2):
        parents.append(_random_parent(r, n) if shape == "random"
                       else np.array([-1] + [0] * (n - 1), np.int32))
    anc = np.stack([orc.ancestors(p)[0] for p in parents])
    out, lse = orc.tree_attention(q, k, v, np.array([L, L]), anc, np.array([n, n]))
    for b in range(2):
        for i in range(n):
            path, u = [], i
            while u >= 0:
                path.append(u)
                u = parents[b][u] if u > 0 else -1
            path = sorted(path)
            idx = list(range(L)) + [L + j for j in path]
            Kt = _expand_kv(torch.from_numpy(k[b][:, idx]), Hq // Hkv)
            Vt = _expand_kv(torch.from_numpy(v[b][:, idx]), Hq // Hkv)
            Q = torch.from_numpy(q[b, i][:, None, :].copy())               # [Hq][1][D]
            ref = _sdpa(Q, Kt, Vt)[:, 0].numpy()
            assert np.allclose(out[b, i], ref, atol=1e-12, rtol=1e-12)


def test_padding_rows_and_subset(orc):
    r = np.random.default_rng(12)
    n, N = 5, 9
    q, k, v = _make(r, 1, N, 2, 1, 4, 20 + N)
    parent = _random_parent(r, n)
    anc = np.zeros((1, N, 1), np.uint64)
    anc[0, :n] = orc.ancestors(parent)[0]
    out, lse = orc.tree_attention(q, k, v, np.array([20]), anc, np.array([n]))
    assert np.all(out[0, n:] == 0) and np.all(np.isneginf(lse[0, n:]))
    sub = orc.tree_attention_rows(q, k, v, np.array([20]), anc, np.array([n]), [(0, 3)])
    assert np.array_equal(sub[(0, 3)][0], out[0, 3])
