"""Pins of the rotary embedding on tree positions (oracle/rope.py).

The rotation is checked against its complex-number definition, its
relative-position property and its invariants; tree attention with it is
checked against torch's scaled_dot_product_attention (CPU, fp64) over plain
sequences whose keys and queries were rotated at their sequence positions:
a chain tree is the causal case, and any node equals plain attention over
the context plus its own root-to-node path (PTD sec. 3.1: a node's position
follows from the size of pi(v)).  The commit is checked by what it is for:
after it, a kept node's rotated query over the committed, fully rotated
prefix reproduces the attention it received in verification."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

BASE = 10000.0


def _complex_rope(x, pos, base):
    """Pair i as z = x_i + 1j x_{i+D/2}, turned by e^{1j pos theta_i}, with
    theta_i = exp(-(2i/D) ln base)."""
    D = x.shape[-1]
    z = x[..., :D // 2] + 1j * x[..., D // 2:]
    theta = np.exp(-(2.0 * np.arange(D // 2) / D) * np.log(base))
    z = z * np.exp(1j * np.asarray(pos, np.float64)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("D", [8, 64, 128])
def test_rope_matches_complex_rotation(D):
    r = np.random.default_rng(D)
    x = r.standard_normal((5, 3, D))
    pos = r.integers(0, 40000, size=(5, 3))
    np.testing.assert_allclose(oracle.rope(x, pos, BASE), _complex_rope(x, pos, BASE),
                               rtol=0, atol=1e-9)
    np.testing.assert_allclose(oracle.rope(x, pos, 1e6), _complex_rope(x, pos, 1e6),
                               rtol=0, atol=1e-9)


def test_rope_invariants():
    r = np.random.default_rng(3)
    D = 64
    x = r.standard_normal((7, D))
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(7, np.int64), BASE), x)
    y = oracle.rope(x, np.arange(7) * 997, BASE)
    # each pair keeps its length
    np.testing.assert_allclose(np.hypot(y[:, :D // 2], y[:, D // 2:]),
                               np.hypot(x[:, :D // 2], x[:, D // 2:]), rtol=1e-12)
    # pair 0 turns by pos radians exactly (theta_0 = 1)
    ang = np.arctan2(y[:, D // 2], y[:, 0]) - np.arctan2(x[:, D // 2], x[:, 0])
    np.testing.assert_allclose(np.angle(np.exp(1j * (ang - np.arange(7) * 997))), 0, atol=1e-9)


def test_rope_scores_depend_on_offset_only():
    r = np.random.default_rng(4)
    D = 128
    q, k = r.standard_normal(D), r.standard_normal(D)
    for m, n in [(5, 3), (4096, 4000), (30000, 29999), (7, 7)]:
        a = oracle.rope(q, m, BASE) @ oracle.rope(k, n, BASE)
        b = oracle.rope(q, m - n, BASE) @ k
        c = oracle.rope(q, m + 1234, BASE) @ oracle.rope(k, n + 1234, BASE)
        assert abs(a - b) < 1e-9 and abs(a - c) < 1e-9


def _sdpa(q, k, v, mask):
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                          torch.from_numpy(v), attn_mask=torch.from_numpy(mask))


def _cache(r, Hkv, L, n, D, cap):
    """Context keys stored rotated at their positions; tree rows raw."""
    kraw = r.standard_normal((Hkv, cap, D))
    k = kraw.copy()
    k[:, :L] = oracle.rope(kraw[:, :L], np.arange(L)[None, :], BASE)
    v = r.standard_normal((Hkv, cap, D))
    return kraw, k, v


@pytest.mark.parametrize("L,n", [(0, 6), (33, 9), (70, 17)])
def test_chain_with_rope_equals_causal_rotated_sequence(L, n):
    r = np.random.default_rng(L + n)
    Hq, Hkv, D = 4, 2, 16
    G = Hq // Hkv
    cap = L + n + 2
    kraw, k, v = _cache(r, Hkv, L, n, D, cap)
    q = r.standard_normal((1, n, Hq, D))
    parent = np.arange(-1, n - 1, dtype=np.int32)
    anc, depth = oracle.ancestors(parent)
    pos = (L + depth)[None].astype(np.int32)
    out, _ = oracle.tree_attention_rope(q, k[None], v[None], np.array([L]), anc[None],
                                        np.array([n]), pos, BASE)
    seq = np.arange(L + n)
    Q = oracle.rope(q[0].transpose(1, 0, 2), seq[L:][None, :], BASE)           # [Hq][n][D]
    Kt = np.repeat(oracle.rope(kraw[:, :L + n], seq[None, :], BASE), G, axis=0)
    Vt = np.repeat(v[:, :L + n], G, axis=0)
    mask = np.ones((n, L + n), bool)
    mask[:, L:] = np.tril(np.ones((n, n), bool))
    ref = _sdpa(Q, Kt, Vt, mask).numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(out[0], ref, atol=1e-11, rtol=0)


def test_branching_node_equals_attention_over_its_rotated_path():
    r = np.random.default_rng(8)
    L, n, Hq, Hkv, D = 21, 19, 2, 1, 32
    cap = L + n
    kraw, k, v = _cache(r, Hkv, L, n, D, cap)
    q = r.standard_normal((1, n, Hq, D))
    parent = np.full(n, -1, np.int32)
    for i in range(1, n):
        parent[i] = r.integers(max(0, i - 4), i)
    anc, depth = oracle.ancestors(parent)
    pos = (L + depth)[None].astype(np.int32)
    out, _ = oracle.tree_attention_rope(q, k[None], v[None], np.array([L]), anc[None],
                                        np.array([n]), pos, BASE)
    for i in range(n):
        path = [i]
        while parent[path[-1]] >= 0:
            path.append(int(parent[path[-1]]))
        path = path[::-1]
        rows = np.concatenate([np.arange(L), L + np.array(path)])
        seqpos = np.arange(len(rows))          # a plain sequence: context, then the path
        Kp = oracle.rope(kraw[:, rows], seqpos[None, :], BASE)
        Qp = oracle.rope(q[0, i][:, None, :], np.array([[len(rows) - 1]]), BASE)  # [Hq][1][D]
        ref = _sdpa(Qp, np.repeat(Kp, Hq // Hkv, 0), np.repeat(v[:, rows], Hq // Hkv, 0),
                    np.ones((1, len(rows)), bool)).numpy()[:, 0]
        np.testing.assert_allclose(out[0, i], ref, atol=1e-11, rtol=0)
    # the oracle's rows variant agrees with the full call
    rr = oracle.tree_attention_rope_rows(q, k[None], v[None], np.array([L]), anc[None],
                                         np.array([n]), pos, BASE, [(0, 3), (0, n - 1)])
    np.testing.assert_array_equal(rr[(0, 3)][0], out[0, 3])


def test_commit_with_rope_reproduces_verification():
    r = np.random.default_rng(12)
    L, n, Hq, Hkv, D = 30, 16, 4, 2, 16
    G = Hq // Hkv
    cap = L + n + 4
    _, k, v = _cache(r, Hkv, L, n, D, cap)
    q = r.standard_normal((1, n, Hq, D))
    parent = np.array([-1, 0, 0, 1, 1, 2, 3, 3, 4, 6, 6, 7, 9, 9, 10, 12], np.int32)
    anc, depth = oracle.ancestors(parent)
    pos = (L + depth)[None].astype(np.int32)
    out, _ = oracle.tree_attention_rope(q, k[None], v[None], np.array([L]), anc[None],
                                        np.array([n]), pos, BASE)
    path = [0, 1, 3, 6, 9, 12]
    acc = np.full((1, 8), -1, np.int32)
    acc[0, :len(path)] = path
    k2, v2, new = oracle.kv_commit_rope(k[None], v[None], np.array([L]),
                                        np.array([len(path) - 1]), acc, BASE)
    assert new[0] == L + len(path)
    # every key row below the new length is now rotated at its own position
    for j, node in enumerate(path):
        nk = L + j + 1
        qr = oracle.rope(q[0, node], L + j, BASE)                      # [Hq][D]
        for h in range(Hq):
            s = k2[0, h // G, :nk] @ qr[h] / np.sqrt(D)
            w = np.exp(s - s.max())
            ref = (w / w.sum()) @ v2[0, h // G, :nk]
            np.testing.assert_allclose(out[0, node, h], ref, atol=1e-11, rtol=0)
    # rows past the new length and the context keep their values
    np.testing.assert_array_equal(k2[0, :, :L], k[:, :L])
    np.testing.assert_array_equal(k2[0, :, L + len(path):], k[:, L + len(path):])
