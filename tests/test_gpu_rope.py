"""GPU parity of the rotary-embedding variants with the fp64 oracle.

tv_tree_attention_verify_rope: max abs error <= 1e-2 and norm-wise relative
error <= 2e-2 per sequence, as the plain attention (the rotated bf16 values
are rounded to bf16 before the products).  tv_kv_commit_rope: V rows, rows
left alone and lengths bit-exact; each rotated K element within the
rounding of its fp32 rotation to the cache dtype (2^-8 relative for bf16,
nearest even), plus the fp32 rotation's own error, at most 5e-7 times the
pair's magnitude (angle reduced in fp64, sin/cos in fp32)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv
import workloads
from gpu_util import assert_attention_close, bf16_dev, dev, host

pytestmark = pytest.mark.gpu


def _tree(r, kind, n, N):
    parent = np.full(N, -1, np.int32)
    for i in range(1, n):
        parent[i] = i - 1 if kind == "chain" else (0 if kind == "star" else r.integers(0, i))
    anc = np.zeros((N, (N + 63) // 64), np.uint64)
    depth = np.full(N, -1, np.int32)
    a, d = oracle.ancestors(parent[:n], words=(N + 63) // 64)
    anc[:n], depth[:n] = a, d
    return anc, depth


CASES = [
    # name, b, N, Hq, Hkv, D, Ls, ns, kind, dtype, splits, base
    ("f32", 2, 20, 4, 2, 128, [70, 0], [20, 13], "random", "f32", 0, 1e4),
    ("bf16-d128", 1, 20, 4, 2, 128, [100], [20], "random", "bf16", 0, 1e4),
    ("bf16-d64", 1, 33, 8, 8, 64, [257], [30], "random", "bf16", 0, 1e4),
    ("chain", 1, 40, 4, 1, 128, [64], [40], "chain", "bf16", 0, 1e6),
    ("no-context", 1, 24, 8, 2, 128, [0], [24], "random", "bf16", 0, 1e6),
    ("ragged-batch", 3, 33, 8, 2, 128, [1000, 37, 513], [33, 1, 20], "random", "bf16", 0, 1e6),
    ("far-positions", 1, 65, 8, 2, 128, [30000], [65], "random", "bf16", 3, 1e6),
    ("4b-heads", 1, 65, 32, 8, 128, [4096], [65], "random", "bf16", 0, 1e6),
    ("wide-tree", 1, 257, 8, 2, 128, [300], [257], "random", "bf16", 0, 1e4),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_rope(case):
    name, b, N, Hq, Hkv, D, Ls, ns, kind, dt, splits, base = case
    r = np.random.default_rng(zlib.crc32(name.encode()))
    cap = max(Ls) + N + 5
    q = r.standard_normal((b, N, Hq, D)).astype(np.float32)
    k = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    v = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    if dt == "bf16":
        q, k, v = workloads.round_bf16(q), workloads.round_bf16(k), workloads.round_bf16(v)
    trees = [_tree(r, kind, ns[s], N) for s in range(b)]
    anc = np.stack([t[0] for t in trees])
    ctx = np.array(Ls, np.int32)
    pos = np.stack([np.where(t[1] >= 0, Ls[s] + t[1], -1) for s, t in enumerate(trees)])
    pos = pos.astype(np.int32)
    nn = np.array(ns, np.int32)
    put = bf16_dev if dt == "bf16" else dev
    out, lse = tv.tv_tree_attention_verify(put(q), put(k), put(v), dev(ctx),
                                           dev(anc.view(np.int64)), dev(nn), max(Ls),
                                           splits=splits, pos=dev(pos), rope_base=base)
    torch.cuda.synchronize()
    ro, rl = oracle.tree_attention_rope(q, k, v, ctx, anc, nn, pos, base)
    assert_attention_close(out, lse, ro, rl, nn, name)
    # a rotation that moves nothing: pos 0 everywhere equals the plain call
    if name == "bf16-d128":
        z = np.zeros_like(pos)
        o0, _ = tv.tv_tree_attention_verify(put(q), put(k), put(v), dev(ctx),
                                            dev(anc.view(np.int64)), dev(nn), max(Ls),
                                            pos=dev(z), rope_base=base)
        o1, _ = tv.tv_tree_attention_verify(put(q), put(k), put(v), dev(ctx),
                                            dev(anc.view(np.int64)), dev(nn), max(Ls))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(o0), host(o1))


def test_attention_rope_full_size_rows():
    """The 8B shape (32q/8kv, D 128, context 8192, 257 tree rows) in the
    launch configuration the round uses, checked on sampled rows."""
    cfg = workloads.CONFIGS["8b"]
    b, N, L = 1, cfg["B"] + 1, cfg["L"]
    cap = L + N
    q, k, v = workloads.qkv(cfg, b, N, cap, salt=5)
    parent, _, _ = workloads.random_trees(cfg, b, N, salt=5, max_depth=cfg["K"])
    anc, depth = oracle.ancestors(parent[0])
    pos = (L + depth)[None].astype(np.int32)
    nn = np.array([N], np.int32)
    ctx = np.array([L], np.int32)
    out, lse = tv.tv_tree_attention_verify(bf16_dev(q), bf16_dev(k), bf16_dev(v), dev(ctx),
                                           dev(anc[None].view(np.int64)), dev(nn), L,
                                           pos=dev(pos), rope_base=1e6)
    torch.cuda.synchronize()
    rows = [(0, i) for i in (0, 1, 2, 77, 128, 200, N - 1)]
    ref = oracle.tree_attention_rope_rows(q, k, v, ctx, anc[None], nn, pos, 1e6, rows)
    g = host(out)
    gl = host(lse)
    for (s, i), (o, l) in ref.items():
        d = g[s, i] - o
        assert np.abs(d).max() <= 1e-2, i
        assert np.linalg.norm(d) / np.linalg.norm(o) <= 2e-2, i
        assert np.abs(gl[s, i] - l).max() <= 1e-2, i


def _commit_case(r, b, Hkv, D, Ls, paths, width, cap, dt):
    k = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    v = r.standard_normal((b, Hkv, cap, D)).astype(np.float32)
    if dt == "bf16":
        k, v = workloads.round_bf16(k), workloads.round_bf16(v)
    acc = np.full((b, width), -1, np.int32)
    alen = np.empty(b, np.int32)
    for s, p in enumerate(paths):
        if p is None:
            alen[s] = -1
            continue
        acc[s, :len(p)] = p
        alen[s] = len(p) - 1
    return k, v, np.array(Ls, np.int32), alen, acc


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_commit_rope_matches_oracle(dt, D):
    r = np.random.default_rng(D + (1 if dt == "bf16" else 2))
    b, Hkv, width = 5, 3, 20
    Ls = [40, 0, 100, 7, 3000]
    cap = 3000 + 40
    paths = [[0, 2, 5, 6, 11, 19], [0], None, [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11],
             [0, 3, 3]]  # the last is not strictly increasing: refused
    k, v, ctx, alen, acc = _commit_case(r, b, Hkv, D, Ls, paths, width, cap, dt)
    base = 1e6 if D == 128 else 1e4
    put = bf16_dev if dt == "bf16" else dev
    kg, vg = put(k), put(v)
    new = tv.tv_kv_commit(kg, vg, dev(ctx), dev(alen), dev(acc), rope_base=base)
    torch.cuda.synchronize()
    ko, vo, no = oracle.kv_commit_rope(k, v, ctx, alen, acc, base)
    np.testing.assert_array_equal(host(new), no)
    np.testing.assert_array_equal(host(vg), vo)
    kh = host(kg).astype(np.float64)
    rel = 2.0 ** -8 if dt == "bf16" else 2.0 ** -23
    for s in range(b):
        L, a = int(ctx[s]), int(alen[s])
        kept = a + 1 if (a >= 0 and no[s] == L + a + 1) else 0
        # rows outside the kept range are untouched
        np.testing.assert_array_equal(kh[s, :, :L], k[s, :, :L])
        np.testing.assert_array_equal(kh[s, :, L + kept:], k[s, :, L + kept:])
        if kept == 0:
            continue
        src = k[s][:, [L + int(x) for x in acc[s, :kept]]].astype(np.float64)
        pair = np.abs(src[..., :D // 2]) + np.abs(src[..., D // 2:])
        pair = np.concatenate([pair, pair], axis=-1)
        got, want = kh[s, :, L:L + kept], ko[s, :, L:L + kept]
        bound = rel * np.abs(want) + 5e-7 * pair
        assert (np.abs(got - want) <= bound).all(), (s, np.abs(got - want).max())


def test_verify_then_commit_rope_round_trip():
    """Verification with fused rotation, commit with rotation, then the plain
    (rotation-free) attention of a kept node over the committed prefix gives
    what that node received in verification, to the attention tolerance."""
    r = np.random.default_rng(21)
    b, N, Hq, Hkv, D, L = 1, 24, 8, 2, 128, 500
    cap = L + N + 4
    q = workloads.round_bf16(r.standard_normal((b, N, Hq, D)).astype(np.float32))
    k = workloads.round_bf16(r.standard_normal((b, Hkv, cap, D)).astype(np.float32))
    v = workloads.round_bf16(r.standard_normal((b, Hkv, cap, D)).astype(np.float32))
    anc, depth = _tree(r, "random", N, N)
    pos = (L + depth)[None].astype(np.int32)
    ctx = np.array([L], np.int32)
    nn = np.array([N], np.int32)
    kg, vg = bf16_dev(k), bf16_dev(v)
    out, _ = tv.tv_tree_attention_verify(bf16_dev(q), kg, vg, dev(ctx),
                                         dev(anc[None].view(np.int64)), dev(nn), L,
                                         pos=dev(pos), rope_base=1e6)
    # the deepest node's path is kept
    u = int(np.argmax(depth))
    path = [i for i in range(N) if (int(anc[u, i // 64]) >> (i % 64)) & 1]
    acc = np.full((b, N), -1, np.int32)
    acc[0, :len(path)] = path
    tv.tv_kv_commit(kg, vg, dev(ctx), dev(np.array([len(path) - 1], np.int32)), dev(acc),
                    rope_base=1e6)
    torch.cuda.synchronize()
    kc = host(kg).astype(np.float64)
    vc = host(vg).astype(np.float64)
    nk = L + len(path)
    qr = oracle.rope(q[0, u].astype(np.float64), L + len(path) - 1, 1e6)
    G = Hq // Hkv
    o = host(out)[0, u]
    for h in range(Hq):
        s = kc[0, h // G, :nk] @ qr[h] / np.sqrt(D)
        w = np.exp(s - s.max())
        ref = (w / w.sum()) @ vc[0, h // G, :nk]
        assert np.abs(o[h] - ref).max() <= 1e-2
