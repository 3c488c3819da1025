"""Helpers shared by the GPU tests: device transfer and comparison with the oracle."""
import numpy as np
import torch

import workloads

ATOL = 1e-2     # attention: max |gpu - oracle|
RTOL_NORM = 2e-2  # attention: ||gpu - oracle||_2 / ||oracle||_2 per sequence


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_dev(a32):
    """float32 array of bf16-representable values -> bf16 device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(workloads.round_bf16(a32))).to(torch.bfloat16).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def assert_tree_equal(g, o, b):
    """GPU tree (dict of tensors) == oracle tree (dict of arrays), sequence b."""
    n = int(o["n_nodes"][b])
    assert int(host(g["n_nodes"])[b]) == n, "n_nodes"
    for f in ("parent", "token", "depth", "pos"):
        gg = host(g[f])[b]
        assert np.array_equal(gg, o[f][b]), (f, np.nonzero(gg != o[f][b])[0][:10])
    gs = host(g["score"])[b]
    assert np.array_equal(gs.view(np.uint64), o["score"][b].view(np.uint64)), "score bits"
    ga = host(g["anc"])[b].view(np.uint64)
    assert np.array_equal(ga, o["anc"][b]), "anc"


def assert_attention_close(out_gpu, lse_gpu, ref_out, ref_lse, n_nodes, label=""):
    g = host(out_gpu).astype(np.float64)
    for b in range(g.shape[0]):
        n = int(n_nodes[b])
        d = g[b, :n] - ref_out[b, :n]
        mx = np.abs(d).max()
        rel = np.linalg.norm(d) / max(np.linalg.norm(ref_out[b, :n]), 1e-30)
        assert mx <= ATOL, f"{label} seq {b}: max abs {mx}"
        assert rel <= RTOL_NORM, f"{label} seq {b}: rel norm {rel}"
        assert np.all(g[b, n:] == 0)
        if lse_gpu is not None:
            lg = host(lse_gpu)[b].astype(np.float64)
            assert np.abs(lg[:n] - ref_lse[b, :n]).max() <= 1e-2, f"{label} lse"
            assert np.all(np.isneginf(lg[n:]))


def assert_accept_equal(g, o, label=""):
    for f in ("accept_len", "accepted_nodes", "out_tokens"):
        gg = host(g[f])
        assert np.array_equal(gg, o[f]), (label, f, gg[:4], o[f][:4])
