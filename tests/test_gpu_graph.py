"""Every call of the library captured in a HIP graph (torch.cuda.graph) and
replayed several times, with eager work and synchronisations between the
replays: each replay must reproduce the eager results bit for bit (the
calls launch kernels only; no memset or allocation enters the graph)."""
import numpy as np
import pytest
import torch

import tree_verification_best_amd as tv
import workloads
from gpu_util import bf16_dev, dev

pytestmark = pytest.mark.gpu


def _scrub(tensors):
    for t in tensors:
        t.fill_(-7 if t.dtype in (torch.int32, torch.int64) else float("nan"))


def _check_replays(graph, outs, want, restore=None, keep=(), reps=3):
    """keep: outputs modified in place from inputs that restore() resets."""
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(reps):
        if restore is not None:
            restore()
        _scrub([t for name, t in outs.items() if name not in keep])
        torch.cuda.synchronize()
        graph.replay()
        # eager work of the program's own between replays
        other.mul_(1.5).add_(float(rep))
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, want[name]), (rep, name)


def test_round_replays():
    c = workloads.CONFIGS["4b"]
    b, N, K, V = 2, c["B"] + 1, c["K"], c["V"]
    draft, target = workloads.logits(c, b, N)
    roots = dev(workloads.root_tokens(c, b))
    ctx = dev(np.array([700, 1500], np.int32))
    cap = 1500 + N
    q, k, v = workloads.qkv(c, b, N, cap)
    d, t = dev(draft), dev(target)
    qd, kd, vd = bf16_dev(q), bf16_dev(k), bf16_dev(v)
    wsb = torch.empty(tv.tree_build_workspace(b, K, V, c["k"], c["B"]), dtype=torch.uint8,
                      device="cuda")
    wsa = torch.empty(tv.attention_workspace(b, N, c["Hq"], c["Hkv"], c["D"], 1500),
                      dtype=torch.uint8, device="cuda")
    wsc = torch.zeros(tv.accept_workspace(b, N, K, V, tv.TV_SAMPLED), dtype=torch.uint8,
                      device="cuda")
    tree = tv.tv_tree_build(d, c["k"], c["B"], roots, ctx, workspace=wsb)
    out = torch.empty((b, N, c["Hq"], c["D"]), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, N, c["Hq"]), dtype=torch.float32, device="cuda")
    out_rope = torch.empty((b, N, c["Hq"], c["D"]), dtype=torch.bfloat16, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    acc = dict(accept_len=torch.empty((b,), **i32), accepted_nodes=torch.empty((b, K + 1), **i32),
               out_tokens=torch.empty((b, K + 1), **i32))
    cost = dev(1.0 + 0.01 * np.arange(N))
    n_out = torch.empty((b,), **i32)

    def round_():
        tv.tv_tree_build(d, c["k"], c["B"], roots, ctx, workspace=wsb, out=tree)
        tv.tv_tree_attention_verify(qd, kd, vd, ctx, tree["anc"], tree["n_nodes"], 1500,
                                    workspace=wsa, out=out, lse=lse)
        tv.tv_tree_attention_verify(qd, kd, vd, ctx, tree["anc"], tree["n_nodes"], 1500,
                                    workspace=wsa, out=out_rope, lse=None, want_lse=False,
                                    pos=tree["pos"], rope_base=1e6)
        tv.tv_tree_accept(t, tree["parent"], tree["token"], tree["depth"], tree["n_nodes"],
                          mode=tv.TV_SAMPLED, seed=9, round=4, max_depth=K, workspace=wsc,
                          out=acc)
        tv.tv_tree_budget(tree["score"], tree["n_nodes"], cost, n_nodes_out=n_out)

    round_()
    torch.cuda.synchronize()
    outs = dict(tree, out=out, lse=lse, rope=out_rope, n_out=n_out, **acc)
    want = {name: x.clone() for name, x in outs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        round_()
    _check_replays(g, outs, want)


def test_commit_and_expand_replay():
    c = workloads.CONFIGS["4b"]
    b, Hkv, D, cap, width = 2, 8, 128, 600, 9
    r = np.random.default_rng(5)
    k0 = bf16_dev(r.standard_normal((b, Hkv, cap, D)).astype(np.float32))
    v0 = bf16_dev(r.standard_normal((b, Hkv, cap, D)).astype(np.float32))
    kk, vv = k0.clone(), v0.clone()
    ctx = dev(np.array([100, 400], np.int32))
    alen = dev(np.array([4, 2], np.int32))
    nodes = np.full((b, width), -1, np.int32)
    nodes[0, :5] = [0, 3, 4, 9, 20]
    nodes[1, :3] = [0, 1, 5]
    nodes = dev(nodes)
    newl = torch.empty((b,), dtype=torch.int32, device="cuda")
    # layer-wise drafting at the 8B frontier shape
    W, m, N = 8, 8, 257
    xl = [dev(a) for a in workloads.expand_logits(dict(c, dtype="f32"), b, W, 3)]
    roots = dev(np.array([5, 6], np.int32))
    tree = tv.tv_tree_root(roots, ctx, N)
    front0 = torch.full((b, W), -1, dtype=torch.int32, device="cuda")
    front0[:, 0] = 0
    front = front0.clone()
    nxt = torch.empty_like(front)
    wsx = torch.empty(tv.tree_expand_workspace(b, W, c["V"], m), dtype=torch.uint8, device="cuda")

    def restore():
        kk.copy_(k0)
        vv.copy_(v0)

    def calls():
        tv.tv_kv_commit(kk, vv, ctx, alen, nodes, new_ctx_len=newl, rope_base=1e4)
        tv.tv_tree_root(roots, ctx, N, out=tree)
        front.copy_(front0)
        for x in xl:
            tv.tv_tree_expand(x, m, front, tree, ctx, next_frontier=nxt, workspace=wsx)
            front.copy_(nxt)

    restore()
    calls()
    torch.cuda.synchronize()
    outs = dict(tree, k=kk, v=vv, newl=newl, front=front)
    want = {name: x.clone() for name, x in outs.items()}
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    _check_replays(g, outs, want, restore=restore, keep=("k", "v"))
