"""Benchmark: one tree-verification round per step on one MI355X.

A step is the whole round on one batch of synthetic input already resident in
HBM: tv_tree_build -> tv_tree_attention_verify (one layer) -> tv_tree_accept.
The timed steps replay the round captured in a HIP graph (one graph per input
set; --eager times eager launches instead); the same steps are then run
eagerly with HIP events around every call, which gives the per-call times and
the roofline (torch on this platform cannot record timing events inside a
graph).
The KV commit that closes a round (tv_kv_commit), the cost-aware tree size
(tv_tree_budget) and a layer-wise build of the same capacity (tv_tree_root +
K drafting steps of tv_tree_expand, frontier width 8) are timed after the
steps, as replays of captured graphs, and reported as per_call.commit,
per_call.budget and per_call.expand (one drafting step).  The verification
with the rotary embedding fused (tv_tree_attention_verify_rope, base 1e6) is
timed per call after the steps and reported as per_call.attention_rope.
config.b_sweep_ms is the verification time against the tree budget B (one
sequence, context 4096, B = 16 .. 512), the measured cost that the timed
tv_tree_budget call takes as its cost curve.  config.cpu_all_cores repeats
the CPU baseline spread over the usable host cores (at most 16).
The default workload is the 4B-class GQA layer (32 query / 8 KV heads, head
dim 128, bf16, context 4096, K = 16 draft positions, top-8, budget 64,
vocabulary 151936, sampled acceptance at T = 1).  Inputs rotate over enough
independent sets (>= 1 GiB) that every step reads HBM, not the 256 MB
Infinity Cache.

Prints ONE JSON line (rank 0).  `value` = tree node x query-head rows
verified per second (rounds/s x N x Hq); config.batch_ms splits the timed
steps into five equal batches (median beside the mean).  `roofline` is for
the dominant kernel of the verification pass, k_attn_partial: its
algorithmic bytes (every input of the call read once) or the call's flops
over its own duration, from HIP events on the call's stream that the
library records just before the partial kernel and between it and the
combine (its timing hook), with the whole call's figures in
roofline.call.  Its `traffic` comes from the HBM byte counters recorded in
profiles/attention_<workload>_traffic.md when that record was taken on the
current attention source (else null).  per_call.attention_8b is the
verification call at the 256-node shape (8B-class layer), timed the same
way after the steps.  mean_accept_len is the mean accept length over every
timed eager step (summed on the device).  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 500] [--warmup 50] [--workload 4b] [--eager]
    python bench.py --copy-calibration      # a plain device copy of known size,
                                            # the reference for the byte counters
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
EXPAND_W = 8   # frontier width of the layer-wise build timed beside the round
ROPE_BASE = 1e6   # rotary base of the fused-rotation verification timed beside the round
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="4b", choices=["4b", "8b", "long", "batched", "tiny"])
    ap.add_argument("--temperature", type=float, default=1.0, help="0 = greedy")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of captured rounds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--round-only", action="store_true",
                    help="time the round alone: no rotary, commit, budget, expansion or budget "
                         "sweep calls after the steps (clean per-kernel profiles)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run 20 plain 256 MiB device-to-device copies and exit")
    return ap.parse_args()


def copy_calibration():
    """20 launches of a plain copy of 256 MiB: FETCH_SIZE / WRITE_SIZE of this
    kernel divided by 256 MiB give the counters' scale factor."""
    import torch
    x = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(20):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": x.numel(), "launches": 20}), flush=True)


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per launch of k_attn_partial (FETCH_SIZE + WRITE_SIZE, each
    scaled by the copy calibration) from the committed counter record, if it
    was taken on the current attention source."""
    rec = os.path.join(ROOT, "profiles", f"attention_{workload}_traffic.md")
    src = os.path.join(ROOT, "tree_verification_best_amd", "csrc", "tv_attention.hip")
    if not os.path.exists(rec):
        return None
    vals = {}
    for line in open(rec):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256_16") != source_digest(src):
        return None
    try:
        return int(vals["k_attn_partial_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(c, b, N, Lsum, build):
    """Each input read once, each output written once, at its dtype."""
    V, K, Hq, Hkv, D = c["V"], c["K"], c["Hq"], c["Hkv"], c["D"]
    el = 2 if c["dtype"] == "bf16" else 4
    W = (N + 63) // 64
    out = {}
    out["build"] = (b * K * V * 4 + b * N * (4 * 4 + 8 + 8 * W)) if build else 0
    kv = 2 * Hkv * D * el * (Lsum + b * N)            # context rows + tree rows, K and V
    qo = 2 * b * N * Hq * D * el + b * N * Hq * 4     # Q in, O out, lse out
    out["attention"] = kv + qo + b * N * 8 * W
    out["accept"] = b * N * V * 4 + b * N * 12
    return out


def attention_flops(c, n_nodes, depths, ctx):
    """4 Hq D sum_i (L + depth_i + 1): unmasked score entries x 2 matmuls x 2."""
    tot = 0
    for s in range(len(n_nodes)):
        n = int(n_nodes[s])
        tot += sum(int(ctx[s]) + int(depths[s][i]) + 1 for i in range(n))
    return 4 * c["Hq"] * c["D"] * tot


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(c, sets0, seconds, workers=1):
    """The oracle, untuned, on the same first input set: whole rounds until
    `seconds` of wall time are spent (at least one).  BLAS runs on one
    thread; with workers > 1 the oracle spreads its independent parts over
    that many workers (the builder's draft positions on OpenMP threads, the
    attention's (sequence, node) rows on worker processes), with the same
    results."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    prev = oracle.set_threads(workers)
    try:
        return _cpu_rounds(c, sets0, seconds, np, threadpool_limits, oracle)
    finally:
        oracle.set_threads(prev)


def _cpu_rounds(c, sets0, seconds, np, threadpool_limits, oracle):
    """Whole oracle rounds on input set 0 until `seconds` have passed."""
    draft, target, q, k, v, roots, ctx = sets0
    b, N = target.shape[0], target.shape[1]
    mode = oracle.GREEDY if c["_T"] == 0 else oracle.SAMPLED
    rounds, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            if c["build"]:
                tr = oracle.tree_build(draft, c["k"], c["B"], roots, ctx)
                parent, token, depth, anc, nn = (tr["parent"], tr["token"], tr["depth"],
                                                 tr["anc"], tr["n_nodes"])
            else:
                parent, token, depth, nn = c["_tree"]
                anc = np.stack([oracle.ancestors(parent[s])[0] for s in range(b)])
            oracle.tree_attention(q, k, v, ctx, anc, nn)
            oracle.tree_accept(target, parent, token, depth, nn, mode=mode,
                               temperature=max(c["_T"], 1e-3), seed=1234, round=rounds,
                               max_depth=c["K"])
            rounds += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    return rounds, dt


def b_sweep(c, dev, stream, budgets=(16, 64, 128, 256, 512), L=4096, reps=50):
    """Verification time (ms per call) of one sequence at context L for each
    tree budget B, on seeded random trees and Q/K/V."""
    import numpy as np
    import torch

    import tree_verification_best_amd as tv
    import workloads

    nmax = max(budgets) + 1
    cap = L + nmax
    q, k, v = workloads.qkv(c, 1, nmax, cap, salt=99)
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(a).to(dev, tdt) for a in (q, k, v))
    ctx = torch.tensor([L], dtype=torch.int32, device=dev)
    out = {}
    for B in budgets:
        N = B + 1
        parent, _, _ = workloads.random_trees(dict(c, name="sweep"), 1, N, salt=B,
                                              max_depth=16, max_children=8)
        nn = torch.tensor([N], dtype=torch.int32, device=dev)
        t = tv.tv_tree_ancestors(torch.from_numpy(parent).to(dev), nn, ctx)
        qn = qd[:, :N].contiguous()
        ws = torch.empty(tv.attention_workspace(1, N, c["Hq"], c["Hkv"], c["D"], L),
                         dtype=torch.uint8, device=dev)
        o = torch.empty(qn.shape, dtype=tdt, device=dev)
        for _ in range(5):
            tv.tv_tree_attention_verify(qn, kd, vd, ctx, t["anc"], nn, L, workspace=ws, out=o,
                                        want_lse=False)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            tv.tv_tree_attention_verify(qn, kd, vd, ctx, t["anc"], nn, L, workspace=ws, out=o,
                                        want_lse=False)
        e1.record(stream)
        torch.cuda.synchronize()
        out[B] = e0.elapsed_time(e1) / reps
    return out


def attention_8b(dev, stream, rotate_gib=1.0, reps=100):
    """The verification call at the 256-node shape (8B-class layer: 32 query /
    8 KV heads, D=128, bf16, context 8192, the tree the builder makes from the
    8B-class draft marginals: K=16, top-16, B=256), per call with HIP events
    on its stream and the partial/combine split from the timing hook; Q/K/V
    ~ N(0,1) drawn on the device from seeded generators, rotated over >= 1 GiB
    of sets."""
    import numpy as np
    import torch

    import tree_verification_best_amd as tv
    import workloads

    c = dict(workloads.CONFIGS["8b"])
    b, N, L = 1, c["B"] + 1, c["L"]
    draft, _ = workloads.logits(c, b, N)
    roots = torch.from_numpy(workloads.root_tokens(c, b)).to(dev)
    ctx = torch.full((b,), L, dtype=torch.int32, device=dev)
    tree = tv.tv_tree_build(torch.from_numpy(draft).to(dev), c["k"], c["B"], roots, ctx)
    cap = L + N
    per_set = 2 * (2 * c["Hkv"] * cap * c["D"] + N * c["Hq"] * c["D"])
    nsets = max(2, math.ceil(rotate_gib * 2 ** 30 / per_set))
    sets = []
    for i in range(nsets):
        g = torch.Generator(device=dev)
        g.manual_seed(880000 + i)
        sets.append([torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
                     for shape in ((b, N, c["Hq"], c["D"]), (b, c["Hkv"], cap, c["D"]),
                                   (b, c["Hkv"], cap, c["D"]))])
    ws = torch.empty(tv.attention_workspace(b, N, c["Hq"], c["Hkv"], c["D"], L),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((b, N, c["Hq"], c["D"]), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, N, c["Hq"]), dtype=torch.float32, device=dev)

    def timed(hook):
        # hook: the library also records events just before the partial
        # kernel and between the two kernels (extra markers; see above)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        for e in evs:
            e[1].record(stream)
            e[3].record(stream)
        torch.cuda.synchronize()
        for i in range(reps + 5):
            q, k, v = sets[i % nsets]
            if i >= 5:
                evs[i - 5][0].record(stream)
                if hook:
                    tv.lib().tv_debug_set_attention_events(evs[i - 5][3].cuda_event,
                                                           evs[i - 5][1].cuda_event)
            tv.tv_tree_attention_verify(q, k, v, ctx, tree["anc"], tree["n_nodes"], L,
                                        workspace=ws, out=out, lse=lse)
            if i >= 5:
                if hook:
                    tv.lib().tv_debug_set_attention_events(None, None)
                evs[i - 5][2].record(stream)
        torch.cuda.synchronize()
        return evs

    evs = timed(False)
    call = sum(e[0].elapsed_time(e[2]) for e in evs) / reps
    evs = timed(True)
    part = sum(e[3].elapsed_time(e[1]) for e in evs) / reps
    comb = sum(e[1].elapsed_time(e[2]) for e in evs) / reps
    flops = attention_flops(c, tree["n_nodes"].cpu().numpy(), tree["depth"].cpu().numpy(),
                            ctx.cpu().numpy())
    byts = algorithmic_bytes(c, b, N, L, False)["attention"]

    def tf(ms):
        return flops / (ms * 1e-3) / 1e12

    return dict(ms=round(call, 5), algorithmic_MB=round(byts / 1e6, 3),
                GBps=round(byts / (call * 1e-3) / 1e9, 1), GFLOP=round(flops / 1e9, 3),
                TFLOPs=round(tf(call), 2), mfma_frac=round(tf(call) / MFMA_BF16_PEAK_TFLOPS, 4),
                kernel_ms={"k_attn_partial": round(part, 5), "k_attn_combine": round(comb, 5)},
                kernel_TFLOPs=round(tf(part), 2),
                kernel_mfma_frac=round(tf(part) / MFMA_BF16_PEAK_TFLOPS, 4),
                input_sets=nsets, nodes=int(tree["n_nodes"][0].item()))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import tree_verification_best_amd as tv
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    c = dict(workloads.CONFIGS[args.workload])
    c["_T"] = args.temperature
    b, N, V, K = c["batch"], c["B"] + 1, c["V"], c["K"]
    bf = c["dtype"] == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32

    # ---- input sets ------------------------------------------------------
    def make_set(salt):
        draft, target = workloads.logits(c, b, N, salt=salt)
        roots = workloads.root_tokens(c, b, salt=salt)
        ctx = workloads.context_lengths(c, b, salt=0)
        cap = int(ctx.max()) + N
        q, k, v = workloads.qkv(c, b, N, cap, salt=salt)
        return draft, target, q, k, v, roots, ctx

    first = make_set(0)
    per_set = sum(a.nbytes for a in first[:2]) + sum(a.nbytes // (2 if bf else 1)
                                                      for a in first[2:5])
    nsets = max(2, math.ceil(args.rotate_gib * 2 ** 30 / per_set))
    tree_in = None
    if not c["build"]:
        parent, token, depth = workloads.random_trees(c, b, N, max_depth=K,
                                                      max_children=c.get("max_children", 4))
        nn = np.full(b, N, np.int32)
        c["_tree"] = (parent, token, depth, nn)
        first = (first[0], workloads.plant(first[1], parent, token, nn, 9.0)) + first[2:]
        tree_in = [torch.from_numpy(a).to(dev) for a in (parent, token, nn)]

    def to_dev(s):
        draft, target, q, k, v, roots, ctx = s
        # logits stay fp32 (4 bytes per element); Q/K/V use the layer's dtype
        return dict(draft=torch.from_numpy(draft).to(dev), target=torch.from_numpy(target).to(dev),
                    q=torch.from_numpy(q).to(dev, tdt), k=torch.from_numpy(k).to(dev, tdt),
                    v=torch.from_numpy(v).to(dev, tdt), roots=torch.from_numpy(roots).to(dev),
                    ctx=torch.from_numpy(ctx).to(dev))

    sets = [to_dev(first)]
    for i in range(1, nsets):
        s = make_set(i)
        if not c["build"]:
            s = (s[0], workloads.plant(s[1], *c["_tree"][:2], c["_tree"][3], 9.0)) + s[2:]
        sets.append(to_dev(s))
    ctx0 = first[6]
    max_ctx = int(ctx0.max())

    # ---- preallocated outputs and workspaces -----------------------------
    W = (N + 63) // 64
    i32 = dict(dtype=torch.int32, device=dev)
    tree = dict(parent=torch.empty((b, N), **i32), token=torch.empty((b, N), **i32),
                depth=torch.empty((b, N), **i32), pos=torch.empty((b, N), **i32),
                score=torch.empty((b, N), dtype=torch.float64, device=dev),
                anc=torch.empty((b, N, W), dtype=torch.int64, device=dev),
                n_nodes=torch.empty((b,), **i32))
    sampled = args.temperature > 0
    mode = tv.TV_SAMPLED if sampled else tv.TV_GREEDY
    ws_b = torch.empty(max(tv.tree_build_workspace(b, K, V, c["k"], c["B"]), 1), dtype=torch.uint8, device=dev) if c["build"] else None
    ws_a = torch.empty(tv.attention_workspace(b, N, c["Hq"], c["Hkv"], c["D"], max_ctx), dtype=torch.uint8, device=dev)
    ws_c = torch.zeros(tv.accept_workspace(b, N, K, V, mode), dtype=torch.uint8, device=dev)
    attn_out = torch.empty((b, N, c["Hq"], c["D"]), dtype=tdt, device=dev)
    lse = torch.empty((b, N, c["Hq"]), dtype=torch.float32, device=dev)
    acc = dict(accept_len=torch.empty((b,), **i32), accepted_nodes=torch.empty((b, K + 1), **i32),
               out_tokens=torch.empty((b, K + 1), **i32))
    new_ctx = torch.empty((b,), **i32)
    if not c["build"]:
        tree["parent"].copy_(tree_in[0])
        tree["token"].copy_(tree_in[1])
        tree["n_nodes"].copy_(tree_in[2])

    stream = torch.cuda.current_stream(dev)

    def round_(step, ev=None, hk=None):
        s = sets[step % nsets]
        if ev is not None:
            ev[0].record(stream)
        if c["build"]:
            tv.tv_tree_build(s["draft"], c["k"], c["B"], s["roots"], s["ctx"], workspace=ws_b, out=tree)
        else:
            tv.tv_tree_ancestors(tree["parent"], tree["n_nodes"], s["ctx"],
                                 out=dict(depth=tree["depth"], pos=tree["pos"], anc=tree["anc"]))
        if ev is not None:
            ev[1].record(stream)
        if hk is not None:
            tv.lib().tv_debug_set_attention_events(hk[0].cuda_event, hk[1].cuda_event)
        tv.tv_tree_attention_verify(s["q"], s["k"], s["v"], s["ctx"], tree["anc"], tree["n_nodes"],
                                    max_ctx, workspace=ws_a, out=attn_out, lse=lse)
        if hk is not None:
            tv.lib().tv_debug_set_attention_events(None, None)
        if ev is not None:
            ev[2].record(stream)
        tv.tv_tree_accept(s["target"], tree["parent"], tree["token"], tree["depth"], tree["n_nodes"],
                          mode=mode, temperature=max(args.temperature, 1e-3), seed=1234, round=step,
                          max_depth=K, workspace=ws_c, out=acc)
        if ev is not None:
            ev[3].record(stream)

    def commit_(step):
        # the accepted path's K/V rows move behind the context (in place; the
        # input set's context lengths are kept, so every call sees the same shapes)
        s = sets[step % nsets]
        tv.tv_kv_commit(s["k"], s["v"], s["ctx"], acc["accept_len"], acc["accepted_nodes"],
                        new_ctx_len=new_ctx)

    # every timed eager step adds its accept lengths on the device (after the
    # step's last event, so outside the per-call brackets)
    acc_sum = torch.zeros((b,), dtype=torch.int64, device=dev)

    def eager_steps(first, n, evs=None, hks=None):
        for i in range(n):
            round_(first + i, evs[i] if evs is not None else None,
                   hks[i] if hks is not None else None)
            if evs is not None and hks is None:
                acc_sum.add_(acc["accept_len"])

    for i in range(args.warmup):
        round_(i)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    graph_ms = None
    batch_ms = []
    wall = 0.0
    if not args.eager:
        # the timed region: replays of the round captured once per input set
        # (launches only; the calls allocate nothing and set no memory)
        graphs = []
        for i in range(nsets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                round_(i)
            graphs.append(g)
        for i in range(min(args.warmup, 2 * nsets)):
            graphs[i % nsets].replay()
        torch.cuda.synchronize()
        # five equal batches of the K steps, each bracketed by events (the
        # events add no work): their median is reported beside the mean
        nb = 5 if args.steps >= 5 else 1
        edges = [round(j * args.steps / nb) for j in range(nb + 1)]
        bev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
        t0 = time.perf_counter()
        start.record(stream)
        for j in range(nb):
            bev[j].record(stream)
            for i in range(edges[j], edges[j + 1]):
                graphs[i % nsets].replay()
        bev[nb].record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
        graph_ms = start.elapsed_time(end) / args.steps
        batch_ms = [bev[j].elapsed_time(bev[j + 1]) / (edges[j + 1] - edges[j]) for j in range(nb)]

    # eager launches of the same steps with HIP events around every call on
    # the stream the calls run on (events cannot be recorded inside a graph
    # on this platform): the per-call times and the roofline come from here
    # evs[i]: before build, after build, after attention, after accept
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    eager_steps(args.warmup, args.steps, evs)
    end.record(stream)
    torch.cuda.synchronize()
    wall += time.perf_counter() - t0
    eager_ms = start.elapsed_time(end) / args.steps
    ms_per_step = graph_ms if graph_ms is not None else eager_ms

    calls = {}
    for name, (a, z) in (("build", (0, 1)), ("attention", (1, 2)), ("accept", (2, 3))):
        calls[name] = sum(evs[i][a].elapsed_time(evs[i][z]) for i in range(args.steps)) / args.steps
    kern = {}
    if bf:
        # a second eager pass of the same steps in which the library records
        # an event just before the partial kernel and one between it and the
        # combine (its timing hook; every event recorded once beforehand so
        # that it exists before its handle is passed on): the partial kernel
        # is timed between those two, the combine to the event after the
        # call.  The extra markers lengthen the call, so the per-call times
        # above come from the pass without them.
        hks = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        evs2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for h in hks:
            h[0].record(stream)
            h[1].record(stream)
        torch.cuda.synchronize()
        eager_steps(args.warmup, args.steps, evs2, hks)
        torch.cuda.synchronize()
        kern["k_attn_partial"] = sum(hks[i][0].elapsed_time(hks[i][1])
                                     for i in range(args.steps)) / args.steps
        kern["k_attn_combine"] = sum(hks[i][1].elapsed_time(evs2[i][2])
                                     for i in range(args.steps)) / args.steps
    mean_accept = float(acc_sum.sum().item()) / (args.steps * b)
    sweep = {}
    att8 = None
    if not args.round_only:
        # verification with the rotary embedding fused (queries and tree keys
        # turned at the tree's position ids), per call with events like the plain
        # call, over the same input sets and the last step's tree
        nrope = min(args.steps, 100)
        rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nrope)]
        for i in range(nrope + 5):
            s = sets[i % nsets]
            if i >= 5:
                rev[i - 5][0].record(stream)
            tv.tv_tree_attention_verify(s["q"], s["k"], s["v"], s["ctx"], tree["anc"], tree["n_nodes"],
                                        max_ctx, workspace=ws_a, out=attn_out, lse=lse,
                                        pos=tree["pos"], rope_base=ROPE_BASE)
            if i >= 5:
                rev[i - 5][1].record(stream)
        torch.cuda.synchronize()
        calls["attention_rope"] = sum(e[0].elapsed_time(e[1]) for e in rev) / nrope
        # the commit, outside the timed steps (acc holds the last step's walk).
        # One call is shorter than the host's launch path, so the calls are
        # captured into a graph and the replays timed, as device time.
        ncommit = 50
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            for i in range(ncommit):
                commit_(i)
        cg.replay()
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        reps = 4
        c0.record(stream)
        for _ in range(reps):
            cg.replay()
        c1.record(stream)
        torch.cuda.synchronize()
        calls["commit"] = c0.elapsed_time(c1) / (reps * ncommit)
        # verification time against the tree budget (the pages' time-vs-budget
        # figure): one sequence with this workload's heads, context 4096, random
        # trees of B + 1 nodes, per call with events
        sweep = b_sweep(c, dev, stream)
        if args.workload != "8b" and bf:
            att8 = attention_8b(dev, stream, args.rotate_gib)
        if c["build"]:
            # the cost-aware tree size over the last step's tree; the cost of n
            # draft nodes is the measured verification time, interpolated
            # between the sweep's budgets
            import numpy as np
            sb = sorted(sweep)
            cost_h = np.interp(np.arange(N), sb, [sweep[x] for x in sb])
            cost = torch.from_numpy(cost_h).to(dev)
            n_out = torch.empty((b,), **i32)
            bg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(bg):
                for _ in range(ncommit):
                    tv.tv_tree_budget(tree["score"], tree["n_nodes"], cost, n_nodes_out=n_out)
            bg.replay()
            torch.cuda.synchronize()
            c0.record(stream)
            for _ in range(reps):
                bg.replay()
            c1.record(stream)
            torch.cuda.synchronize()
            calls["budget"] = c0.elapsed_time(c1) / (reps * ncommit)
            # a layer-wise build of the same tree capacity: tv_tree_root, then K
            # drafting steps of tv_tree_expand at a frontier of EXPAND_W slots with
            # top-k children, on the drafter's next-token logits (the same dtype
            # as the draft marginals); per_call.expand is one step (the root
            # call's share included)
            xl = [torch.from_numpy(a).to(dev) for a in
                  workloads.expand_logits(dict(c, dtype="f32"), b, EXPAND_W, K)]
            xtree = {f: torch.empty_like(t) for f, t in tree.items()}
            front = torch.empty((b, EXPAND_W), **i32)
            nxt = torch.empty((b, EXPAND_W), **i32)
            ws_x = torch.empty(tv.tree_expand_workspace(b, EXPAND_W, V, c["k"]), dtype=torch.uint8,
                               device=dev)
            f0 = torch.full((b, EXPAND_W), -1, **i32)
            f0[:, 0] = 0

            def layerwise_():
                tv.tv_tree_root(sets[0]["roots"], sets[0]["ctx"], N, out=xtree)
                front.copy_(f0)
                for j in range(K):
                    tv.tv_tree_expand(xl[j], c["k"], front, xtree, sets[0]["ctx"],
                                      next_frontier=nxt, workspace=ws_x)
                    front.copy_(nxt)

            layerwise_()
            xg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(xg):
                layerwise_()
            xg.replay()
            torch.cuda.synchronize()
            c0.record(stream)
            for _ in range(reps):
                xg.replay()
            c1.record(stream)
            torch.cuda.synchronize()
            calls["expand"] = c0.elapsed_time(c1) / (reps * K)

    # ---- accounting ------------------------------------------------------
    nn_h = tree["n_nodes"].cpu().numpy()
    dep_h = tree["depth"].cpu().numpy()
    Lsum = int(ctx0.sum())
    abytes = algorithmic_bytes(c, b, N, Lsum, c["build"])
    # the commit reads and writes each accepted draft's K and V rows once
    # (the last step's accept lengths stand for the mean)
    el = 2 if c["dtype"] == "bf16" else 4
    moved = float(acc["accept_len"].clamp(min=0).sum().item())
    abytes["commit"] = int(2 * 2 * c["Hkv"] * c["D"] * el * moved)
    abytes["budget"] = b * N * 8 + N * 8 + b * 8   # scores and costs in, counts in and out
    abytes["attention_rope"] = abytes["attention"] + b * N * 4   # plus the position ids
    if "expand" in calls:
        # one drafting step reads the frontier's logit rows once and writes
        # up to EXPAND_W * k new rows (4 int32, one f64, the ancestor row)
        new_rows = min(EXPAND_W * c["k"], N - 1)
        abytes["expand"] = b * (EXPAND_W * V * 4 + new_rows * (16 + 8 + 8 * W) + EXPAND_W * 8)
    aflops = attention_flops(c, nn_h, dep_h, ctx0)
    rows = b * N * c["Hq"]
    rounds_per_s = 1e3 / ms_per_step
    value = rounds_per_s * rows
    roof = None
    per_call = {}
    for name, ms in calls.items():
        gbs = abytes[name] / (ms * 1e-3) / 1e9
        per_call[name] = dict(ms=round(ms, 5), algorithmic_MB=round(abytes[name] / 1e6, 3),
                              GBps=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
    for name in ("attention", "attention_rope"):
        if name in calls:
            tf = aflops / (calls[name] * 1e-3) / 1e12
            per_call[name]["TFLOPs"] = round(tf, 2)
            per_call[name]["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
    if att8 is not None:
        per_call["attention_8b"] = att8
    if "attention" in calls:
        # the verification pass: HBM-bound below the ridge point, else MFMA.
        # The dominant kernel is k_attn_partial: it reads every input of the
        # call once (K/V rows, Q, the ancestor rows); the combine writes O and
        # the lse.  achieved = its algorithmic bytes (or the call's flops) over
        # its own event-to-event time; the whole call's figure is beside it.
        ms = calls["attention"]
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        intensity = aflops / abytes["attention"]
        out_bytes = b * N * c["Hq"] * (c["D"] * el + 4)
        kbytes = abytes["attention"] - out_bytes
        kms = kern.get("k_attn_partial", ms)
        traffic = recorded_traffic(args.workload)
        hbm = intensity < ridge

        def fig(nbytes, t):
            if hbm:
                a = nbytes / (t * 1e-3) / 1e9
                return round(a, 1), round(a / HBM_PEAK_GBS, 4)
            a = aflops / (t * 1e-3) / 1e12
            return round(a, 2), round(a / MFMA_BF16_PEAK_TFLOPS, 4)

        ach, frac = fig(kbytes, kms)
        cach, cfrac = fig(abytes["attention"], ms)
        roof = {"bound": "hbm" if hbm else "mfma", "achieved": ach,
                "peak": HBM_PEAK_GBS if hbm else MFMA_BF16_PEAK_TFLOPS,
                "unit": "GB/s" if hbm else "TFLOP/s", "frac": frac, "traffic": traffic,
                "kernel": "k_attn_partial" if bf else "k_attn_f32", "kernel_ms": round(kms, 5),
                "kernel_algorithmic_bytes": kbytes,
                "call": {"name": "tv_tree_attention_verify", "ms": round(ms, 5),
                         "achieved": cach, "frac": cfrac,
                         "algorithmic_bytes": abytes["attention"],
                         "kernels_ms": {k: round(v, 5) for k, v in kern.items()}},
                "algorithmic_flops": aflops,
                "intensity_flop_per_byte": round(intensity, 1)}
        if bf:
            # the two kernels' bracketed times added: the partial between the
            # library's events, the combine from there to the event after the
            # call (the gap before the call left out)
            pair = kern["k_attn_partial"] + kern["k_attn_combine"]
            roof["call"]["kernels_frac"] = fig(abytes["attention"], pair)[1]

    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        model = cpu_model()
        r, dt = cpu_baseline(c, first, args.cpu_seconds, workers=1)
        cpu = {"value": round(r / dt * rows, 1), "unit": "node-heads/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{r} whole round(s) of the {args.workload} workload (input set 0), "
                         f"{dt:.1f} s, single thread (BLAS limited to 1), {model}"}
        # the same spread over the host cores this process may use, at most
        # 16 (one GPU's share of the host); `affinity_cores` is the uncapped
        # count
        affinity = len(os.sched_getaffinity(0))
        ncores = min(16, affinity)
        r, dt = cpu_baseline(c, first, args.cpu_seconds, workers=ncores)
        cpu_all = {"value": round(r / dt * rows, 1), "unit": "node-heads/s", "cores": ncores,
                   "affinity_cores": affinity, "kind": "oracle",
                   "sample": f"{r} whole round(s), {dt:.1f} s, {ncores} workers (draft "
                             f"positions on OpenMP threads, attention rows on processes), "
                             f"BLAS 1 thread each"}

    res = {
        "metric": "verify rounds/s as tree node x query-head rows verified per second",
        "value": round(value, 1),
        "unit": "node-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 attention / f32 logits / u64 weights",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {c['Hq']}q/{c['Hkv']}kv heads, D={c['D']}, "
                               f"{c['dtype']}, batch {b}, ctx {c['L']}, K={K}, top-{c['k']}, "
                               f"B={c['B']}, V={V}, T={args.temperature}",
                   "rounds_per_s": round(rounds_per_s, 2), "nodes": N,
                   "input_sets": nsets, "graph": not args.eager,
                   "eager_ms_per_step": round(eager_ms, 5),
                   "batch_ms": [round(x, 5) for x in batch_ms],
                   "batch_ms_median": round(sorted(batch_ms)[len(batch_ms) // 2], 5) if batch_ms else None,
                   "round_algorithmic_MB": round(sum(abytes[n] for n in ("build", "attention", "accept")
                                                     if n in abytes) / 1e6, 2),
                   "attention_GFLOP": round(aflops / 1e9, 3),
                   "mean_accept_len": round(mean_accept, 4),
                   "accept_len_samples": args.steps * b,
                   "per_call": per_call, "wall_s": round(wall, 3),
                   "b_sweep_ms": {str(k): round(v, 5) for k, v in sweep.items()},
                   "cpu_all_cores": cpu_all},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
