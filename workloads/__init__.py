"""Seeded synthetic inputs for one tree-verification round.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle are fed from it.

Shapes follow the workloads of the pages (TAPS sec. 3.1 and Fig. 3: Qwen3-4B /
8B class targets, node budgets 64..512, per-position top-K marginals from a
diffusion drafter); the concrete sizes are the five configurations below.
The pages name no public dataset for this path; these seeded draws stand in
for the drafter's marginals, the target's logits and the KV cache.

Distributions:
  * Q, K, V ~ N(0, 1), rounded to bf16 (fp32 for the tiny configuration).
  * Draft / target logits, per sequence: base rows beta0, beta1 ~ N(0, sigma^2);
    target row 0 (the root) = beta0 + 0.25 e, target rows i >= 1 =
    beta1 + 0.25 e_i; draft row 1 = beta0 + N(0, 1); draft rows j >= 2 =
    beta1 + N(0, 1).  So the drafter's marginal at each position is the
    target's distribution plus unit noise, as the configurations ask
    ("draft = target + N(0,1)"), without the generator knowing the tree.
    The tiny configuration draws draft and target rows i.i.d. N(0, 2^2).
  * Random trees (batched configuration): node i >= 1 takes a uniform parent
    among earlier nodes of depth < max_depth with fewer than max_children
    children; tokens are uniform; the parent's target row is raised by
    `plant` at the child's token, so that walks go past the root.
  * Layer-wise drafting (one call per drafting step): the drafter's
    next-token rows at the W frontier slots are beta + N(0, 1) with one
    beta ~ N(0, sigma^2) per sequence, shared by all steps and slots, so the
    top-m sets of different slots overlap as those of one context do.
  * sigma in "N(0, sigma)" is read as the standard deviation.
"""
import numpy as np

CONFIGS = {
    "tiny": dict(name="tiny", batch=1, Hq=1, Hkv=1, D=64, dtype="f32", L=128, K=4, k=4,
                 B=16, V=1000, sigma=2.0, temperatures=(0.0, 1.0), build=True),
    "4b": dict(name="4b", batch=1, Hq=32, Hkv=8, D=128, dtype="bf16", L=4096, K=16, k=8,
               B=64, V=151936, sigma=3.0, temperatures=(0.0, 1.0), build=True),
    "8b": dict(name="8b", batch=1, Hq=32, Hkv=8, D=128, dtype="bf16", L=8192, K=16, k=16,
               B=256, V=151936, sigma=3.0, temperatures=(1.0,), build=True),
    "batched": dict(name="batched", batch=16, Hq=32, Hkv=8, D=128, dtype="bf16",
                    L=(1024, 8192), K=16, k=4, B=32, V=151936, sigma=3.0,
                    temperatures=(0.0, 1.0), build=False, max_children=4),
    "long": dict(name="long", batch=1, Hq=32, Hkv=8, D=128, dtype="bf16", L=32768, K=32,
                 k=16, B=512, V=151936, sigma=3.0, temperatures=(0.0, 1.0), build=True),
}
SEED_BASE = 20260000
CONFIG_INDEX = {"tiny": 1, "4b": 2, "8b": 3, "batched": 4, "long": 5}


def rng(cfg_name, stream, salt=0):
    """Independent Philox stream per (configuration, tensor, salt)."""
    ss = np.random.SeedSequence([SEED_BASE + CONFIG_INDEX.get(cfg_name, 0), stream, salt])
    return np.random.Generator(np.random.Philox(ss))


STREAM_DRAFT, STREAM_TARGET, STREAM_Q, STREAM_K, STREAM_V, STREAM_TREE, STREAM_CTX, \
    STREAM_ROOT, STREAM_EXPAND = range(9)


def round_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    (torch's CPU conversion, multi-threaded, for the large caches)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def logits(cfg, batch, N, salt=0):
    """(draft [b][K][V], target [b][N][V]) float32 logits."""
    K, V, sig = cfg["K"], cfg["V"], cfg["sigma"]
    r = rng(cfg["name"], STREAM_DRAFT, salt)
    if cfg["name"] == "tiny":
        draft = r.standard_normal((batch, K, V), dtype=np.float32) * np.float32(sig)
        target = r.standard_normal((batch, N, V), dtype=np.float32) * np.float32(sig)
        return draft, target
    draft = np.empty((batch, K, V), np.float32)
    target = np.empty((batch, N, V), np.float32)
    for b in range(batch):
        beta0 = r.standard_normal(V, dtype=np.float32) * np.float32(sig)
        beta1 = r.standard_normal(V, dtype=np.float32) * np.float32(sig)
        target[b, 0] = beta0 + np.float32(0.25) * r.standard_normal(V, dtype=np.float32)
        for i in range(1, N):
            target[b, i] = beta1 + np.float32(0.25) * r.standard_normal(V, dtype=np.float32)
        draft[b, 0] = beta0 + r.standard_normal(V, dtype=np.float32)
        for j in range(1, K):
            draft[b, j] = beta1 + r.standard_normal(V, dtype=np.float32)
    return draft, target


def context_lengths(cfg, batch, salt=0):
    L = cfg["L"]
    if isinstance(L, tuple):
        r = rng(cfg["name"], STREAM_CTX, salt)
        return r.integers(L[0], L[1] + 1, size=batch).astype(np.int32)
    return np.full(batch, L, np.int32)


def root_tokens(cfg, batch, salt=0):
    r = rng(cfg["name"], STREAM_ROOT, salt)
    return r.integers(0, cfg["V"], size=batch).astype(np.int32)


def qkv(cfg, batch, N, cap, salt=0, dtype=None):
    """Q [b][N][Hq][D], K/V caches [b][Hkv][cap][D] as float32 arrays holding
    bf16-representable values (or plain fp32 for the fp32 configuration)."""
    dtype = dtype or cfg["dtype"]
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    q = rng(cfg["name"], STREAM_Q, salt).standard_normal((batch, N, Hq, D), dtype=np.float32)
    k = rng(cfg["name"], STREAM_K, salt).standard_normal((batch, Hkv, cap, D), dtype=np.float32)
    v = rng(cfg["name"], STREAM_V, salt).standard_normal((batch, Hkv, cap, D), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def random_trees(cfg, batch, N, salt=0, max_depth=16, max_children=4):
    """Random parent arrays [b][N] (parent[i] < i, root 0) and uniform tokens.

    Also returns each node's depth, which the generator tracks to respect the
    depth limit (it is the node's distance from the root)."""
    r = rng(cfg["name"], STREAM_TREE, salt)
    V = cfg["V"]
    parent = np.full((batch, N), -1, np.int32)
    depth = np.zeros((batch, N), np.int32)
    token = r.integers(0, V, size=(batch, N)).astype(np.int32)
    for b in range(batch):
        nkids = np.zeros(N, np.int64)
        for i in range(1, N):
            ok = [p for p in range(i) if depth[b, p] < max_depth and nkids[p] < max_children]
            p = ok[int(r.integers(0, len(ok)))]
            parent[b, i] = p
            depth[b, i] = depth[b, p] + 1
            nkids[p] += 1
    return parent, token, depth


def plant(target, parent, token, n_nodes, boost):
    """Raise each parent's target logit at its children's tokens by `boost`."""
    out = target.copy()
    b = target.shape[0]
    for s in range(b):
        for i in range(1, int(n_nodes[s])):
            p = parent[s, i]
            if p >= 0:
                out[s, p, token[s, i]] += np.float32(boost)
    return out


def expand_logits(cfg, batch, W, steps, salt=0):
    """Drafter next-token logits for `steps` layer-wise drafting steps:
    list of float32 [b][W][V] (bf16-representable for bf16 configurations)."""
    V, sig = cfg["V"], cfg["sigma"]
    r = rng(cfg["name"], STREAM_EXPAND, salt)
    beta = r.standard_normal((batch, 1, V), dtype=np.float32) * np.float32(sig)
    out = []
    for _ in range(steps):
        x = beta + r.standard_normal((batch, W, V), dtype=np.float32)
        out.append(round_bf16(x) if cfg["dtype"] == "bf16" else x)
    return out
