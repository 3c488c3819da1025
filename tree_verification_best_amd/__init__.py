"""tree_verification_best_amd -- one tree-verification round of speculative
decoding on an AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libtreeverify.so`` (C ABI in
``include/treeverify.h``).  Every step of the round runs in the library's HIP
kernels; this module only checks tensors, allocates outputs and workspaces
with torch and passes device pointers and the current HIP stream.  There is
no CPU fallback: if the library is missing or no GPU is present the calls
raise.

    tv_tree_build            draft marginals -> prefix-closed draft tree
    tv_tree_ancestors        depth / positions / ancestor rows of a parent array
    tv_tree_check            structural check of a caller-supplied tree
    tv_tree_attention_verify tree-masked GQA attention over context + tree
    tv_tree_accept           greedy or sampled acceptance walk
    tv_tree_root             a root-only tree (start of a layer-wise build)
    tv_tree_expand           one drafting step of a layer-wise (Top_W) builder
    tv_tree_budget           cost-aware tree size (best-first prefix)
    tv_kv_commit             keep the accepted path in the KV cache
    tv_tree_attention_verify_rope / tv_kv_commit_rope
                             the same with the rotary embedding at the tree's
                             position ids (pos / rope_base arguments)
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(_HERE, "libtreeverify.so")

TV_OK, TV_ERR_INVALID, TV_ERR_UNSUPPORTED, TV_ERR_WORKSPACE, TV_ERR_DEVICE = range(5)
TV_F32, TV_BF16 = 0, 1
TV_GREEDY, TV_SAMPLED = 0, 1
TV_PROPOSAL_POINT_MASS, TV_PROPOSAL_DRAFT = 0, 1

EXPORTS = ("tv_status_string", "tv_version", "tv_tree_build_workspace", "tv_tree_build",
           "tv_tree_ancestors", "tv_tree_attention_workspace", "tv_tree_attention_verify",
           "tv_tree_accept_workspace", "tv_tree_accept", "tv_tree_budget", "tv_kv_commit",
           "tv_tree_root", "tv_tree_expand_workspace", "tv_tree_expand",
           "tv_tree_attention_verify_rope", "tv_kv_commit_rope", "tv_tree_check",
           "tv_debug_set_spin_limit", "tv_tree_build_noalloc", "tv_debug_set_attention_events",
           "tv_debug_weights")

_lib = None


class TreeVerifyError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _load().tv_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg}")


def _load():
    """Load libtreeverify.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBPATH):
        raise ImportError(f"{LIBPATH} is missing: run `python -m tree_verification_best_amd.build`")
    L = ctypes.CDLL(LIBPATH)
    c = ctypes
    vp, i32, f32, sz, u64 = c.c_void_p, c.c_int, c.c_float, c.c_size_t, c.c_uint64
    L.tv_status_string.argtypes = [i32]
    L.tv_status_string.restype = c.c_char_p
    L.tv_version.argtypes = []
    L.tv_version.restype = i32
    L.tv_debug_set_spin_limit.argtypes = [i32]
    L.tv_debug_set_spin_limit.restype = i32
    L.tv_tree_build_workspace.argtypes = [i32, i32, i32, i32, i32]
    L.tv_tree_build_workspace.restype = sz
    L.tv_tree_build.argtypes = [vp, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp,
                                vp, vp, vp, vp, sz, vp]
    L.tv_tree_build.restype = i32
    L.tv_debug_weights.argtypes = [c.c_uint32, c.c_uint32, f32, f32, i32, vp, vp]
    L.tv_debug_weights.restype = i32
    L.tv_debug_set_attention_events.argtypes = [vp, vp]
    L.tv_debug_set_attention_events.restype = i32
    L.tv_tree_build_noalloc.argtypes = [vp, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, vp]
    L.tv_tree_build_noalloc.restype = i32
    L.tv_tree_ancestors.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp]
    L.tv_tree_ancestors.restype = i32
    L.tv_tree_attention_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.tv_tree_attention_workspace.restype = sz
    L.tv_tree_attention_verify.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                           i32, i32, i32, f32, i32, vp, i32, vp, vp, sz, vp]
    L.tv_tree_attention_verify.restype = i32
    L.tv_tree_accept_workspace.argtypes = [i32, i32, i32, i32, i32, i32]
    L.tv_tree_accept_workspace.restype = sz
    L.tv_tree_accept.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, f32, i32,
                                 u64, u64, i32, vp, vp, vp, vp, sz, vp]
    L.tv_tree_accept.restype = i32
    L.tv_tree_budget.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
    L.tv_tree_budget.restype = i32
    L.tv_kv_commit.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]
    L.tv_kv_commit.restype = i32
    L.tv_tree_attention_verify_rope.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, c.c_double, i32,
                                                i32, i32, i32, i32, i32, i32, f32, i32, vp, i32,
                                                vp, vp, sz, vp]
    L.tv_tree_attention_verify_rope.restype = i32
    L.tv_kv_commit_rope.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, i32, c.c_double,
                                    vp, vp]
    L.tv_kv_commit_rope.restype = i32
    L.tv_tree_check.argtypes = [vp, vp, vp, i32, i32, vp, vp]
    L.tv_tree_check.restype = i32
    L.tv_tree_root.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.tv_tree_root.restype = i32
    L.tv_tree_expand_workspace.argtypes = [i32, i32, i32, i32]
    L.tv_tree_expand_workspace.restype = sz
    L.tv_tree_expand.argtypes = [vp, i32, i32, i32, i32, i32, f32, vp, vp, i32, vp, vp, vp, vp,
                                 vp, vp, vp, vp, vp, sz, vp]
    L.tv_tree_expand.restype = i32
    _lib = L
    return L


def lib():
    return _load()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _dt(t):
    if t.dtype == torch.float32:
        return TV_F32
    if t.dtype == torch.bfloat16:
        return TV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check(status, where):
    if status != TV_OK:
        raise TreeVerifyError(status, where)


def _workspace(nbytes, device, workspace, zero=False):
    """The caller's workspace, or a new one (zero-filled where the call needs
    zeros in a new workspace)."""
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace, workspace.numel() * workspace.element_size()
    make = torch.zeros if zero else torch.empty
    buf = make(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    return buf, buf.numel()


# --------------------------------------------------------------------------
# the four calls
# --------------------------------------------------------------------------
def tree_build_workspace(batch, K, V, topk, budget):
    return _load().tv_tree_build_workspace(batch, K, V, topk, budget)


def _tree_out(b, N, dev):
    W = (N + 63) // 64
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(parent=torch.empty((b, N), **i32), token=torch.empty((b, N), **i32),
                depth=torch.empty((b, N), **i32), pos=torch.empty((b, N), **i32),
                score=torch.empty((b, N), dtype=torch.float64, device=dev),
                anc=torch.empty((b, N, W), dtype=torch.int64, device=dev),
                n_nodes=torch.empty((b,), **i32))


def tv_tree_build(draft_logits, topk, budget, root_token, ctx_len, build_temp=1.0,
                  workspace=None, out=None):
    """draft_logits [b][K][V] (f32/bf16) -> dict of tree tensors [b][budget+1]."""
    L = _load()
    b, K, V = draft_logits.shape
    dev = draft_logits.device
    if out is None:
        out = _tree_out(b, budget + 1, dev)
    need = L.tv_tree_build_workspace(b, K, V, topk, budget)
    ws, wsb = _workspace(need, dev, workspace)
    st = L.tv_tree_build(_dev(draft_logits, "draft_logits"), _dt(draft_logits), b, K, V, topk,
                         budget, float(build_temp), _dev(root_token, "root_token", torch.int32),
                         _dev(ctx_len, "ctx_len", torch.int32), _dev(out["parent"], "parent"),
                         _dev(out["token"], "token"), _dev(out["depth"], "depth"),
                         _dev(out["pos"], "pos"), _dev(out["score"], "score"),
                         _dev(out["anc"], "anc"), _dev(out["n_nodes"], "n_nodes"),
                         ws.data_ptr(), wsb, _stream(dev))
    _check(st, "tv_tree_build")
    return out


def tv_tree_build_noalloc(draft_logits, topk, budget, root_token, ctx_len, build_temp=1.0,
                          out=None):
    """tv_tree_build on the library's static scratch: no workspace argument
    and no device allocation when `out` is given."""
    L = _load()
    b, K, V = draft_logits.shape
    if out is None:
        out = _tree_out(b, budget + 1, draft_logits.device)
    st = L.tv_tree_build_noalloc(_dev(draft_logits, "draft_logits"), _dt(draft_logits), b, K, V,
                                 topk, budget, float(build_temp),
                                 _dev(root_token, "root_token", torch.int32),
                                 _dev(ctx_len, "ctx_len", torch.int32),
                                 _dev(out["parent"], "parent"), _dev(out["token"], "token"),
                                 _dev(out["depth"], "depth"), _dev(out["pos"], "pos"),
                                 _dev(out["score"], "score"), _dev(out["anc"], "anc"),
                                 _dev(out["n_nodes"], "n_nodes"), _stream(draft_logits.device))
    _check(st, "tv_tree_build_noalloc")
    return out


def tv_tree_ancestors(parent, n_nodes, ctx_len, out=None):
    L = _load()
    b, N = parent.shape
    dev = parent.device
    W = (N + 63) // 64
    if out is None:
        out = dict(depth=torch.empty((b, N), dtype=torch.int32, device=dev),
                   pos=torch.empty((b, N), dtype=torch.int32, device=dev),
                   anc=torch.empty((b, N, W), dtype=torch.int64, device=dev))
    st = L.tv_tree_ancestors(_dev(parent, "parent", torch.int32),
                             _dev(n_nodes, "n_nodes", torch.int32),
                             _dev(ctx_len, "ctx_len", torch.int32), b, N,
                             _dev(out["depth"], "depth"), _dev(out["pos"], "pos"),
                             _dev(out["anc"], "anc"), _stream(dev))
    _check(st, "tv_tree_ancestors")
    return out


def attention_workspace(batch, N, Hq, Hkv, D, max_ctx, splits=0):
    return _load().tv_tree_attention_workspace(batch, N, Hq, Hkv, D, max_ctx, splits)


def tv_tree_attention_verify(q, k_cache, v_cache, ctx_len, anc_mask, n_nodes, max_ctx,
                             scale=None, splits=0, want_lse=True, workspace=None, out=None,
                             lse=None, out_dtype=torch.float32, pos=None, rope_base=None):
    """q [b][N][Hq][D]; caches [b][Hkv][cap][D] -> (out [b][N][Hq][D], lse [b][N][Hq]).

    out is fp32 by default (the accumulated result); bf16 inputs may ask for
    out_dtype=torch.bfloat16.  With pos [b][N] and rope_base the call is
    tv_tree_attention_verify_rope (queries and tree keys rotated at pos)."""
    L = _load()
    b, N, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((b, N, Hq), dtype=torch.float32, device=dev)
    need = L.tv_tree_attention_workspace(b, N, Hq, Hkv, D, int(max_ctx), int(splits))
    ws, wsb = _workspace(need, dev, workspace)
    head = (_dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
            _dt(q), _dev(ctx_len, "ctx_len", torch.int32), _dev(anc_mask, "anc_mask", torch.int64),
            _dev(n_nodes, "n_nodes", torch.int32))
    tail = (b, N, Hq, Hkv, D, cap, int(max_ctx), scale, int(splits), _dev(out, "out"), _dt(out),
            _dev(lse, "lse", torch.float32) if lse is not None else None, ws.data_ptr(), wsb,
            _stream(dev))
    if pos is None:
        if rope_base is not None:
            raise ValueError("rope_base needs pos")
        st = L.tv_tree_attention_verify(*head, *tail)
        _check(st, "tv_tree_attention_verify")
    else:
        if rope_base is None:
            raise ValueError("pos needs rope_base")
        if tuple(pos.shape) != (b, N):
            raise ValueError("pos must be [b][N]")
        st = L.tv_tree_attention_verify_rope(*head, _dev(pos, "pos", torch.int32),
                                             float(rope_base), *tail)
        _check(st, "tv_tree_attention_verify_rope")
    return out, lse


def accept_workspace(batch, N, K, V, mode, proposal=TV_PROPOSAL_POINT_MASS):
    return _load().tv_tree_accept_workspace(batch, N, K, V, mode, proposal)


def tv_tree_accept(target_logits, parent, token, depth, n_nodes, *, mode, max_depth,
                   temperature=1.0, proposal=TV_PROPOSAL_POINT_MASS, seed=0, round=0,
                   draft_logits=None, workspace=None, out=None):
    """target_logits [b][N][V] -> dict(accept_len [b], accepted_nodes, out_tokens [b][max_depth+1])."""
    L = _load()
    b, N, V = target_logits.shape
    dev = target_logits.device
    K = draft_logits.shape[1] if draft_logits is not None else 0
    width = max_depth + 1
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(accept_len=torch.empty((b,), **i32),
                   accepted_nodes=torch.empty((b, width), **i32),
                   out_tokens=torch.empty((b, width), **i32))
    need = L.tv_tree_accept_workspace(b, N, max(K, 1), V, mode, proposal)
    ws, wsb = _workspace(need, dev, workspace, zero=mode == TV_SAMPLED)
    dptr = _dev(draft_logits, "draft_logits", target_logits.dtype) if draft_logits is not None else None
    st = L.tv_tree_accept(_dev(target_logits, "target_logits"), dptr, _dt(target_logits), b, N,
                          K, V, _dev(parent, "parent", torch.int32),
                          _dev(token, "token", torch.int32), _dev(depth, "depth", torch.int32),
                          _dev(n_nodes, "n_nodes", torch.int32), int(mode), float(temperature),
                          int(proposal), int(seed) & (2 ** 64 - 1), int(round) & (2 ** 64 - 1),
                          int(max_depth), _dev(out["accept_len"], "accept_len"),
                          _dev(out["accepted_nodes"], "accepted_nodes"),
                          _dev(out["out_tokens"], "out_tokens"), ws.data_ptr(), wsb,
                          _stream(dev))
    _check(st, "tv_tree_accept")
    return out


def tv_kv_commit(k_cache, v_cache, ctx_len, accept_len, accepted_nodes, new_ctx_len=None,
                 rope_base=None):
    """Moves the accepted path's K/V rows behind the context, in place; returns
    new_ctx_len [b] (a new tensor unless one is given; ctx_len itself may be).
    With rope_base the call is tv_kv_commit_rope (kept keys rotated at the
    rows they land on)."""
    L = _load()
    b, Hkv, cap, D = k_cache.shape
    if new_ctx_len is None:
        new_ctx_len = torch.empty((b,), dtype=torch.int32, device=k_cache.device)
    head = (_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache", k_cache.dtype), _dt(k_cache), b,
            Hkv, cap, D, _dev(ctx_len, "ctx_len", torch.int32),
            _dev(accept_len, "accept_len", torch.int32),
            _dev(accepted_nodes, "accepted_nodes", torch.int32), accepted_nodes.shape[1])
    tail = (_dev(new_ctx_len, "new_ctx_len", torch.int32), _stream(k_cache.device))
    if rope_base is None:
        st = L.tv_kv_commit(*head, *tail)
        _check(st, "tv_kv_commit")
    else:
        st = L.tv_kv_commit_rope(*head, float(rope_base), *tail)
        _check(st, "tv_kv_commit_rope")
    return new_ctx_len


def tv_tree_budget(score, n_nodes, cost, n_nodes_out=None):
    """score [b][N] f64, n_nodes [b], cost [>= N] f64 -> n_nodes_out [b] (the
    best-first prefix maximising (1 + S_n) / cost[n], plus the root)."""
    L = _load()
    b, N = score.shape
    if n_nodes_out is None:
        n_nodes_out = torch.empty((b,), dtype=torch.int32, device=score.device)
    st = L.tv_tree_budget(_dev(score, "score", torch.float64), _dev(n_nodes, "n_nodes", torch.int32),
                          _dev(cost, "cost", torch.float64), b, N, cost.numel(),
                          _dev(n_nodes_out, "n_nodes_out", torch.int32), _stream(score.device))
    _check(st, "tv_tree_budget")
    return n_nodes_out


def tv_tree_check(parent, n_nodes, depth=None, status=None):
    """parent [b][N] (and optionally depth) -> status [b] int32: 0 well formed,
    1 n_nodes outside [1, N], 2 + i for the first row i that breaks a rule."""
    L = _load()
    b, N = parent.shape
    if status is None:
        status = torch.empty((b,), dtype=torch.int32, device=parent.device)
    st = L.tv_tree_check(_dev(parent, "parent", torch.int32),
                         _dev(depth, "depth", torch.int32) if depth is not None else None,
                         _dev(n_nodes, "n_nodes", torch.int32), b, N,
                         _dev(status, "status", torch.int32), _stream(parent.device))
    _check(st, "tv_tree_check")
    return status


def tree_expand_workspace(batch, W, V, m):
    return _load().tv_tree_expand_workspace(batch, W, V, m)


def tv_tree_root(root_token, ctx_len, N, out=None):
    """A batch of trees of capacity N holding only their roots (row 0)."""
    L = _load()
    b = root_token.shape[0]
    dev = root_token.device
    i32 = dict(dtype=torch.int32, device=dev)
    if out is None:
        out = dict(parent=torch.empty((b, N), **i32), token=torch.empty((b, N), **i32),
                   depth=torch.empty((b, N), **i32), pos=torch.empty((b, N), **i32),
                   score=torch.empty((b, N), dtype=torch.float64, device=dev),
                   anc=torch.empty((b, N, (N + 63) // 64), dtype=torch.int64, device=dev),
                   n_nodes=torch.empty((b,), **i32))
    if tuple(out["anc"].shape) != (b, N, (N + 63) // 64):
        raise ValueError("anc must be [b][N][ceil(N/64)]")
    st = L.tv_tree_root(_dev(root_token, "root_token", torch.int32),
                        _dev(ctx_len, "ctx_len", torch.int32), b, N, _dev(out["parent"], "parent"),
                        _dev(out["token"], "token"), _dev(out["depth"], "depth"),
                        _dev(out["pos"], "pos"), _dev(out["score"], "score"),
                        _dev(out["anc"], "anc"), _dev(out["n_nodes"], "n_nodes"), _stream(dev))
    _check(st, "tv_tree_root")
    return out


def tv_tree_expand(node_logits, m, frontier, tree, ctx_len, build_temp=1.0,
                   next_frontier=None, workspace=None):
    """One drafting step: node_logits [b][W][V] (f32/bf16) at the frontier
    rows frontier [b][W]; tree (dict as from tv_tree_build) is extended in
    place.  Returns next_frontier [b][W] (may be `frontier` itself)."""
    L = _load()
    b, W, V = node_logits.shape
    N = tree["parent"].shape[1]
    dev = node_logits.device
    if tuple(frontier.shape) != (b, W):
        raise ValueError("frontier must be [b][W]")
    if tuple(tree["anc"].shape) != (b, N, (N + 63) // 64):
        raise ValueError("anc must be [b][N][ceil(N/64)]")
    if next_frontier is None:
        next_frontier = torch.empty((b, W), dtype=torch.int32, device=dev)
    need = L.tv_tree_expand_workspace(b, W, V, m)
    ws, wsb = _workspace(need, dev, workspace)
    st = L.tv_tree_expand(_dev(node_logits, "node_logits"), _dt(node_logits), b, W, V, m,
                          float(build_temp), _dev(ctx_len, "ctx_len", torch.int32),
                          _dev(frontier, "frontier", torch.int32), N,
                          _dev(tree["parent"], "parent", torch.int32),
                          _dev(tree["token"], "token", torch.int32),
                          _dev(tree["depth"], "depth", torch.int32),
                          _dev(tree["pos"], "pos", torch.int32),
                          _dev(tree["score"], "score", torch.float64),
                          _dev(tree["anc"], "anc", torch.int64),
                          _dev(tree["n_nodes"], "n_nodes", torch.int32),
                          _dev(next_frontier, "next_frontier", torch.int32),
                          ws.data_ptr(), wsb, _stream(dev))
    _check(st, "tv_tree_expand")
    return next_frontier
