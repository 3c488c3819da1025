"""Plain CPU oracle for one tree-verification round.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``tree_verification_best_amd`` and never imports it.

* ``oracle.c`` (built by ``oracle/build.py`` into ``_liboracle.so``): draft
  candidates and their probabilities, best-first and exhaustive subtree
  selection, ancestor sets, the greedy and sampled acceptance walks and the
  Philox4x64-10 generator.
* ``oracle.attention``: tree-masked attention in fp64 numpy; ``oracle.rope``: the
  same with rotary embedding at the tree position ids, and the commit that
  rotates the kept keys.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "_liboracle.so")
_lib = None

GREEDY, SAMPLED = 0, 1
POINT_MASS, DRAFT = 0, 1

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(dtype=np.uint64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def lib():
    """Load (building on first use if absent) the oracle's shared library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        from . import build as _b
        _b.build()
    L = ctypes.CDLL(_LIBPATH)
    c = ctypes
    L.tvo_exp_spec.argtypes = [c.c_float]
    L.tvo_exp_spec.restype = c.c_float
    L.tvo_exp_spec_n.argtypes = [_f32p, _f32p, c.c_int64]
    L.tvo_exp_spec_n.restype = None
    L.tvo_constants.argtypes = [_f32p]
    L.tvo_constants.restype = None
    L.tvo_weight.argtypes = [c.c_float, c.c_float, c.c_float]
    L.tvo_weight.restype = c.c_uint64
    L.tvo_row_weights.argtypes = [_f32p, c.c_int, c.c_float, _u64p]
    L.tvo_row_weights.restype = c.c_uint64
    L.tvo_philox4x64_10.argtypes = [_u64p, _u64p, _u64p]
    L.tvo_philox4x64_10.restype = None
    L.tvo_topk.argtypes = [_f32p, c.c_int, c.c_int, _i32p, _f32p]
    L.tvo_topk.restype = c.c_int
    L.tvo_draft_candidates.argtypes = [_f32p, c.c_int, c.c_int, c.c_int, c.c_float, _i32p,
                                       _f64p, _u64p]
    L.tvo_draft_candidates.restype = c.c_int
    sel = [_i32p, _f64p, c.c_int, c.c_int, c.c_int, c.c_int32, _i32p, _i32p, _i32p, _f64p]
    L.tvo_select_best_first.argtypes = sel
    L.tvo_select_best_first.restype = c.c_int
    L.tvo_select_exhaustive.argtypes = sel
    L.tvo_select_exhaustive.restype = c.c_int
    L.tvo_ancestors.argtypes = [_i32p, c.c_int, c.c_int, _u64p, _i32p]
    L.tvo_ancestors.restype = c.c_int
    L.tvo_tree_build.argtypes = [_f32p, c.c_int, c.c_int, c.c_int, c.c_int, c.c_int, c.c_float,
                                 _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, _f64p, _u64p, _i32p]
    L.tvo_tree_build.restype = c.c_int
    L.tvo_tree_accept.argtypes = [_f32p, c.c_void_p, c.c_int, c.c_int, c.c_int, c.c_int,
                                  _i32p, _i32p, _i32p, _i32p, c.c_int, c.c_float, c.c_int,
                                  c.c_uint64, c.c_uint64, c.c_int, _i32p, _i32p, _i32p]
    L.tvo_tree_accept.restype = c.c_int
    L.tvo_weight_range.argtypes = [c.c_uint32, c.c_int64, c.c_float, c.c_float, _u64p]
    L.tvo_weight_range.restype = None
    L.tvo_set_threads.argtypes = [c.c_int]
    L.tvo_set_threads.restype = c.c_int
    L.tvo_set_threads(_threads)
    _lib = L
    return L


_threads = 1


def set_threads(n):
    """Threads for the independent parts of a round: the draft positions of
    the builder (OpenMP in oracle.c) and the (sequence, node) rows of the
    attention (a thread pool).  Each part is computed exactly as with one
    thread, so results do not depend on this.  Returns the previous value."""
    global _threads
    prev = _threads
    _threads = max(1, int(n))
    if _lib is not None:
        _lib.tvo_set_threads(_threads)
    return prev


def threads():
    return _threads


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# --------------------------------------------------------------------------
# numerics
# --------------------------------------------------------------------------
def exp_spec(x):
    x = _f32(x)
    y = np.empty_like(x)
    lib().tvo_exp_spec_n(x.reshape(-1), y.reshape(-1), x.size)
    return y


def constants():
    out = np.zeros(4, np.float32)
    lib().tvo_constants(out)
    return out


def weight(logit, row_max, inv_t=1.0):
    return int(lib().tvo_weight(float(np.float32(logit)), float(np.float32(row_max)),
                                float(np.float32(inv_t))))


def weight_range(first_bits, count, row_max=0.0, inv_t=1.0):
    """weight() of the `count` fp32 values with bit patterns first_bits, first_bits + 1, ..."""
    out = np.empty(int(count), np.uint64)
    lib().tvo_weight_range(int(first_bits), int(count), float(row_max), float(inv_t), out)
    return out


def row_weights(row, temperature=1.0):
    """(W[v], Z) of one logits row at the given temperature."""
    row = _f32(row)
    W = np.zeros(row.shape[0], np.uint64)
    inv_t = np.float32(1.0) / np.float32(temperature)
    Z = lib().tvo_row_weights(row, row.shape[0], float(inv_t), W)
    return W, int(Z)


def philox(counter, key):
    ctr = np.ascontiguousarray(counter, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, np.uint64)
    lib().tvo_philox4x64_10(ctr, k, out)
    return out


# --------------------------------------------------------------------------
# tree build
# --------------------------------------------------------------------------
def topk(row, k):
    row = _f32(row)
    ids = np.zeros(k, np.int32)
    vals = np.zeros(k, np.float32)
    if lib().tvo_topk(row, row.shape[0], k, ids, vals):
        raise ValueError("bad top-k arguments")
    return ids, vals


def draft_candidates(draft, k, build_temp=1.0):
    """draft [K][V] -> (cand_tok [K][k], cand_q [K][k], Z [K])."""
    draft = _f32(draft)
    K, V = draft.shape
    tok = np.zeros((K, k), np.int32)
    q = np.zeros((K, k), np.float64)
    Z = np.zeros(K, np.uint64)
    if lib().tvo_draft_candidates(draft, K, V, k, build_temp, tok, q, Z):
        raise ValueError("bad candidate arguments")
    return tok, q, Z


def _select(fn, cand_tok, cand_q, budget, root_token):
    cand_tok = _i32(cand_tok)
    cand_q = np.ascontiguousarray(cand_q, dtype=np.float64)
    K, k = cand_tok.shape
    N = budget + 1
    parent = np.full(N, -1, np.int32)
    token = np.full(N, -1, np.int32)
    depth = np.full(N, -1, np.int32)
    score = np.zeros(N, np.float64)
    n = fn(cand_tok, cand_q, K, k, budget, root_token, parent, token, depth, score)
    if n < 1:
        raise ValueError("selection failed")
    return dict(parent=parent[:n], token=token[:n], depth=depth[:n], score=score[:n], n=n)


def select_best_first(cand_tok, cand_q, budget, root_token=0):
    return _select(lib().tvo_select_best_first, cand_tok, cand_q, budget, root_token)


def select_exhaustive(cand_tok, cand_q, budget, root_token=0):
    return _select(lib().tvo_select_exhaustive, cand_tok, cand_q, budget, root_token)


def ancestors(parent, words=None):
    parent = _i32(parent)
    n = parent.shape[0]
    words = words or (n + 63) // 64
    anc = np.zeros((n, words), np.uint64)
    depth = np.zeros(n, np.int32)
    if lib().tvo_ancestors(parent, n, words, anc, depth):
        raise ValueError("malformed parent array")
    return anc, depth


def tree_build(draft, k, budget, root_token, ctx_len, build_temp=1.0):
    """Whole builder; draft [b][K][V] float.  Returns the boundary's arrays."""
    draft = _f32(draft)
    b, K, V = draft.shape
    N = budget + 1
    W = (N + 63) // 64
    out = dict(parent=np.zeros((b, N), np.int32), token=np.zeros((b, N), np.int32),
               depth=np.zeros((b, N), np.int32), pos=np.zeros((b, N), np.int32),
               score=np.zeros((b, N), np.float64), anc=np.zeros((b, N, W), np.uint64),
               n_nodes=np.zeros(b, np.int32))
    rc = lib().tvo_tree_build(draft, b, K, V, k, budget, build_temp, _i32(root_token),
                              _i32(ctx_len), out["parent"], out["token"], out["depth"],
                              out["pos"], out["score"], out["anc"], out["n_nodes"])
    if rc:
        raise ValueError("tree build failed")
    return out


# --------------------------------------------------------------------------
# acceptance
# --------------------------------------------------------------------------
def tree_accept(target, parent, token, depth, n_nodes, *, mode, temperature=1.0,
                proposal=POINT_MASS, seed=0, round=0, max_depth, draft=None):
    """target [b][N][V]; parent/token/depth [b][N]; n_nodes [b].

    Returns dict(accept_len [b], accepted_nodes [b][max_depth+1],
    out_tokens [b][max_depth+1]).  accept_len is -1 for a sequence the DRAFT
    proposal cannot take (a node with several children)."""
    target = _f32(target)
    b, N, V = target.shape
    K = 0
    dptr = None
    if draft is not None:
        draft = _f32(draft)
        K = draft.shape[1]
        dptr = draft.ctypes.data_as(ctypes.c_void_p)
    width = max_depth + 1
    acc_len = np.zeros(b, np.int32)
    acc_nodes = np.zeros((b, width), np.int32)
    out_tok = np.zeros((b, width), np.int32)
    lib().tvo_tree_accept(target, dptr, b, N, K, V, _i32(parent), _i32(token), _i32(depth),
                          _i32(n_nodes), mode, temperature, proposal, seed, round, max_depth,
                          acc_len, acc_nodes, out_tok)
    return dict(accept_len=acc_len, accepted_nodes=acc_nodes, out_tokens=out_tok)


from .attention import tree_attention, tree_attention_rows  # noqa: E402,F401
from .commit import kv_commit  # noqa: E402,F401
from .budget import tree_budget  # noqa: E402,F401
from .expand import tree_expand, tree_root  # noqa: E402,F401
from .rope import (inv_freq, kv_commit_rope, rope, tree_attention_rope,  # noqa: E402,F401
                   tree_attention_rope_rows)


def tree_check(parent, n_nodes, depth=None):
    """Structural check of trees (PTD sec. 3.1: one parent per node, parents
    first): 0 well formed, 1 n_nodes outside [1, N], else 2 + the first row
    breaking parent[0] = -1, 0 <= parent[i] < i, depth[0] = 0 and
    depth[i] = depth[parent[i]] + 1 (depth when given)."""
    parent = np.asarray(parent)
    b, N = parent.shape
    out = np.zeros(b, np.int32)
    for s in range(b):
        n = int(n_nodes[s])
        if n < 1 or n > N:
            out[s] = 1
            continue
        for i in range(n):
            p = int(parent[s, i])
            ok = p == -1 if i == 0 else 0 <= p < i
            if ok and depth is not None:
                ok = int(depth[s, 0]) == 0 if i == 0 else int(depth[s, i]) == int(depth[s, p]) + 1
            if not ok:
                out[s] = 2 + i
                break
    return out
