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


def _rows_worker(meta, rows, scale):
    """Pool worker: attach the shared input arrays and compute its rows."""
    from multiprocessing import shared_memory

    from threadpoolctl import threadpool_limits
    shms, arr = [], {}
    try:
        for name, (shm_name, shape, dt) in meta.items():
            shm = shared_memory.SharedMemory(name=shm_name)
            shms.append(shm)
            arr[name] = np.ndarray(shape, np.dtype(dt), buffer=shm.buf)
        out = []
        with threadpool_limits(limits=1):
            for s, i in rows:
                n = int(arr["nn"][s])
                o, l = _one(arr["q"][s, i], arr["k"][s], arr["v"][s], int(arr["ctx"][s]),
                            _visible(arr["anc"][s, i], n), scale)
                out.append((s, i, o, l))
        arr.clear()
        return out
    finally:
        for shm in shms:
            shm.close()


_pool = None   # (workers, executor), kept for later calls


def _executor(workers):
    """A process pool of `workers`, kept between calls.  Its processes come
    from a forkserver that starts as a fresh interpreter (with this module
    preloaded), so they inherit nothing of the calling process's state; a
    worker that dies fails the call (BrokenProcessPool) rather than being
    restarted."""
    global _pool
    if _pool is not None and _pool[0] == workers:
        return _pool[1]
    if _pool is not None:
        _pool[1].shutdown()
    import atexit
    from concurrent.futures import ProcessPoolExecutor
    from multiprocessing import get_context
    ctx = get_context("forkserver")
    ctx.set_forkserver_preload(["oracle.attention"])
    ex = ProcessPoolExecutor(workers, mp_context=ctx)
    if _pool is None:
        atexit.register(lambda: _pool is not None and _pool[1].shutdown())
    _pool = (workers, ex)
    return ex


def _rows_pool(arrays, rows, scale, workers):
    """The rows spread over `workers` processes, the inputs passed once per
    call through shared memory."""
    from multiprocessing import shared_memory
    shms, meta = [], {}
    try:
        for name, a in arrays.items():
            a = np.ascontiguousarray(a)
            shm = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1))
            shms.append(shm)
            np.ndarray(a.shape, a.dtype, buffer=shm.buf)[...] = a
            meta[name] = (shm.name, a.shape, a.dtype.str)
        chunks = [rows[j::workers] for j in range(workers)]
        parts = list(_executor(workers).map(_rows_worker, [meta] * len(chunks), chunks,
                                            [scale] * len(chunks)))
        return [r for part in parts for r in part]
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()


def tree_attention(q, k, v, ctx_len, anc, n_nodes, scale=None):
    """With oracle.set_threads(n > 1), the independent (sequence, node) rows
    are spread over n worker processes; every row is computed exactly as
    alone, so the results are the same."""
    from . import threads
    q = np.asarray(q)
    b, N, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((b, N, Hq, D), np.float64)
    lse = np.full((b, N, Hq), -np.inf, np.float64)
    rows = [(s, i) for s in range(b) for i in range(int(n_nodes[s]))]
    if threads() > 1 and len(rows) > 1:
        res = _rows_pool(dict(q=q, k=k, v=v, ctx=np.asarray(ctx_len), anc=np.asarray(anc),
                              nn=np.asarray(n_nodes)), rows, scale, min(threads(), len(rows)))
    else:
        res = [(s, i) + _one(q[s, i], k[s], v[s], int(ctx_len[s]),
                             _visible(anc[s, i], int(n_nodes[s])), scale) for s, i in rows]
    for s, i, o, l in res:
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
