"""The C ABI without a GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments on the host
before any launch (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import tree_verification_best_amd as tv

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "treeverify.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_[a-z_]+)\s*\(", text)))


def test_header_functions_exported():
    names = _declared()
    assert len(names) == 21
    lib = ctypes.CDLL(tv.LIBPATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tv.EXPORTS)


def test_version_and_status_strings():
    L = tv.lib()
    assert L.tv_version() == 10000
    for s in range(5):
        assert L.tv_status_string(s).startswith(b"TV_")
    assert b"unknown" in L.tv_status_string(17)


def test_workspace_queries():
    L = tv.lib()
    assert L.tv_tree_build_workspace(1, 16, 151936, 8, 64) > 0
    assert L.tv_tree_build_workspace(1, 0, 100, 4, 8) == 0        # K < 1
    assert L.tv_tree_build_workspace(1, 4, 1 << 19, 4, 8) == 0    # V too large
    assert L.tv_tree_build_workspace(1, 4, 100, 65, 8) == 0       # topk > 64
    assert L.tv_tree_build_workspace(1, 4, 100, 4, 1024) == 0     # budget > 1023
    assert L.tv_tree_attention_workspace(1, 65, 32, 8, 128, 4096, 0) > 0
    assert L.tv_tree_attention_workspace(1, 65, 32, 7, 128, 4096, 0) == 0   # Hq % Hkv
    assert L.tv_tree_attention_workspace(1, 65, 32, 8, 96, 4096, 0) == 0    # D
    assert L.tv_tree_accept_workspace(1, 65, 16, 151936, tv.TV_GREEDY, 0) > 0
    g = L.tv_tree_accept_workspace(1, 65, 16, 151936, tv.TV_GREEDY, 0)
    s = L.tv_tree_accept_workspace(1, 65, 16, 151936, tv.TV_SAMPLED, 0)
    d = L.tv_tree_accept_workspace(1, 65, 16, 151936, tv.TV_SAMPLED, 1)
    assert g < s < d
    assert L.tv_tree_expand_workspace(1, 8, 151936, 8) > 0
    assert L.tv_tree_expand_workspace(1, 65, 100, 4) == 0    # W > 64
    assert L.tv_tree_expand_workspace(1, 8, 100, 101) == 0   # m > V


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _build(**kw):
    a = dict(draft=FAKE, dt=0, batch=1, K=4, V=100, topk=4, budget=8, temp=1.0, root=FAKE,
             ctx=FAKE, parent=FAKE, token=FAKE, depth=FAKE, pos=FAKE, score=FAKE, anc=FAKE,
             n=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return tv.lib().tv_tree_build(a["draft"], a["dt"], a["batch"], a["K"], a["V"], a["topk"],
                                  a["budget"], a["temp"], a["root"], a["ctx"], a["parent"],
                                  a["token"], a["depth"], a["pos"], a["score"], a["anc"],
                                  a["n"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(draft=None), tv.TV_ERR_INVALID),
    (dict(n=None), tv.TV_ERR_INVALID),
    (dict(dt=5), tv.TV_ERR_INVALID),
    (dict(temp=0.0), tv.TV_ERR_INVALID),
    (dict(temp=float("nan")), tv.TV_ERR_INVALID),
    (dict(K=0), tv.TV_ERR_INVALID),
    (dict(topk=101), tv.TV_ERR_INVALID),
    (dict(budget=-1), tv.TV_ERR_INVALID),
    (dict(K=65), tv.TV_ERR_UNSUPPORTED),
    (dict(topk=65, V=1000), tv.TV_ERR_UNSUPPORTED),
    (dict(V=(1 << 18) + 1), tv.TV_ERR_UNSUPPORTED),
    (dict(budget=1024), tv.TV_ERR_UNSUPPORTED),
    (dict(K=64, topk=64, V=1 << 18, budget=870), tv.TV_ERR_UNSUPPORTED),  # selection LDS
    (dict(ws=None), tv.TV_ERR_WORKSPACE),
    (dict(wsb=16), tv.TV_ERR_WORKSPACE),
])
def test_build_rejects(kw, status):
    assert _build(**kw) == status


def _build_noalloc(**kw):
    a = dict(draft=FAKE, dt=0, batch=1, K=4, V=100, topk=4, budget=8, temp=1.0, root=FAKE,
             ctx=FAKE, parent=FAKE, token=FAKE, depth=FAKE, pos=FAKE, score=FAKE, anc=FAKE,
             n=FAKE)
    a.update(kw)
    return tv.lib().tv_tree_build_noalloc(a["draft"], a["dt"], a["batch"], a["K"], a["V"],
                                          a["topk"], a["budget"], a["temp"], a["root"],
                                          a["ctx"], a["parent"], a["token"], a["depth"],
                                          a["pos"], a["score"], a["anc"], a["n"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(draft=None), tv.TV_ERR_INVALID),
    (dict(anc=None), tv.TV_ERR_INVALID),
    (dict(temp=-1.0), tv.TV_ERR_INVALID),
    (dict(K=65), tv.TV_ERR_UNSUPPORTED),
    (dict(budget=1024), tv.TV_ERR_UNSUPPORTED),
    # the shape's workspace exceeds the static scratch: refused before any device call
    (dict(batch=512, K=16, V=151936, topk=16, budget=64), tv.TV_ERR_UNSUPPORTED),
])
def test_build_noalloc_rejects(kw, status):
    assert _build_noalloc(**kw) == status


def test_build_noalloc_limit_matches_workspace():
    """Shapes up to the scratch size pass the size check; the first beyond it fails."""
    L = tv.lib()
    cap = 4 << 20
    fits = [b for b in range(1, 200) if L.tv_tree_build_workspace(b, 16, 151936, 16, 64) <= cap]
    assert fits and fits[-1] < 199
    over = fits[-1] + 1
    assert L.tv_tree_build_workspace(over, 16, 151936, 16, 64) > cap
    assert _build_noalloc(batch=over, K=16, V=151936, topk=16, budget=64) == \
        tv.TV_ERR_UNSUPPORTED


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=1, ctx=FAKE, anc=FAKE, n=FAKE, batch=1, N=17, Hq=4,
             Hkv=2, D=128, cap=200, max_ctx=128, scale=0.1, splits=0, out=FAKE, odt=0,
             lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return tv.lib().tv_tree_attention_verify(a["q"], a["k"], a["v"], a["dt"], a["ctx"],
                                             a["anc"], a["n"], a["batch"], a["N"], a["Hq"],
                                             a["Hkv"], a["D"], a["cap"], a["max_ctx"],
                                             a["scale"], a["splits"], a["out"], a["odt"],
                                             a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), tv.TV_ERR_INVALID),
    (dict(out=None), tv.TV_ERR_INVALID),
    (dict(Hkv=3), tv.TV_ERR_INVALID),
    (dict(cap=100), tv.TV_ERR_INVALID),          # max_ctx + N > cap
    (dict(scale=-1.0), tv.TV_ERR_INVALID),
    (dict(splits=-2), tv.TV_ERR_INVALID),
    (dict(odt=7), tv.TV_ERR_INVALID),
    (dict(dt=0, odt=1), tv.TV_ERR_UNSUPPORTED),        # fp32 inputs give fp32 output
    (dict(D=96), tv.TV_ERR_UNSUPPORTED),
    (dict(N=1025, cap=5000), tv.TV_ERR_UNSUPPORTED),
    (dict(ws=None), tv.TV_ERR_WORKSPACE),
    (dict(wsb=8), tv.TV_ERR_WORKSPACE),
])
def test_attention_rejects(kw, status):
    assert _attn(**kw) == status


def _acc(**kw):
    a = dict(t=FAKE, d=None, dt=0, batch=1, N=17, K=4, V=100, parent=FAKE, token=FAKE,
             depth=FAKE, n=FAKE, mode=1, temp=1.0, prop=0, seed=1, rnd=0, maxd=4, al=FAKE,
             an=FAKE, ot=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return tv.lib().tv_tree_accept(a["t"], a["d"], a["dt"], a["batch"], a["N"], a["K"], a["V"],
                                   a["parent"], a["token"], a["depth"], a["n"], a["mode"],
                                   a["temp"], a["prop"], a["seed"], a["rnd"], a["maxd"],
                                   a["al"], a["an"], a["ot"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(t=None), tv.TV_ERR_INVALID),
    (dict(al=None), tv.TV_ERR_INVALID),
    (dict(mode=3), tv.TV_ERR_INVALID),
    (dict(prop=2), tv.TV_ERR_INVALID),
    (dict(temp=0.0), tv.TV_ERR_INVALID),
    (dict(prop=1), tv.TV_ERR_INVALID),            # DRAFT without draft logits
    (dict(maxd=0), tv.TV_ERR_INVALID),
    (dict(V=(1 << 18) + 1), tv.TV_ERR_UNSUPPORTED),
    (dict(N=1025), tv.TV_ERR_UNSUPPORTED),
    (dict(batch=5000, N=17), tv.TV_ERR_UNSUPPORTED),   # rows beyond the grid limit
    (dict(ws=None), tv.TV_ERR_WORKSPACE),
])
def test_accept_rejects(kw, status):
    assert _acc(**kw) == status


def test_ancestors_rejects():
    L = tv.lib()
    assert L.tv_tree_ancestors(None, FAKE, FAKE, 1, 8, FAKE, FAKE, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_ancestors(FAKE, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_ancestors(FAKE, FAKE, FAKE, 1, 1025, FAKE, FAKE, FAKE, None) == \
        tv.TV_ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 4, 100))
    with pytest.raises(ValueError):
        tv.tv_tree_build(x, 4, 8, torch.zeros(1, dtype=torch.int32),
                         torch.zeros(1, dtype=torch.int32))


def _commit(**kw):
    a = dict(k=FAKE, v=FAKE, dt=1, batch=1, Hkv=2, cap=64, D=128, ctx=FAKE, al=FAKE, an=FAKE,
             width=17, new=FAKE)
    a.update(kw)
    return tv.lib().tv_kv_commit(a["k"], a["v"], a["dt"], a["batch"], a["Hkv"], a["cap"],
                                 a["D"], a["ctx"], a["al"], a["an"], a["width"], a["new"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), tv.TV_ERR_INVALID),
    (dict(new=None), tv.TV_ERR_INVALID),
    (dict(dt=4), tv.TV_ERR_INVALID),
    (dict(batch=0), tv.TV_ERR_INVALID),
    (dict(width=0), tv.TV_ERR_INVALID),
    (dict(D=96), tv.TV_ERR_UNSUPPORTED),
    (dict(width=1025), tv.TV_ERR_UNSUPPORTED),
])
def test_commit_rejects(kw, status):
    assert _commit(**kw) == status


def test_budget_rejects():
    L = tv.lib()
    assert L.tv_tree_budget(None, FAKE, FAKE, 1, 8, 8, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_budget(FAKE, FAKE, FAKE, 1, 8, 7, FAKE, None) == tv.TV_ERR_INVALID  # ncost < N
    assert L.tv_tree_budget(FAKE, FAKE, FAKE, 0, 8, 8, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_budget(FAKE, FAKE, FAKE, 1, 1025, 2000, FAKE, None) == tv.TV_ERR_UNSUPPORTED


def test_root_rejects():
    L = tv.lib()
    f = [FAKE] * 7
    assert L.tv_tree_root(None, FAKE, 1, 8, *f, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_root(FAKE, FAKE, 0, 8, *f, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_root(FAKE, FAKE, 1, 0, *f, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_root(FAKE, FAKE, 1, 1025, *f, None) == tv.TV_ERR_UNSUPPORTED


def _expand(**kw):
    a = dict(x=FAKE, dt=0, batch=1, W=4, V=100, m=4, temp=1.0, ctx=FAKE, front=FAKE, N=64,
             nxt=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return tv.lib().tv_tree_expand(a["x"], a["dt"], a["batch"], a["W"], a["V"], a["m"],
                                   a["temp"], a["ctx"], a["front"], a["N"], *([FAKE] * 7),
                                   a["nxt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tv.TV_ERR_INVALID),
    (dict(nxt=None), tv.TV_ERR_INVALID),
    (dict(dt=3), tv.TV_ERR_INVALID),
    (dict(temp=0.0), tv.TV_ERR_INVALID),
    (dict(temp=float("nan")), tv.TV_ERR_INVALID),
    (dict(W=0), tv.TV_ERR_INVALID),
    (dict(m=101), tv.TV_ERR_INVALID),
    (dict(N=0), tv.TV_ERR_INVALID),
    (dict(W=65), tv.TV_ERR_UNSUPPORTED),
    (dict(m=65), tv.TV_ERR_UNSUPPORTED),
    (dict(N=1025), tv.TV_ERR_UNSUPPORTED),
    (dict(V=1 << 19), tv.TV_ERR_UNSUPPORTED),
    (dict(wsb=16), tv.TV_ERR_WORKSPACE),
    (dict(ws=None), tv.TV_ERR_WORKSPACE),
])
def test_expand_rejects(kw, status):
    assert _expand(**kw) == status


def _attn_rope(pos=FAKE, base=1e4, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=1, ctx=FAKE, anc=FAKE, n=FAKE, batch=1, N=17, Hq=4,
             Hkv=2, D=128, cap=200, max_ctx=128, scale=0.1, splits=0, out=FAKE, odt=0,
             lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return tv.lib().tv_tree_attention_verify_rope(
        a["q"], a["k"], a["v"], a["dt"], a["ctx"], a["anc"], a["n"], pos, base, a["batch"],
        a["N"], a["Hq"], a["Hkv"], a["D"], a["cap"], a["max_ctx"], a["scale"], a["splits"],
        a["out"], a["odt"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=None), tv.TV_ERR_INVALID),
    (dict(base=1.0), tv.TV_ERR_INVALID),
    (dict(base=0.5), tv.TV_ERR_INVALID),
    (dict(base=float("inf")), tv.TV_ERR_INVALID),
    (dict(base=float("nan")), tv.TV_ERR_INVALID),
    (dict(q=None), tv.TV_ERR_INVALID),
    (dict(D=96), tv.TV_ERR_UNSUPPORTED),
    (dict(wsb=8), tv.TV_ERR_WORKSPACE),
])
def test_attention_rope_rejects(kw, status):
    assert _attn_rope(**kw) == status


def test_commit_rope_rejects():
    L = tv.lib()

    def call(base=1e4, k=FAKE, D=128):
        return L.tv_kv_commit_rope(k, FAKE, 1, 1, 2, 64, D, FAKE, FAKE, FAKE, 17, base, FAKE,
                                   None)
    assert call(base=1.0) == tv.TV_ERR_INVALID
    assert call(base=float("nan")) == tv.TV_ERR_INVALID
    assert call(k=None) == tv.TV_ERR_INVALID
    assert call(D=96) == tv.TV_ERR_UNSUPPORTED


def test_check_rejects():
    L = tv.lib()
    assert L.tv_tree_check(None, None, FAKE, 1, 8, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_check(FAKE, None, FAKE, 0, 8, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_check(FAKE, None, FAKE, 1, 0, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_tree_check(FAKE, None, FAKE, 1, 8, None, None) == tv.TV_ERR_INVALID


def test_spin_limit_hook():
    """The sampled row pass's wait bound: set, capped at the default, restored."""
    L = tv.lib()
    assert L.tv_debug_set_spin_limit(0) == 48
    assert L.tv_debug_set_spin_limit(10 ** 9) == 0
    assert L.tv_debug_set_spin_limit(-1) == 48  # capped at the default
    assert L.tv_debug_set_spin_limit(-1) == 48


def test_debug_hooks_reject_on_host():
    L = tv.lib()
    assert L.tv_debug_weights(0, 16, 0.0, 1.0, 0, None, None) == tv.TV_ERR_INVALID
    assert L.tv_debug_weights(0, 0, 0.0, 1.0, 0, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_debug_weights(0, 16, float("inf"), 1.0, 0, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_debug_weights(0, 16, 0.0, 0.0, 0, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_debug_weights(0, 16, 0.0, 0.7, 1, FAKE, None) == tv.TV_ERR_INVALID
    assert L.tv_debug_set_attention_events(None, None) == tv.TV_OK
