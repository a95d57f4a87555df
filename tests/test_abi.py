"""The C ABI library without a GPU: it loads, exports what include/rac.h
declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

import rotary_position_embedding_causal_amd as rac
from rotary_position_embedding_causal_amd import dispatch_fit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rac.h")

# aligned fake device addresses: never dereferenced, every case fails validation first
P = 1 << 20
Q, K, V, O, L = (ctypes.c_void_p(P * (i + 1)) for i in range(5))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(rac.EXPORTED)


def test_library_exports_every_declared_symbol():
    L_ = rac.lib()
    for name in declared_functions():
        assert hasattr(L_, name), name


def fused(**kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    return rac.lib().attn_rope_causal_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                          a["Hq"], a["Hkv"], a["N"], a["D"], a["base"],
                                          a["dtype"], None)


def plain(**kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Hq=4, Hkv=2, N=64, D=64, dtype=0)
    a.update(kw)
    return rac.lib().attn_causal_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                     a["Hkv"], a["N"], a["D"], a["dtype"], None)


def prerot(**kw):
    a = dict(q=Q, k=K, qr=O, kr=L, B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    return rac.lib().rope_prerotate(a["q"], a["k"], a["qr"], a["kr"], a["B"], a["Hq"], a["Hkv"],
                                    a["N"], a["D"], a["base"], a["dtype"], None)


def qonly(**kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    return rac.lib().attn_rope_q_causal_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                            a["Hq"], a["Hkv"], a["N"], a["D"], a["base"],
                                            a["dtype"], None)


def prerot_k(**kw):
    a = dict(k=K, kr=L, B=1, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    return rac.lib().rope_prerotate_k(a["k"], a["kr"], a["B"], a["Hkv"], a["N"], a["D"],
                                      a["base"], a["dtype"], None)


BAD = [
    (dict(dtype=2), rac.RAC_ERR_ARG),
    (dict(D=96), rac.RAC_ERR_UNSUPPORTED),
    (dict(D=256), rac.RAC_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), rac.RAC_ERR_ARG),
    (dict(Hq=0), rac.RAC_ERR_ARG),
    (dict(Hkv=0), rac.RAC_ERR_ARG),
    (dict(B=-1), rac.RAC_ERR_ARG),
    (dict(N=-5), rac.RAC_ERR_ARG),
    (dict(N=rac.RAC_MAX_N + 1), rac.RAC_ERR_ARG),
    (dict(Hq=65536, Hkv=1), rac.RAC_ERR_ARG),
    (dict(q=None), rac.RAC_ERR_ARG),
    (dict(v=None), rac.RAC_ERR_ARG),
    (dict(out=None), rac.RAC_ERR_ARG),
    (dict(q=ctypes.c_void_p(P + 8)), rac.RAC_ERR_ALIGN),
    (dict(lse=ctypes.c_void_p(5 * P + 4)), rac.RAC_ERR_ALIGN),
    (dict(out=Q), rac.RAC_ERR_ARG),                       # out aliases q
    (dict(out=ctypes.c_void_p(P + 4096)), rac.RAC_ERR_ARG),  # out overlaps q
    (dict(lse=O), rac.RAC_ERR_ARG),                       # lse overlaps out
]


@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_attention_rejects_bad_arguments(kw, code):
    assert plain(**kw) == code
    assert rac.last_error() != ""
    assert fused(**kw) == code
    assert qonly(**kw) == code


@pytest.mark.parametrize("base", [0.0, -1.0, float("inf"), float("nan")])
def test_rope_base_must_be_positive_and_finite(base):
    assert fused(base=base) == rac.RAC_ERR_ARG
    assert prerot(base=base) == rac.RAC_ERR_ARG
    assert "rope_base" in rac.last_error()
    assert qonly(base=base) == rac.RAC_ERR_ARG
    assert prerot_k(base=base) == rac.RAC_ERR_ARG


def test_prerotate_overlap_rules():
    assert prerot(qr=None) == rac.RAC_ERR_ARG
    assert prerot(qr=K) == rac.RAC_ERR_ARG                    # q_rot over k
    assert prerot(kr=ctypes.c_void_p(P + 64)) == rac.RAC_ERR_ARG  # k_rot inside q
    assert prerot(qr=ctypes.c_void_p(P + 16)) == rac.RAC_ERR_ARG  # partial in-place
    assert prerot(kr=ctypes.c_void_p(2 * P + 16)) == rac.RAC_ERR_ARG
    assert prerot(q=ctypes.c_void_p(P + 2)) == rac.RAC_ERR_ALIGN
    assert prerot(D=32) == rac.RAC_ERR_UNSUPPORTED
    assert prerot(B=65535, Hq=8, Hkv=8) == rac.RAC_ERR_ARG


def test_prerotate_k_argument_rules():
    assert prerot_k(kr=None) == rac.RAC_ERR_ARG
    assert prerot_k(k=None) == rac.RAC_ERR_ARG
    assert prerot_k(kr=ctypes.c_void_p(2 * P + 16)) == rac.RAC_ERR_ARG  # partial in-place
    assert prerot_k(k=ctypes.c_void_p(2 * P + 8)) == rac.RAC_ERR_ALIGN
    assert prerot_k(D=96) == rac.RAC_ERR_UNSUPPORTED
    assert prerot_k(dtype=3) == rac.RAC_ERR_ARG
    assert prerot_k(Hkv=0) == rac.RAC_ERR_ARG
    assert prerot_k(N=-1) == rac.RAC_ERR_ARG
    assert prerot_k(B=65535, Hkv=9) == rac.RAC_ERR_ARG  # more key slabs than the grid holds
    assert prerot_k(B=0) == rac.RAC_OK
    assert prerot_k(N=0, k=None, kr=None) == rac.RAC_OK


def test_stream_copy_argument_rules():
    cp = rac.lib().rac_stream_copy
    assert cp(Q, ctypes.c_void_p(P + 16), 4096, None) == rac.RAC_ERR_ARG  # overlap
    assert cp(Q, K, P + 16, None) == rac.RAC_ERR_ARG                     # overlap
    assert cp(Q, K, 24, None) == rac.RAC_ERR_ARG                       # not a multiple of 16
    assert cp(None, K, 16, None) == rac.RAC_ERR_ARG
    assert cp(Q, None, 16, None) == rac.RAC_ERR_ARG
    assert cp(ctypes.c_void_p(P + 8), K, 16, None) == rac.RAC_ERR_ALIGN
    assert cp(Q, ctypes.c_void_p(2 * P + 4), 16, None) == rac.RAC_ERR_ALIGN
    assert cp(None, None, 0, None) == rac.RAC_OK
    assert rac.last_error() == ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(B=0, q=None, k=None, v=None,
                                                           out=None, lse=None)])
def test_empty_problem_is_a_noop(kw):
    assert plain(**kw) == rac.RAC_OK
    assert fused(**kw) == rac.RAC_OK
    assert qonly(**kw) == rac.RAC_OK
    pk = {key: val for key, val in kw.items() if key in ("B", "N")}
    assert prerot(**pk) == rac.RAC_OK
    assert rac.last_error() == ""


def test_binding_maps_codes_to_exceptions():
    with pytest.raises(NotImplementedError):
        rac.check(rac.RAC_ERR_UNSUPPORTED, "x")
    with pytest.raises(ValueError):
        rac.check(rac.RAC_ERR_ARG, "x")
    with pytest.raises(rac.RacError):
        rac.check(rac.RAC_ERR_HIP, "x")
    rac.check(rac.RAC_OK, "x")


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(rac, "_lib", None)
    monkeypatch.setattr(rac, "LIB_PATH", "/nonexistent/librac.so")
    with pytest.raises(RuntimeError, match="librac.so is missing"):
        rac.lib()


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        rac.attn_causal_fwd(x, x, x)


def auto(**kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0,
             ws=ctypes.c_void_p(P * 16), wbytes=1 << 20)
    a.update(kw)
    return rac.lib().attn_rope_causal_auto(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                           a["Hq"], a["Hkv"], a["N"], a["D"], a["base"],
                                           a["dtype"], a["ws"], a["wbytes"], None)


@pytest.mark.parametrize("kw,code", BAD)
def test_dispatcher_rejects_bad_arguments(kw, code):
    assert auto(**kw) == code


def test_dispatcher_workspace_rules():
    # workspace overlapping an input or output is rejected before any launch
    assert auto(ws=ctypes.c_void_p(P * 1 + 4096)) == rac.RAC_ERR_ARG
    assert "workspace" in rac.last_error()
    assert auto(ws=ctypes.c_void_p(P * 16 + 8)) == rac.RAC_ERR_ALIGN
    assert auto(base=-1.0) == rac.RAC_ERR_ARG
    assert auto(B=0) == rac.RAC_OK


PATH_CODES = {"fused": rac.RAC_PATH_FUSED, "prerotate": rac.RAC_PATH_PREROTATE,
              "split": rac.RAC_PATH_SPLIT}


def _model_choice(B, Hq, Hkv, N, D):
    """The path-cost model's choice, or None within 1e-9 of a tie."""
    p = dispatch_fit.load_params()
    t = dispatch_fit.model_us(p, B, Hq, Hkv, N, D)
    order = sorted(t.values())
    if order[1] - order[0] <= 1e-9 * order[0]:
        return None
    return dispatch_fit.choose(p, B, Hq, Hkv, N, D)


def test_auto_plan_follows_the_cost_model():
    """With room for any workspace, rac_auto_plan takes the path the fitted
    model (dispatch_model.h, evaluated here from the same constants) costs
    least -- over batch, heads, GQA ratio, length and head dim."""
    seen = set()
    for D in (64, 128):
        for Hq, Hkv in ((4, 4), (16, 16), (32, 32), (32, 8), (64, 8), (8, 1)):
            for B in (1, 2, 8, 64):
                for N in (1, 64, 300, 1024, 1500, 2048, 3000, 4096, 6144, 8192, 16384, 32768,
                          65536):
                    want = _model_choice(B, Hq, Hkv, N, D)
                    if want is None:
                        continue
                    path, need = rac.auto_plan(B, Hq, Hkv, N, D, rac.RAC_BF16, 1 << 62)
                    assert path == PATH_CODES[want], (B, Hq, Hkv, N, D, want)
                    seen.add(want)
    assert seen == set(PATH_CODES)  # the grid reaches every path


def test_auto_plan_workspace_fallbacks():
    """The preferred path's bytes, and the fallbacks when the workspace is short."""
    for B, H, Hkv, N, D in ((1, 16, 16, 16384, 64), (1, 32, 8, 8192, 128), (1, 16, 16, 512, 64),
                            (8, 32, 32, 4096, 128)):
        want = dispatch_fit.choose(dispatch_fit.load_params(), B, H, Hkv, N, D)
        path, need = rac.auto_plan(B, H, Hkv, N, D, rac.RAC_FP16, 1 << 40)
        assert path == PATH_CODES[want]
        q, k = B * H * N * D * 2, B * Hkv * N * D * 2
        if want == "prerotate":
            assert need == ((q + 255) // 256) * 256 + k
            assert rac.auto_plan(B, H, Hkv, N, D, 1, need - 1)[0] == rac.RAC_PATH_SPLIT
            assert rac.auto_plan(B, H, Hkv, N, D, 1, k - 1)[0] == rac.RAC_PATH_FUSED
        elif want == "split":
            assert need == k
            assert rac.auto_plan(B, H, Hkv, N, D, 1, need - 1)[0] == rac.RAC_PATH_FUSED
        else:
            assert need == 0
        assert rac.auto_plan(B, H, Hkv, N, D, 0, 0)[0] == rac.RAC_PATH_FUSED


def test_auto_plan_empty_and_grid_limits():
    assert rac.auto_plan(0, 16, 16, 8192, 64, 1, 0) == (rac.RAC_PATH_FUSED, 0)
    # a path whose streaming pass exceeds its grid (8 * 65535 slabs) is passed over:
    # pre-rotation falls back to split, split to fused
    fell_back = set()
    for B, Hq, Hkv, N, D in ((65535, 32, 16, 4096, 64), (65535, 32, 8, 4096, 64),
                             (20000, 16, 16, 16384, 64), (40000, 16, 16, 16384, 64),
                             (20000, 16, 16, 32768, 128), (40000, 16, 16, 32768, 128),
                             (4000, 128, 8, 8192, 128)):
        pref = dispatch_fit.choose(dispatch_fit.load_params(), B, Hq, Hkv, N, D)
        assert pref != "fused", (B, Hq, Hkv, N, D)
        fits = {"prerotate": B * (Hq + Hkv) <= 8 * 65535, "split": B * Hkv <= 8 * 65535}
        want = pref
        if not fits[want]:
            want = "split" if want == "prerotate" and fits["split"] else "fused"
            fell_back.add((pref, want))
        assert rac.auto_plan(B, Hq, Hkv, N, D, 0, 1 << 60)[0] == PATH_CODES[want], (B, Hq, N)
    assert ("prerotate", "split") in fell_back and any(w == "fused" for _, w in fell_back)
    with pytest.raises(NotImplementedError):
        rac.auto_plan(1, 4, 4, 64, 96, 0, 0)
    with pytest.raises(ValueError):
        rac.auto_plan(1, 4, 3, 64, 64, 0, 0)


def bwd(fused=True, pairing=None, **kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, do=ctypes.c_void_p(P * 6), dq=ctypes.c_void_p(P * 7),
             dk=ctypes.c_void_p(P * 8), dv=ctypes.c_void_p(P * 9), delta=ctypes.c_void_p(P * 10),
             B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    args = [a[x] for x in ("q", "k", "v", "out", "lse", "do", "dq", "dk", "dv", "delta", "B",
                           "Hq", "Hkv", "N", "D")]
    if pairing is not None:
        return rac.lib().attn_rope_causal_bwd_ex(*args, a["base"], pairing, a["dtype"], None)
    if fused:
        return rac.lib().attn_rope_causal_bwd(*args, a["base"], a["dtype"], None)
    return rac.lib().attn_causal_bwd(*args, a["dtype"], None)


# shape and type errors of the forward list apply unchanged (every pointer
# here is a fake, never-dereferenced address: each case must fail validation)
BAD_BWD = BAD[:10]


@pytest.mark.parametrize("kw,code", BAD_BWD, ids=[str(b[0]) for b in BAD_BWD])
def test_backward_rejects_bad_arguments(kw, code):
    assert bwd(True, **kw) == code
    assert bwd(False, **kw) == code
    assert bwd(pairing=0, **kw) == code
    assert bwd(pairing=1, **kw) == code


@pytest.mark.parametrize("name", ["q", "k", "v", "out", "lse", "do", "dq", "dk", "dv", "delta"])
def test_backward_requires_every_pointer(name):
    assert bwd(True, **{name: None}) == rac.RAC_ERR_ARG
    assert bwd(False, **{name: None}) == rac.RAC_ERR_ARG
    assert bwd(pairing=1, **{name: None}) == rac.RAC_ERR_ARG
    assert bwd(True, **{name: ctypes.c_void_p(P * 11 + 8)}) == rac.RAC_ERR_ALIGN
    assert bwd(pairing=1, **{name: ctypes.c_void_p(P * 11 + 8)}) == rac.RAC_ERR_ALIGN


def test_backward_pairing_rules():
    for pairing in (-1, 2, 7):
        assert bwd(pairing=pairing) == rac.RAC_ERR_ARG
        assert "pairing" in rac.last_error()
    # the half-split backward runs through the streaming pass, whose grid
    # holds B * (Hq + Hkv) <= 524280 slabs
    assert bwd(pairing=1, B=65535, Hq=8, Hkv=8) == rac.RAC_ERR_ARG
    assert "524280" in rac.last_error()
    assert bwd(pairing=1, dq=ctypes.c_void_p(P * 1 + 64)) == rac.RAC_ERR_ARG  # dq over q
    assert bwd(pairing=1, base=0.0) == rac.RAC_ERR_ARG
    assert bwd(pairing=1, B=0) == rac.RAC_OK and bwd(pairing=0, B=0) == rac.RAC_OK


def test_backward_overlap_and_empty_rules():
    assert bwd(dq=ctypes.c_void_p(P * 1 + 64)) == rac.RAC_ERR_ARG    # dq over q
    assert bwd(delta=ctypes.c_void_p(P * 9)) == rac.RAC_ERR_ARG      # delta over dv
    assert bwd(False, dk=ctypes.c_void_p(P * 7 + 16)) == rac.RAC_ERR_ARG  # dk over dq
    assert bwd(base=0.0) == rac.RAC_ERR_ARG
    assert bwd(base=float("nan")) == rac.RAC_ERR_ARG
    assert bwd(B=0) == rac.RAC_OK and bwd(N=0, q=None) == rac.RAC_OK
    assert bwd(False, B=0) == rac.RAC_OK


@pytest.mark.parametrize("pairing", [None, 0, 1])
def test_rope_prerotate_bwd_argument_rules(pairing):
    if pairing is None:
        f = rac.lib().rope_prerotate_bwd
    else:
        def f(*a):
            return rac.lib().rope_prerotate_bwd_ex(*a[:10], pairing, *a[10:])
    assert f(Q, K, None, L, 1, 4, 2, 64, 64, 1e4, 0, None) == rac.RAC_ERR_ARG
    assert f(Q, K, ctypes.c_void_p(P + 16), L, 1, 4, 2, 64, 64, 1e4, 0, None) == rac.RAC_ERR_ARG
    assert f(Q, K, ctypes.c_void_p(P * 3 + 8), L, 1, 4, 2, 64, 64, 1e4, 0, None) == rac.RAC_ERR_ALIGN
    assert f(Q, K, O, L, 1, 4, 2, 64, 96, 1e4, 0, None) == rac.RAC_ERR_UNSUPPORTED
    assert f(Q, K, O, L, 1, 4, 2, 64, 64, -1.0, 0, None) == rac.RAC_ERR_ARG
    assert f(Q, K, O, L, 1, 4, 3, 64, 64, 1e4, 0, None) == rac.RAC_ERR_ARG
    assert f(Q, K, O, L, 65535, 8, 8, 64, 64, 1e4, 0, None) == rac.RAC_ERR_ARG
    assert f(Q, K, O, L, 0, 4, 2, 64, 64, 1e4, 0, None) == rac.RAC_OK
    if pairing is not None:
        assert rac.lib().rope_prerotate_bwd_ex(Q, K, O, L, 1, 4, 2, 64, 64, 1e4, 5, 0,
                                               None) == rac.RAC_ERR_ARG


def fused_ex(pairing=1, **kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    return rac.lib().attn_rope_causal_fwd_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                             a["Hq"], a["Hkv"], a["N"], a["D"], a["base"],
                                             pairing, a["dtype"], None)


def prerot_ex(pairing=1, **kw):
    a = dict(q=Q, k=K, qr=O, kr=L, B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    return rac.lib().rope_prerotate_ex(a["q"], a["k"], a["qr"], a["kr"], a["B"], a["Hq"],
                                       a["Hkv"], a["N"], a["D"], a["base"], pairing, a["dtype"],
                                       None)


@pytest.mark.parametrize("pairing", [0, 1])
@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_pairing_entry_points_reject_bad_arguments(kw, code, pairing):
    assert fused_ex(pairing, **kw) == code
    assert rac.last_error() != ""


@pytest.mark.parametrize("pairing", [-1, 2, 7])
def test_unknown_pairing_is_rejected(pairing):
    assert fused_ex(pairing) == rac.RAC_ERR_ARG
    assert "pairing" in rac.last_error()
    assert prerot_ex(pairing) == rac.RAC_ERR_ARG
    assert "pairing" in rac.last_error()
    # checked before the empty-problem shortcut, like every other argument
    assert fused_ex(pairing, B=0) == rac.RAC_ERR_ARG
    assert prerot_ex(pairing, N=0) == rac.RAC_ERR_ARG


@pytest.mark.parametrize("pairing", [0, 1])
def test_pairing_prerotate_rules(pairing):
    assert prerot_ex(pairing, qr=None) == rac.RAC_ERR_ARG
    assert prerot_ex(pairing, qr=K) == rac.RAC_ERR_ARG
    assert prerot_ex(pairing, qr=ctypes.c_void_p(P + 16)) == rac.RAC_ERR_ARG
    assert prerot_ex(pairing, q=ctypes.c_void_p(P + 2)) == rac.RAC_ERR_ALIGN
    assert prerot_ex(pairing, D=32) == rac.RAC_ERR_UNSUPPORTED
    assert prerot_ex(pairing, base=0.0) == rac.RAC_ERR_ARG
    assert prerot_ex(pairing, B=65535, Hq=8, Hkv=8) == rac.RAC_ERR_ARG
    assert fused_ex(pairing, base=float("nan")) == rac.RAC_ERR_ARG
    assert prerot_ex(pairing, B=0) == rac.RAC_OK
    assert fused_ex(pairing, N=0, q=None, k=None, v=None, out=None, lse=None) == rac.RAC_OK
    assert rac.last_error() == ""


def test_binding_pairing_names():
    assert rac._pairing("adjacent") == rac.RAC_PAIR_ADJACENT
    assert rac._pairing("half") == rac.RAC_PAIR_HALF
    assert rac._pairing(1) == rac.RAC_PAIR_HALF
    with pytest.raises(ValueError):
        rac._pairing("interleaved")


S_ = ctypes.c_void_p(P * 7)  # fake slopes address


def alibi(pairing=2, **kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, slopes=S_, B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4,
             dtype=0)
    a.update(kw)
    return rac.lib().attn_alibi_causal_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                           a["Hq"], a["Hkv"], a["N"], a["D"], a["slopes"],
                                           a["base"], pairing, a["dtype"], None)


@pytest.mark.parametrize("pairing", [0, 1, 2])
@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_alibi_rejects_bad_arguments(kw, code, pairing):
    assert alibi(pairing, **kw) == code
    assert rac.last_error() != ""


def test_alibi_argument_rules():
    assert alibi(slopes=None) == rac.RAC_ERR_ARG
    assert "slopes" in rac.last_error()
    assert alibi(slopes=ctypes.c_void_p(P * 7 + 2)) == rac.RAC_ERR_ALIGN
    assert alibi(slopes=ctypes.c_void_p(4 * P + 64)) == rac.RAC_ERR_ARG      # inside out
    assert alibi(slopes=ctypes.c_void_p(5 * P + 16)) == rac.RAC_ERR_ARG      # inside lse
    assert alibi(3) == rac.RAC_ERR_ARG and "pairing" in rac.last_error()
    assert alibi(-1) == rac.RAC_ERR_ARG
    # rope_base matters only with a rotation
    assert alibi(0, base=0.0) == rac.RAC_ERR_ARG and "rope_base" in rac.last_error()
    assert alibi(1, base=float("nan")) == rac.RAC_ERR_ARG
    assert alibi(2, base=0.0, B=0) == rac.RAC_OK
    assert alibi(2, N=0, slopes=None, q=None) == rac.RAC_OK
    assert rac.last_error() == ""


def alibi_bwd(pairing=2, **kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, do=ctypes.c_void_p(P * 6), dq=ctypes.c_void_p(P * 7),
             dk=ctypes.c_void_p(P * 8), dv=ctypes.c_void_p(P * 9), delta=ctypes.c_void_p(P * 10),
             slopes=ctypes.c_void_p(P * 11), B=1, Hq=4, Hkv=2, N=64, D=64, base=1e4, dtype=0)
    a.update(kw)
    args = [a[x] for x in ("q", "k", "v", "out", "lse", "do", "dq", "dk", "dv", "delta", "B",
                           "Hq", "Hkv", "N", "D", "slopes", "base")]
    return rac.lib().attn_alibi_causal_bwd(*args, pairing, a["dtype"], None)


@pytest.mark.parametrize("pairing", [0, 1, 2])
@pytest.mark.parametrize("kw,code", BAD_BWD, ids=[str(b[0]) for b in BAD_BWD])
def test_alibi_backward_rejects_bad_arguments(kw, code, pairing):
    assert alibi_bwd(pairing, **kw) == code


def test_alibi_backward_argument_rules():
    assert alibi_bwd(slopes=None) == rac.RAC_ERR_ARG
    assert "slopes" in rac.last_error()
    assert alibi_bwd(slopes=ctypes.c_void_p(P * 11 + 2)) == rac.RAC_ERR_ALIGN
    assert alibi_bwd(slopes=ctypes.c_void_p(P * 7 + 64)) == rac.RAC_ERR_ARG    # inside dq
    assert alibi_bwd(slopes=ctypes.c_void_p(P * 10 + 16)) == rac.RAC_ERR_ARG   # inside delta
    assert alibi_bwd(dq=ctypes.c_void_p(P * 1 + 64)) == rac.RAC_ERR_ARG        # dq over q
    assert alibi_bwd(do=None) == rac.RAC_ERR_ARG
    assert alibi_bwd(3) == rac.RAC_ERR_ARG and "pairing" in rac.last_error()
    assert alibi_bwd(-1) == rac.RAC_ERR_ARG
    assert alibi_bwd(0, base=0.0) == rac.RAC_ERR_ARG and "rope_base" in rac.last_error()
    assert alibi_bwd(1, base=float("nan")) == rac.RAC_ERR_ARG
    # with RoPE the streaming pass forms the rotated operands: its grid
    for pairing in (0, 1):
        assert alibi_bwd(pairing, B=65535, Hq=8, Hkv=8) == rac.RAC_ERR_ARG
        assert "524280" in rac.last_error()
    assert alibi_bwd(2, base=0.0, B=0) == rac.RAC_OK
    assert alibi_bwd(2, N=0, slopes=None, q=None) == rac.RAC_OK
    assert rac.last_error() == ""


def test_kernel_timer_arguments():
    """rac_time_next_kernel stores or clears an event pair (no HIP call); a
    lone event is an argument error."""
    L_ = rac.lib()
    assert L_.rac_time_next_kernel(None, None) == rac.RAC_OK
    assert L_.rac_time_next_kernel(Q, None) == rac.RAC_ERR_ARG
    assert "both events or neither" in rac.last_error()
    assert L_.rac_time_next_kernel(None, K) == rac.RAC_ERR_ARG
    assert L_.rac_time_next_kernel(Q, K) == rac.RAC_OK  # armed (never launched here) ...
    assert L_.rac_time_next_kernel(None, None) == rac.RAC_OK  # ... and disarmed


def test_valid_call_without_a_device_reports_hip_error():
    """On a machine with no HIP device, calls whose arguments pass validation
    reach the runtime and come back as RAC_ERR_HIP with a message (no crash,
    nothing enqueued); the pointers are never dereferenced."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a HIP device is present: the runtime would accept the call")
    assert fused() == rac.RAC_ERR_HIP and rac.last_error() != ""
    assert plain() == rac.RAC_ERR_HIP and rac.last_error() != ""
    assert prerot() == rac.RAC_ERR_HIP and rac.last_error() != ""
    assert auto() == rac.RAC_ERR_HIP and rac.last_error() != ""
    # the empty problem still succeeds without touching the runtime
    assert fused(N=0) == rac.RAC_OK and rac.last_error() == ""
