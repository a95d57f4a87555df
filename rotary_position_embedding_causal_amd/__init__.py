"""RoPE + causal attention forward for AMD MI355X (gfx950).

Thin Python binding over ``librac.so`` (C ABI in ``include/rac.h``): it only
checks and marshals torch tensors into pointers and sizes, passes torch's
current HIP stream, and turns error codes into exceptions. Every step of the
computation runs in the library's HIP kernels; there is no CPU fallback, and
calling any operation without the built library raises.

Operations (names as in the C ABI):
  attn_rope_causal_fwd(q, k, v, rope_base)  -> (out, lse)   fused RoPE + attention
  rope_prerotate(q, k, rope_base)           -> (q_rot, k_rot)
  attn_causal_fwd(q, k, v)                  -> (out, lse)   on pre-rotated inputs
  rope_prerotate_k(k, rope_base)            -> k_rot          K only (GQA split path)
  attn_rope_q_causal_fwd(q, k_rot, v, rope_base) -> (out, lse) RoPE on Q in the kernel
  attn_rope_causal_auto(q, k, v, rope_base, workspace) -> (out, lse) fastest path
  attn_rope_causal_bwd(q, k, v, out, lse, dout, rope_base) -> (dq, dk, dv, delta)
  attn_causal_bwd(q, k, v, out, lse, dout) -> (dq, dk, dv, delta)  on rotated inputs
  rope_prerotate_bwd(dq_rot, dk_rot, rope_base) -> (dq, dk)
  auto_plan(B, Hq, Hkv, N, D, dtype, workspace_bytes) -> (path, preferred_bytes)
Tensors are contiguous [B, H, N, D] bf16/fp16 on one HIP device; lse is fp32
[B, Hq, N] (natural log).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librac.so")

RAC_BF16, RAC_FP16 = 0, 1
RAC_OK, RAC_ERR_ARG, RAC_ERR_ALIGN, RAC_ERR_UNSUPPORTED, RAC_ERR_HIP = 0, -1, -2, -3, -4
RAC_MAX_N = 1 << 22
EXPORTED = ("attn_rope_causal_fwd", "rope_prerotate", "attn_causal_fwd", "rope_prerotate_k",
            "attn_rope_q_causal_fwd", "attn_rope_causal_auto", "rac_auto_plan",
            "attn_rope_causal_bwd", "attn_causal_bwd", "rope_prerotate_bwd",
            "rope_prerotate_ex", "attn_rope_causal_fwd_ex", "attn_alibi_causal_fwd",
            "rac_last_error", "rac_release_tables", "rac_time_next_kernel",
            "attn_rope_causal_fwd_noalloc", "rac_stream_copy", "attn_rope_causal_bwd_ex",
            "rope_prerotate_bwd_ex", "attn_alibi_causal_bwd")
RAC_NOALLOC_MAX_N = 32768
RAC_PAIR_ADJACENT, RAC_PAIR_HALF, RAC_ROPE_NONE = 0, 1, 2
PAIRINGS = {"adjacent": RAC_PAIR_ADJACENT, "half": RAC_PAIR_HALF, "none": RAC_ROPE_NONE}
RAC_PATH_FUSED, RAC_PATH_PREROTATE, RAC_PATH_SPLIT = 0, 1, 2
PATH_NAMES = {RAC_PATH_FUSED: "fused", RAC_PATH_PREROTATE: "prerotate", RAC_PATH_SPLIT: "split"}

_DTYPES = {torch.bfloat16: RAC_BF16, torch.float16: RAC_FP16}

_lib = None


class RacError(RuntimeError):
    """A HIP runtime failure reported by the library."""


def lib() -> ctypes.CDLL:
    """The loaded librac.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("librac.so is missing at %s: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i, d, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    L.attn_rope_causal_fwd.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, d, i, vp]
    L.attn_rope_causal_fwd.restype = i
    L.rope_prerotate.argtypes = [vp, vp, vp, vp, i, i, i, i, i, d, i, vp]
    L.rope_prerotate.restype = i
    L.attn_causal_fwd.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, i, vp]
    L.attn_causal_fwd.restype = i
    L.rope_prerotate_k.argtypes = [vp, vp, i, i, i, i, d, i, vp]
    L.rope_prerotate_k.restype = i
    L.attn_rope_q_causal_fwd.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, d, i, vp]
    L.attn_rope_q_causal_fwd.restype = i
    sz = ctypes.c_size_t
    L.attn_rope_causal_auto.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, d, i, vp, sz, vp]
    L.attn_rope_causal_auto.restype = i
    L.rac_auto_plan.argtypes = [i, i, i, i, i, i, sz, ctypes.POINTER(i), ctypes.POINTER(sz)]
    L.rac_auto_plan.restype = i
    L.attn_rope_causal_bwd.argtypes = [vp] * 10 + [i] * 5 + [d, i, vp]
    L.attn_rope_causal_bwd.restype = i
    L.attn_causal_bwd.argtypes = [vp] * 10 + [i] * 6 + [vp]
    L.attn_causal_bwd.restype = i
    L.rope_prerotate_bwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, d, i, vp]
    L.rope_prerotate_bwd.restype = i
    L.attn_rope_causal_bwd_ex.argtypes = [vp] * 10 + [i] * 5 + [d, i, i, vp]
    L.attn_rope_causal_bwd_ex.restype = i
    L.rope_prerotate_bwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, d, i, i, vp]
    L.rope_prerotate_bwd_ex.restype = i
    L.attn_alibi_causal_bwd.argtypes = [vp] * 10 + [i] * 5 + [vp, d, i, i, vp]
    L.attn_alibi_causal_bwd.restype = i
    L.rope_prerotate_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, d, i, i, vp]
    L.rope_prerotate_ex.restype = i
    L.attn_rope_causal_fwd_ex.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, d, i, i, vp]
    L.attn_rope_causal_fwd_ex.restype = i
    L.attn_alibi_causal_fwd.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, vp, d, i, i, vp]
    L.attn_alibi_causal_fwd.restype = i
    L.rac_last_error.argtypes = []
    L.rac_last_error.restype = ctypes.c_char_p
    L.rac_release_tables.argtypes = []
    L.rac_release_tables.restype = i
    L.rac_time_next_kernel.argtypes = [vp, vp]
    L.rac_time_next_kernel.restype = i
    L.rac_stream_copy.argtypes = [vp, vp, sz, vp]
    L.rac_stream_copy.restype = i
    L.attn_rope_causal_fwd_noalloc.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, d, i, vp]
    L.attn_rope_causal_fwd_noalloc.restype = i
    _lib = L
    return L


def last_error() -> str:
    return lib().rac_last_error().decode()


def check(rc: int, what: str) -> None:
    """Raise for a non-zero return code of the C ABI."""
    if rc == RAC_OK:
        return
    msg = "%s: %s (code %d)" % (what, last_error(), rc)
    if rc == RAC_ERR_HIP:
        raise RacError(msg)
    if rc == RAC_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise ValueError(msg)


def release_tables() -> None:
    check(lib().rac_release_tables(), "rac_release_tables")


def time_next_kernel(start, stop) -> None:
    """Arms two torch.cuda.Event(enable_timing=True) objects to record the
    start and end of the next forward attention or pre-rotation kernel this
    thread launches (the kernel's own execution, without dispatch latency);
    read it with start.elapsed_time(stop) after synchronising. None, None
    disarms."""
    if start is None and stop is None:
        check(lib().rac_time_next_kernel(None, None), "rac_time_next_kernel")
        return
    for ev in (start, stop):
        if ev.cuda_event == 0:  # torch creates its event at the first record
            ev.record()
    check(lib().rac_time_next_kernel(ctypes.c_void_p(start.cuda_event),
                                     ctypes.c_void_p(stop.cuda_event)), "rac_time_next_kernel")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_qkv(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or (v is not None and v.dim() != 4):
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, D) or (v is not None and v.shape != k.shape):
        raise ValueError("k and v must be [B, Hkv, N, D] matching q %s" % (tuple(q.shape),))
    for t in (q, k) + ((v,) if v is not None else ()):
        if t.device.type != "cuda":
            raise ValueError("tensors must live on a HIP device")
        if t.device != q.device:
            raise ValueError("all tensors must be on the same device")
        if t.dtype != q.dtype:
            raise ValueError("q, k, v must share one dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, D]")
    if q.dtype not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float16, got %s" % q.dtype)
    return B, Hq, Hkv, N, D, _DTYPES[q.dtype]


def _outputs(q, out, lse, want_lse):
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != q.shape[:-1] or lse.dtype != torch.float32
                              or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 tensor [B, Hq, N]")
    return out, lse


def _pairing(pairing) -> int:
    """RAC_PAIR_* from a name ("adjacent", "half") or the integer itself."""
    if isinstance(pairing, str):
        if pairing not in PAIRINGS:
            raise ValueError("pairing must be one of %s" % sorted(PAIRINGS))
        return PAIRINGS[pairing]
    return int(pairing)


def attn_rope_causal_fwd(q, k, v, rope_base: float, out=None, lse=None, want_lse: bool = True):
    """Fused path: RoPE on Q/K inside the causal attention kernel. Returns (out, lse)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, v)
    out, lse = _outputs(q, out, lse, want_lse)
    with torch.cuda.device(q.device):
        rc = lib().attn_rope_causal_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        B, Hq, Hkv, N, D, float(rope_base), dt,
                                        _stream(q.device))
    check(rc, "attn_rope_causal_fwd")
    return out, lse


def attn_rope_causal_fwd_noalloc(q, k, v, rope_base: float, out=None, lse=None,
                                 want_lse: bool = True):
    """attn_rope_causal_fwd with the cos/sin table in the library's static
    device array (the C entry point allocates nothing; pass `out` and `lse`
    to allocate nothing here either). Returns (out, lse)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, v)
    out, lse = _outputs(q, out, lse, want_lse)
    with torch.cuda.device(q.device):
        rc = lib().attn_rope_causal_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                B, Hq, Hkv, N, D, float(rope_base), dt,
                                                _stream(q.device))
    check(rc, "attn_rope_causal_fwd_noalloc")
    return out, lse


def attn_rope_causal_fwd_ex(q, k, v, rope_base: float, pairing="adjacent", out=None, lse=None,
                            want_lse: bool = True):
    """The fused path with a choice of RoPE pairing ("adjacent" or "half"). Returns (out, lse)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, v)
    out, lse = _outputs(q, out, lse, want_lse)
    with torch.cuda.device(q.device):
        rc = lib().attn_rope_causal_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                           B, Hq, Hkv, N, D, float(rope_base), _pairing(pairing),
                                           dt, _stream(q.device))
    check(rc, "attn_rope_causal_fwd_ex")
    return out, lse


def attn_alibi_causal_fwd(q, k, v, slopes, rope_base=None, pairing="adjacent", out=None,
                          lse=None, want_lse: bool = True):
    """Causal attention with the ALiBi penalty -slopes[h] * (i - j) on the scaled
    scores; slopes: fp32 tensor [Hq] on q's device. With rope_base given, RoPE
    (``pairing``) is fused as well. Returns (out, lse)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, v)
    if slopes.shape != (Hq,) or slopes.dtype != torch.float32 or slopes.device != q.device \
            or not slopes.is_contiguous():
        raise ValueError("slopes must be a contiguous fp32 tensor [Hq] on q's device")
    out, lse = _outputs(q, out, lse, want_lse)
    pr = RAC_ROPE_NONE if rope_base is None else _pairing(pairing)
    with torch.cuda.device(q.device):
        rc = lib().attn_alibi_causal_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                         B, Hq, Hkv, N, D, _ptr(slopes),
                                         float(rope_base or 0.0), pr, dt, _stream(q.device))
    check(rc, "attn_alibi_causal_fwd")
    return out, lse


def _rot_outputs(q, k, q_rot, k_rot):
    q_rot = torch.empty_like(q) if q_rot is None else q_rot
    k_rot = torch.empty_like(k) if k_rot is None else k_rot
    for src, dst in ((q, q_rot), (k, k_rot)):
        if dst.shape != src.shape or dst.dtype != src.dtype or not dst.is_contiguous() \
                or dst.device != src.device:
            raise ValueError("q_rot/k_rot must be contiguous tensors like q/k")
    return q_rot, k_rot


def rope_prerotate(q, k, rope_base: float, q_rot=None, k_rot=None):
    """Pre-rotation pass. Returns (q_rot, k_rot); pass q_rot=q, k_rot=k for in place."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, None)
    q_rot, k_rot = _rot_outputs(q, k, q_rot, k_rot)
    with torch.cuda.device(q.device):
        rc = lib().rope_prerotate(_ptr(q), _ptr(k), _ptr(q_rot), _ptr(k_rot), B, Hq, Hkv, N, D,
                                  float(rope_base), dt, _stream(q.device))
    check(rc, "rope_prerotate")
    return q_rot, k_rot


def rope_prerotate_ex(q, k, rope_base: float, pairing="adjacent", q_rot=None, k_rot=None):
    """The pre-rotation pass with a choice of RoPE pairing. Returns (q_rot, k_rot)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, None)
    q_rot, k_rot = _rot_outputs(q, k, q_rot, k_rot)
    with torch.cuda.device(q.device):
        rc = lib().rope_prerotate_ex(_ptr(q), _ptr(k), _ptr(q_rot), _ptr(k_rot), B, Hq, Hkv, N,
                                     D, float(rope_base), _pairing(pairing), dt,
                                     _stream(q.device))
    check(rc, "rope_prerotate_ex")
    return q_rot, k_rot


def attn_causal_fwd(q, k, v, out=None, lse=None, want_lse: bool = True):
    """Causal attention on already-rotated inputs. Returns (out, lse)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, v)
    out, lse = _outputs(q, out, lse, want_lse)
    with torch.cuda.device(q.device):
        rc = lib().attn_causal_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                   B, Hq, Hkv, N, D, dt, _stream(q.device))
    check(rc, "attn_causal_fwd")
    return out, lse


def prerotate_path(q, k, v, rope_base: float, want_lse: bool = True, pairing="adjacent"):
    """The pre-rotation path: rope_prerotate then attn_causal_fwd. Returns (out, lse)."""
    if _pairing(pairing) == RAC_PAIR_ADJACENT:
        q_rot, k_rot = rope_prerotate(q, k, rope_base)
    else:
        q_rot, k_rot = rope_prerotate_ex(q, k, rope_base, pairing)
    return attn_causal_fwd(q_rot, k_rot, v, want_lse=want_lse)


def rope_prerotate_k(k, rope_base: float, k_rot=None):
    """Pre-rotation of K alone (the GQA split path). Returns k_rot; k_rot=k is in place."""
    B, Hkv, Hkv2, N, D, dt = _check_qkv(k, k, None)
    k_rot = torch.empty_like(k) if k_rot is None else k_rot
    if k_rot.shape != k.shape or k_rot.dtype != k.dtype or not k_rot.is_contiguous() \
            or k_rot.device != k.device:
        raise ValueError("k_rot must be a contiguous tensor like k")
    with torch.cuda.device(k.device):
        rc = lib().rope_prerotate_k(_ptr(k), _ptr(k_rot), B, Hkv, N, D, float(rope_base), dt,
                                    _stream(k.device))
    check(rc, "rope_prerotate_k")
    return k_rot


def stream_copy(src, dst) -> None:
    """A plain device copy of src into dst (contiguous, same byte size) with
    the pre-rotation pass's access pattern: its bandwidth ceiling."""
    if not (src.is_contiguous() and dst.is_contiguous()) or src.device != dst.device:
        raise ValueError("src and dst must be contiguous tensors on one device")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must hold the same number of bytes")
    with torch.cuda.device(src.device):
        rc = lib().rac_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(src.device))
    check(rc, "rac_stream_copy")


def attn_rope_q_causal_fwd(q, k_rot, v, rope_base: float, out=None, lse=None,
                           want_lse: bool = True):
    """Causal attention rotating Q in the kernel; K already rotated. Returns (out, lse)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k_rot, v)
    out, lse = _outputs(q, out, lse, want_lse)
    with torch.cuda.device(q.device):
        rc = lib().attn_rope_q_causal_fwd(_ptr(q), _ptr(k_rot), _ptr(v), _ptr(out), _ptr(lse),
                                          B, Hq, Hkv, N, D, float(rope_base), dt,
                                          _stream(q.device))
    check(rc, "attn_rope_q_causal_fwd")
    return out, lse


def split_path(q, k, v, rope_base: float, want_lse: bool = True):
    """The GQA split path: rope_prerotate_k then attn_rope_q_causal_fwd. Returns (out, lse)."""
    return attn_rope_q_causal_fwd(q, rope_prerotate_k(k, rope_base), v, rope_base,
                                  want_lse=want_lse)


def auto_plan(B: int, Hq: int, Hkv: int, N: int, D: int, dtype, workspace_bytes: int = 0):
    """(path, preferred_bytes): the RAC_PATH_* attn_rope_causal_auto takes for this shape
    with `workspace_bytes` of workspace, and the bytes its preferred path needs."""
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    path, need = ctypes.c_int(0), ctypes.c_size_t(0)
    check(lib().rac_auto_plan(B, Hq, Hkv, N, D, dt, int(workspace_bytes), ctypes.byref(path),
                              ctypes.byref(need)), "rac_auto_plan")
    return path.value, need.value


def attn_rope_causal_auto(q, k, v, rope_base: float, workspace=None, out=None, lse=None,
                          want_lse: bool = True):
    """RoPE + causal attention through the path the fitted cost model rates fastest.

    `workspace` is a caller-owned device tensor (any dtype, contiguous) for the rotated
    copies; None or too small falls back to a path that fits (the fused kernel needs
    none). auto_plan() gives the bytes the preferred path needs. Returns (out, lse)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, v)
    out, lse = _outputs(q, out, lse, want_lse)
    wbytes = 0
    if workspace is not None:
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        wbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        rc = lib().attn_rope_causal_auto(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                         B, Hq, Hkv, N, D, float(rope_base), dt,
                                         _ptr(workspace), wbytes, _stream(q.device))
    check(rc, "attn_rope_causal_auto")
    return out, lse


def _bwd_tensors(q, k, v, out, lse, dout):
    B, Hq, Hkv, N, D, dt = _check_qkv(q, k, v)
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError("%s must be a contiguous tensor like q" % name)
    if lse.shape != q.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be the forward's contiguous fp32 [B, Hq, N] log-sum-exp")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    return (B, Hq, Hkv, N, D, dt), (dq, dk, dv, delta)


def attn_rope_causal_bwd(q, k, v, out, lse, dout, rope_base: float):
    """Backward of attn_rope_causal_fwd: gradients with respect to the unrotated q, k and
    to v, from the forward's (out, lse) and dout. Returns (dq, dk, dv, delta)."""
    (B, Hq, Hkv, N, D, dt), (dq, dk, dv, delta) = _bwd_tensors(q, k, v, out, lse, dout)
    with torch.cuda.device(q.device):
        rc = lib().attn_rope_causal_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
                                        B, Hq, Hkv, N, D, float(rope_base), dt, _stream(q.device))
    check(rc, "attn_rope_causal_bwd")
    return dq, dk, dv, delta


def attn_rope_causal_bwd_ex(q, k, v, out, lse, dout, rope_base: float, pairing="adjacent"):
    """Backward of attn_rope_causal_fwd_ex with a choice of RoPE pairing ("adjacent" or
    "half"). Returns (dq, dk, dv, delta)."""
    (B, Hq, Hkv, N, D, dt), (dq, dk, dv, delta) = _bwd_tensors(q, k, v, out, lse, dout)
    with torch.cuda.device(q.device):
        rc = lib().attn_rope_causal_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                           _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
                                           B, Hq, Hkv, N, D, float(rope_base), _pairing(pairing),
                                           dt, _stream(q.device))
    check(rc, "attn_rope_causal_bwd_ex")
    return dq, dk, dv, delta


def attn_alibi_causal_bwd(q, k, v, out, lse, dout, slopes, rope_base=None, pairing="adjacent"):
    """Backward of attn_alibi_causal_fwd (same slopes, rope_base and pairing). Returns
    (dq, dk, dv, delta)."""
    (B, Hq, Hkv, N, D, dt), (dq, dk, dv, delta) = _bwd_tensors(q, k, v, out, lse, dout)
    if slopes.shape != (Hq,) or slopes.dtype != torch.float32 or not slopes.is_contiguous() \
            or slopes.device != q.device:
        raise ValueError("slopes must be a contiguous fp32 [Hq] tensor on q's device")
    pr = RAC_ROPE_NONE if rope_base is None else _pairing(pairing)
    with torch.cuda.device(q.device):
        rc = lib().attn_alibi_causal_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                         _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
                                         B, Hq, Hkv, N, D, _ptr(slopes),
                                         float(rope_base or 0.0), pr, dt, _stream(q.device))
    check(rc, "attn_alibi_causal_bwd")
    return dq, dk, dv, delta


def attn_causal_bwd(q, k, v, out, lse, dout):
    """Backward of attn_causal_fwd (q, k already rotated). Returns (dq, dk, dv, delta)."""
    (B, Hq, Hkv, N, D, dt), (dq, dk, dv, delta) = _bwd_tensors(q, k, v, out, lse, dout)
    with torch.cuda.device(q.device):
        rc = lib().attn_causal_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta),
                                   B, Hq, Hkv, N, D, dt, _stream(q.device))
    check(rc, "attn_causal_bwd")
    return dq, dk, dv, delta


def rope_prerotate_bwd(dq_rot, dk_rot, rope_base: float, dq=None, dk=None):
    """Backward of rope_prerotate: (dq, dk) = R(-p) (dq_rot, dk_rot); dq=dq_rot for in place."""
    return rope_prerotate_bwd_ex(dq_rot, dk_rot, rope_base, "adjacent", dq, dk)


def rope_prerotate_bwd_ex(dq_rot, dk_rot, rope_base: float, pairing="adjacent", dq=None,
                          dk=None):
    """Backward of rope_prerotate_ex with a choice of RoPE pairing. Returns (dq, dk)."""
    B, Hq, Hkv, N, D, dt = _check_qkv(dq_rot, dk_rot, None)
    dq = torch.empty_like(dq_rot) if dq is None else dq
    dk = torch.empty_like(dk_rot) if dk is None else dk
    for src, dst in ((dq_rot, dq), (dk_rot, dk)):
        if dst.shape != src.shape or dst.dtype != src.dtype or not dst.is_contiguous() \
                or dst.device != src.device:
            raise ValueError("dq/dk must be contiguous tensors like dq_rot/dk_rot")
    with torch.cuda.device(dq_rot.device):
        rc = lib().rope_prerotate_bwd_ex(_ptr(dq_rot), _ptr(dk_rot), _ptr(dq), _ptr(dk), B, Hq,
                                         Hkv, N, D, float(rope_base), _pairing(pairing), dt,
                                         _stream(dq_rot.device))
    check(rc, "rope_prerotate_bwd_ex")
    return dq, dk


def prerotate_path_bwd(q, k, v, out, lse, dout, rope_base: float, pairing="adjacent"):
    """Backward of the pre-rotation path: rope_prerotate_ex (the rotated operands the forward
    used), attn_causal_bwd on them, rope_prerotate_bwd_ex. Returns (dq, dk, dv, delta)."""
    q_rot, k_rot = rope_prerotate_ex(q, k, rope_base, pairing)
    dq_rot, dk_rot, dv, delta = attn_causal_bwd(q_rot, k_rot, v, out, lse, dout)
    dq, dk = rope_prerotate_bwd_ex(dq_rot, dk_rot, rope_base, pairing, dq=dq_rot, dk=dk_rot)
    return dq, dk, dv, delta
