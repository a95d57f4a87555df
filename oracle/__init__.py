"""The fp64 CPU oracle for RoPE followed by causal softmax attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this package. The product path never does, and
the oracle shares no code with it: the arithmetic lives in ``rac_oracle.c``
(plain fp64 C, OpenMP over independent rows), this module only marshals numpy
arrays through ctypes.

What it follows (the pages define the method, this file restates it):

* RoPE -- "Fast and Exact Relative-Position Attention via Structure-Aware
  Kernels" (rainbus digest), background "RoPE and parameter-free position
  encodings": each query/key is rotated by an angle set by its absolute
  position. Readings where the pages are silent: adjacent pairs (2i, 2i+1),
  theta_i = base**(-2i/D), position = row index in the sequence,
  counter-clockwise turn by p*theta_i.
* Causal attention -- same digest, background "FlashAttention and online
  softmax" and the forward method (Algorithm 1: o_i = u_i / l_i and L_i),
  with scale 1/sqrt(D); MHA/GQA per "AttnFuse Makes RoPE a First-Class
  Attention Compilation Operation", paragraph 4.
* Backward -- the gradients of that attention with respect to q, k, v by the
  chain rule through the same definition (softmax Jacobian with
  Delta_i = sum_j P_ij dP_ij), and RoPE's gradient, the inverse rotation.
* Two variants of the rotated operands: ``exact`` (fp64 rotation) and
  ``rounded`` (fp64 rotation then one round-to-nearest-even to the storage
  dtype, i.e. what a separate pre-rotation pass writes to memory).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
invariants, closed forms, brute force and library routines.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"bf16": 0, "fp16": 1}


class Oracle:
    """The oracle's entry points, bound to one build of ``rac_oracle.c``."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        lib.oracle_decode.argtypes = [u16p, ctypes.c_int64, ctypes.c_int, f64p]
        lib.oracle_decode.restype = None
        lib.oracle_encode.argtypes = [f64p, ctypes.c_int64, ctypes.c_int, u16p]
        lib.oracle_encode.restype = None
        lib.oracle_rope.argtypes = [f64p, i64p, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                    f64p]
        lib.oracle_rope.restype = None
        lib.oracle_rope_half.argtypes = lib.oracle_rope.argtypes
        lib.oracle_rope_half.restype = None
        lib.oracle_attn_rows.argtypes = [f64p, f64p, f64p] + [ctypes.c_int] * 5 + [
            i64p, ctypes.c_int64, f64p, f64p]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_alibi_rows.argtypes = [f64p, f64p, f64p] + [ctypes.c_int] * 5 + [
            f64p, i64p, ctypes.c_int64, f64p, f64p]
        lib.oracle_attn_alibi_rows.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [f64p] * 4 + [ctypes.c_int] * 5 + [f64p] * 5
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_alibi_bwd.argtypes = [f64p] * 4 + [ctypes.c_int] * 5 + [f64p] * 6
        lib.oracle_attn_alibi_bwd.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def num_threads(self) -> int:
        """OpenMP threads the oracle runs with."""
        return int(self.lib.oracle_num_threads())

    def decode(self, bits: np.ndarray, dtype: str) -> np.ndarray:
        """bf16/fp16 bit patterns (uint16) -> exact fp64 values, same shape."""
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_decode(_ptr(b, ctypes.c_uint16), b.size, DTYPE_CODES[dtype],
                               _ptr(out, ctypes.c_double))
        return out

    def encode(self, x: np.ndarray, dtype: str) -> np.ndarray:
        """fp64 values -> bf16/fp16 bit patterns, one round-to-nearest-even."""
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.oracle_encode(_ptr(a, ctypes.c_double), a.size, DTYPE_CODES[dtype],
                               _ptr(out, ctypes.c_uint16))
        return out

    def rope(self, x: np.ndarray, positions, base: float, pairing: str = "adjacent") -> np.ndarray:
        """Rotate rows of ``x`` (shape [..., D], fp64) by their absolute positions.

        ``positions`` broadcasts against ``x.shape[:-1]``. ``pairing`` is
        "adjacent" (pairs (2i, 2i+1)) or "half" (pairs (i, i + D/2)).
        """
        a = np.ascontiguousarray(x, dtype=np.float64)
        D = a.shape[-1]
        if D % 2:
            raise ValueError("RoPE needs an even head dimension")
        pos = np.ascontiguousarray(np.broadcast_to(np.asarray(positions, dtype=np.int64),
                                                   a.shape[:-1]))
        out = np.empty_like(a)
        rows = a.size // D if D else 0
        fn = {"adjacent": self.lib.oracle_rope, "half": self.lib.oracle_rope_half}[pairing]
        fn(_ptr(a, ctypes.c_double), _ptr(pos, ctypes.c_int64), rows, D, float(base),
           _ptr(out, ctypes.c_double))
        return out

    def rope_bhnd(self, x: np.ndarray, base: float, pairing: str = "adjacent") -> np.ndarray:
        """RoPE on a [B, H, N, D] tensor: row n of every (b, h) sits at position n."""
        return self.rope(x, np.arange(x.shape[-2], dtype=np.int64), base, pairing)

    def attention(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, rows=None, slopes=None):
        """Causal softmax attention, fp64, two-pass.

        q [B, Hq, N, D]; k, v [B, Hkv, N, D]. ``rows`` (optional) lists the
        flattened query rows (b*Hq + h)*N + i to compute. ``slopes``
        (optional, Hq values) adds the ALiBi penalty -slopes[h] * (i - j) to
        the scaled scores. Returns (o, lse): with ``rows=None`` o is
        [B, Hq, N, D] and lse [B, Hq, N]; otherwise o is [len(rows), D] and
        lse [len(rows)].
        """
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        B, Hq, N, D = q.shape
        Hkv = k.shape[1]
        if k.shape != (B, Hkv, N, D) or v.shape != k.shape:
            raise ValueError("k and v must be [B, Hkv, N, D] matching q")
        if rows is None:
            o = np.empty(q.shape, dtype=np.float64)
            lse = np.empty(q.shape[:-1], dtype=np.float64)
            rp, nrows = None, 0
        else:
            r = np.ascontiguousarray(rows, dtype=np.int64)
            o = np.empty((r.size, D), dtype=np.float64)
            lse = np.empty((r.size,), dtype=np.float64)
            rp, nrows = _ptr(r, ctypes.c_int64), r.size
        if slopes is None:
            rc = self.lib.oracle_attn_rows(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                           _ptr(v, ctypes.c_double), B, Hq, Hkv, N, D, rp, nrows,
                                           _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
        else:
            sl = np.ascontiguousarray(slopes, dtype=np.float64)
            if sl.shape != (Hq,):
                raise ValueError("slopes must hold one value per query head")
            rc = self.lib.oracle_attn_alibi_rows(
                _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                B, Hq, Hkv, N, D, _ptr(sl, ctypes.c_double), rp, nrows,
                _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle attention: bad arguments")
        return o, lse

    def rope_attention(self, q_bits, k_bits, v_bits, dtype: str, base: float, rows=None,
                       variant: str = "rounded", pairing: str = "adjacent", slopes=None):
        """RoPE then causal attention, from bf16/fp16 bit patterns.

        ``variant="exact"`` feeds the fp64 rotation straight into attention;
        ``variant="rounded"`` first rounds the rotated q and k to ``dtype``.
        ``base=None`` skips the rotation (plain causal attention on the
        decoded inputs); ``slopes`` as in attention().
        Returns (o, lse, q_rot, k_rot) with q_rot/k_rot the fp64 operands used.
        """
        q = self.decode(q_bits, dtype)
        k = self.decode(k_bits, dtype)
        v = self.decode(v_bits, dtype)
        if base is None:
            qr, kr = q, k
        else:
            qr = self.rope_bhnd(q, base, pairing)
            kr = self.rope_bhnd(k, base, pairing)
        if variant == "rounded":
            qr = self.decode(self.encode(qr, dtype), dtype)
            kr = self.decode(self.encode(kr, dtype), dtype)
        elif variant != "exact":
            raise ValueError("variant must be 'exact' or 'rounded'")
        o, lse = self.attention(qr, kr, v, rows, slopes)
        return o, lse, qr, kr


    def attention_bwd(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                      slopes=None):
        """Gradients of the causal attention above, fp64, from the definition.

        q, dout [B, Hq, N, D]; k, v [B, Hkv, N, D]; ``slopes`` (Hq values) adds
        the ALiBi penalty of attention(..., slopes). Returns (dq, dk, dv, lse,
        delta): the gradients with respect to q, k and v (dk, dv summed over
        the query heads of each GQA group), and per query row L_i and
        Delta_i = sum_j P_ij dP_ij.
        """
        q, k, v, dout = (np.ascontiguousarray(t, dtype=np.float64) for t in (q, k, v, dout))
        B, Hq, N, D = q.shape
        Hkv = k.shape[1]
        if k.shape != (B, Hkv, N, D) or v.shape != k.shape or dout.shape != q.shape:
            raise ValueError("k, v must be [B, Hkv, N, D] and dout like q")
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dv = np.empty_like(v)
        lse = np.empty(q.shape[:-1], dtype=np.float64)
        delta = np.empty(q.shape[:-1], dtype=np.float64)
        p = lambda a: _ptr(a, ctypes.c_double)  # noqa: E731
        if slopes is None:
            rc = self.lib.oracle_attn_bwd(p(q), p(k), p(v), p(dout), B, Hq, Hkv, N, D, p(dq),
                                          p(dk), p(dv), p(lse), p(delta))
        else:
            sl = np.ascontiguousarray(slopes, dtype=np.float64).reshape(-1)
            if sl.shape != (Hq,):
                raise ValueError("slopes must hold one value per query head")
            rc = self.lib.oracle_attn_alibi_bwd(p(q), p(k), p(v), p(dout), B, Hq, Hkv, N, D,
                                                p(sl), p(dq), p(dk), p(dv), p(lse), p(delta))
        if rc != 0:
            raise ValueError("oracle_attn_bwd: bad arguments")
        return dq, dk, dv, lse, delta

    def rope_attention_bwd(self, q_bits, k_bits, v_bits, do_bits, dtype: str, base: float,
                           variant: str = "rounded", pairing: str = "adjacent", slopes=None):
        """Gradients of RoPE then causal attention with respect to the
        unrotated q, k and to v, from bf16/fp16 bit patterns.

        The attention gradients are taken at the rotated operands (``variant``
        as in rope_attention); RoPE's gradient is its inverse rotation, the
        turn by -p theta_i of the same pairs (``pairing`` as in rope()).
        ``base=None`` skips the rotation, ``slopes`` adds the ALiBi penalty
        (as in rope_attention). Returns (dq, dk, dv, delta, lse).
        """
        q = self.decode(q_bits, dtype)
        k = self.decode(k_bits, dtype)
        v = self.decode(v_bits, dtype)
        do = self.decode(do_bits, dtype)
        if base is None:
            qr, kr = q, k
        else:
            qr = self.rope_bhnd(q, base, pairing)
            kr = self.rope_bhnd(k, base, pairing)
        if variant == "rounded":
            qr = self.decode(self.encode(qr, dtype), dtype)
            kr = self.decode(self.encode(kr, dtype), dtype)
        elif variant != "exact":
            raise ValueError("variant must be 'exact' or 'rounded'")
        dqr, dkr, dv, lse, delta = self.attention_bwd(qr, kr, v, do, slopes)
        if base is None:
            return dqr, dkr, dv, delta, lse
        neg = -np.arange(q.shape[-2], dtype=np.int64)
        return (self.rope(dqr, neg, base, pairing), self.rope(dkr, neg, base, pairing), dv, delta,
                lse)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


_default = None


def default() -> Oracle:
    """The oracle built from this directory's rac_oracle.c (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        _default = Oracle(LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def decode(bits, dtype):
    return default().decode(bits, dtype)


def encode(x, dtype):
    return default().encode(x, dtype)


def rope(x, positions, base, pairing="adjacent"):
    return default().rope(x, positions, base, pairing)


def rope_bhnd(x, base, pairing="adjacent"):
    return default().rope_bhnd(x, base, pairing)


def attention(q, k, v, rows=None, slopes=None):
    return default().attention(q, k, v, rows, slopes)


def rope_attention(q_bits, k_bits, v_bits, dtype, base, rows=None, variant="rounded",
                   pairing="adjacent", slopes=None):
    return default().rope_attention(q_bits, k_bits, v_bits, dtype, base, rows, variant, pairing,
                                    slopes)


def attention_bwd(q, k, v, dout, slopes=None):
    return default().attention_bwd(q, k, v, dout, slopes)


def rope_attention_bwd(q_bits, k_bits, v_bits, do_bits, dtype, base, variant="rounded",
                       pairing="adjacent", slopes=None):
    return default().rope_attention_bwd(q_bits, k_bits, v_bits, do_bits, dtype, base, variant,
                                        pairing, slopes)
