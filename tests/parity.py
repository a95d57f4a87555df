"""Helpers shared by the GPU parity tests: oracle references on the same seeded
bits the GPU sees, and the error measures the bounds are stated in.

Bounds (bf16/fp16 outputs against the fp64 oracle): O max-abs <= 2e-2 and
relative L2 <= 1e-2 against both the exact and the rounded-rotation oracle;
LSE max-abs <= 1e-3 against the rounded-rotation oracle (the rotated
operands the kernels feed to the matrix cores are bf16/fp16 values, and the
rounded variant uses exactly those, so the LSE comparison measures the
attention arithmetic; against the exact rotation, bf16 operand rounding
alone moves LSE by a few 1e-3, which is reported, not bounded).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from rotary_position_embedding_causal_amd import inputs

O_MAXABS = 2e-2
O_RELL2 = 1e-2
LSE_MAXABS = 1e-3


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return inputs.bits(t.detach().cpu())


def o_errors(got: np.ndarray, ref: np.ndarray):
    d = got - ref
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def assert_o(got, ref, what=""):
    mx, rel = o_errors(got, ref)
    assert mx <= O_MAXABS and rel <= O_RELL2, "%s: max|dO|=%.3e relL2=%.3e" % (what, mx, rel)
    return mx, rel


def assert_lse(got, ref, what=""):
    mx = float(np.max(np.abs(got - ref)))
    assert mx <= LSE_MAXABS, "%s: max|dLSE|=%.3e" % (what, mx)
    return mx


def sampled_rows(B, H, N, rng, per_head=24):
    """Query rows to check at sizes where the oracle cannot do every row:
    the first and last rows, rows around tile edges, and random rows."""
    fixed = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, N // 2, N - 2, N - 1]
    out = {}
    heads = [(b, h) for b in range(B) for h in range(H)]
    if len(heads) > 8:
        idx = rng.choice(len(heads), 8, replace=False)
        heads = [heads[i] for i in sorted(idx)] + [heads[0], heads[-1]]
    for bh in heads:
        rows = set(i for i in fixed if 0 <= i < N)
        rows.update(rng.integers(0, N, per_head).tolist())
        out[bh] = np.array(sorted(rows), dtype=np.int64)
    return out


def oracle_rows(q_bits, k_bits, v_bits, dtype, base, Hq, Hkv, rows_by_head, variant,
                pairing="adjacent"):
    """Oracle output and LSE for selected rows of selected (b, h).

    Rotates only the heads involved; returns {(b, h): (o [r, D], lse [r])}."""
    res = {}
    group = Hq // Hkv
    for (b, h), rows in rows_by_head.items():
        g = h // group
        q = oracle.decode(q_bits[b, h], dtype)[None, None]
        k = oracle.decode(k_bits[b, g], dtype)[None, None]
        v = oracle.decode(v_bits[b, g], dtype)[None, None]
        qr = oracle.rope_bhnd(q, base, pairing)
        kr = oracle.rope_bhnd(k, base, pairing)
        if variant == "rounded":
            qr = oracle.decode(oracle.encode(qr, dtype), dtype)
            kr = oracle.decode(oracle.encode(kr, dtype), dtype)
        res[(b, h)] = oracle.attention(qr, kr, v, rows=rows)
    return res


# Backward bounds (gradients against the fp64 oracle). The forward's O bounds
# carried over, with the max-abs bound scaled by the tensor's largest
# magnitude: gradients, unlike O (a convex combination of N(0,1) values), are
# not of unit size (dv_j sums dO over every row that sees key j). The error
# sources are the bf16/fp16 roundings of P and dS before the matrix products
# and of the outputs (unit roundoff 2^-9 for bf16): rel-L2 1e-2 is ~5 of them.
G_MAXABS_REL = 2e-2
G_RELL2 = 1e-2


# Peaked softmax (a steep ALiBi slope): dS = P (dP - Delta) cancels where a
# row's P is nearly one-hot, and Delta = rowsum(dO * O) is formed from the
# stored, rounded O, as the two-pass backward defines it, so O's rounding
# reaches dq and dk amplified (fp16's 8x finer rounding cuts the error 8x).
# rel-L2 bound for dq, dk in bf16 when the penalty is at least one unit of
# score per position.
G_RELL2_PEAKED = 2.5e-2


def assert_grad(got, ref, what="", rel_bound=G_RELL2):
    d = got - ref
    scale = max(1.0, float(np.max(np.abs(ref))))
    mx = float(np.max(np.abs(d)))
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    assert mx <= G_MAXABS_REL * scale and (rel <= rel_bound or np.linalg.norm(ref) < 1e-30), \
        "%s: max|d|=%.3e (bound %.3e) relL2=%.3e (bound %.1e)" % (
            what, mx, G_MAXABS_REL * scale, rel, rel_bound)
    return mx, rel
