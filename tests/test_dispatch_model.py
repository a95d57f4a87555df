"""The dispatcher's path-cost model on the CPU: its constants come from the
committed fit, the fit recovers known parameters, and the closed-form
crossover agrees with the model it summarises. (rac_auto_plan against the
model: tests/test_abi.py.)"""
import json
import math
import os

import pytest

from rotary_position_embedding_causal_amd import dispatch_fit as M, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_constants_are_the_committed_fit():
    """csrc/dispatch_model.h holds the fit that profiles/crossover_fit.json
    records (printed to 6 significant digits)."""
    fit = json.load(open(M.SUMMARY))["model"]["fit"]
    hdr = M.load_params()
    for cls in M.CLASSES:
        for name in M.CLASS_PARAMS:
            assert hdr[cls][name] == pytest.approx(fit[cls][name], rel=1e-5), (cls, name)
    for name in M.GLOBAL_PARAMS:
        assert hdr[name] == pytest.approx(fit[name], rel=1e-5, abs=1e-9), name


def _synthetic_rows(p):
    """Kernel and call times that the model with parameters p predicts exactly,
    over the crossover families' shapes plus two batch sizes."""
    names = [n for _, rows in inputs.CROSSOVER_FAMILIES.values() for n in rows]
    names += list(inputs.CROSSOVER_EXTRA)
    rows = []
    for n in names:
        w = inputs.WORKLOADS[n]
        B, Hq, Hkv, N, D = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"]
        c = p[M.class_key(D, Hq, Hkv)]
        r = dict(B=B, Hq=Hq, Hkv=Hkv, N=N, D=D,
                 k_attn=M.kernel_us(c, "attn", B, Hq, N, D),
                 k_fused=M.kernel_us(c, "fused", B, Hq, N, D),
                 k_attn_q=M.kernel_us(c, "q", B, Hq, N, D),
                 k_rope=M.pass_us(p, M.pass_bytes(B, Hq + Hkv, N, D)),
                 k_rope_k=M.pass_us(p, M.pass_bytes(B, Hkv, N, D)))
        r["c_fused"] = r["k_fused"] + 2.0
        r["c_prerotate"] = r["k_rope"] + r["k_attn"] + 2.0 + p["t_gap_us"]
        rows.append(r)
    return rows


def _params():
    p = {"eta_bw": 0.8, "t0_us": 3.0, "t_gap_us": 1.5}
    for i, cls in enumerate(M.CLASSES):
        p[cls] = {"eta_attn": 0.30 + 0.02 * i, "tpro_us_attn": 8.0 + 0.5 * i,
                  "tile_us_attn": 1.2 + 0.3 * i,
                  "eta_fused": 0.25 + 0.01 * i, "tpro_us_fused": 7.5 + 0.5 * i,
                  "tile_us_fused": 1.6 + 0.3 * i,
                  "eta_q": 0.29 + 0.02 * i, "tpro_us_q": 8.25 + 0.5 * i,
                  "tile_us_q": 1.3 + 0.3 * i}
    return p


def test_fit_recovers_the_parameters_that_made_the_times():
    """Every class's fit reproduces the times it was given; where a class
    has several rows in each regime (D = 64: three under-filled, four full)
    its parameters are the ones that made them. (With one under-filled row,
    prologue and per-tile cost are not separable, and only the times are.)"""
    p = _params()
    rows = _synthetic_rows(p)
    got = M.fit(rows)
    for r in rows:
        c = got[M.class_key(r["D"], r["Hq"], r["Hkv"])]
        for k, key in (("attn", "k_attn"), ("fused", "k_fused"), ("q", "k_attn_q")):
            assert M.kernel_us(c, k, r["B"], r["Hq"], r["N"], r["D"]) == pytest.approx(
                r[key], rel=5e-3), (r, k)
    for cls in ("d64_mha", "d64_gqa"):
        for name in M.CLASS_PARAMS:
            # the grids' last steps: 10^(1/2400) (0.1 %) and 0.05 us
            tol = dict(abs=0.051) if name.startswith("tpro") else dict(rel=3e-3)
            assert got[cls][name] == pytest.approx(p[cls][name], **tol), (cls, name)
    assert got["eta_bw"] == pytest.approx(0.8, rel=1e-9)
    assert got["t0_us"] == pytest.approx(3.0, rel=1e-9)
    assert got["t_gap_us"] == pytest.approx(1.5, rel=1e-9)


def test_fit_alphas_are_the_rotation_cost():
    p = _params()
    a = M.alphas(p["d64_mha"])
    assert a["alpha_qk"] == pytest.approx(0.30 / 0.25 - 1.0)
    assert a["alpha_qk_underfilled"] == pytest.approx(1.6 / 1.2 - 1.0)


@pytest.mark.parametrize("Hq,Hkv", [(16, 16), (32, 8), (64, 8)])
def test_closed_form_is_the_model_crossover_when_the_chip_is_full(Hq, Hkv):
    """With no under-filled term and no fixed costs, the model's fused and
    pre-rotation times meet exactly at the closed form
    ((Hq + Hkv) / Hq) * 2 * eta P / (eta_bw BW) / alpha."""
    p = _params()
    p["t0_us"] = p["t_gap_us"] = 0.0
    for cls in M.CLASSES:
        for k in M.KERNELS:
            p[cls]["tile_us_" + k] = p[cls]["tpro_us_" + k] = 0.0
    c = p[M.class_key(128, Hq, Hkv)]
    n_closed = M.n_star_closed(c, p, Hq, Hkv)
    t = M.model_us(p, 1, Hq, Hkv, n_closed, 128, gap=False)
    assert t["fused"] == pytest.approx(t["prerotate"], rel=1e-12)
    n_scan = M.n_star_model(p, 1, Hq, Hkv, 128)
    assert n_scan == pytest.approx(n_closed, rel=1e-3)
    # proportional to the peak-compute to bandwidth ratio
    assert n_closed == pytest.approx(((Hq + Hkv) / Hq) * 2 * c["eta_attn"] * M.MFMA_PEAK
                                     / (0.8 * M.HBM_BW) / (c["eta_attn"] / c["eta_fused"] - 1))


def test_model_times_are_monotonic_in_the_work():
    p = M.load_params()
    for D in (64, 128):
        for Hq, Hkv in ((16, 16), (32, 8)):
            prev = None
            for N in (128, 512, 1024, 4096, 16384, 65536):
                t = M.model_us(p, 1, Hq, Hkv, N, D)
                if prev:
                    assert all(t[k] > prev[k] for k in t)
                prev = t
                t2 = M.model_us(p, 4, Hq, Hkv, N, D)
                assert all(t2[k] >= t[k] for k in t)
                assert all(math.isfinite(v) and v > 0 for v in t.values())
