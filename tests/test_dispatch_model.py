"""The dispatcher's path-cost model on the CPU: its constants come from the
committed fit, its C++ (csrc/dispatch_model.h, compiled here with the host
compiler) gives the same times as this module, the fit recovers known
parameters, the makespan schedules workgroups as the launch deals them, and
the closed-form crossover agrees with the model it summarises.
(rac_auto_plan against the model: tests/test_abi.py.)"""
import json
import math
import os
import shutil
import subprocess

import pytest

from rotary_position_embedding_causal_amd import dispatch_fit as M, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_constants_are_the_committed_fit():
    """csrc/dispatch_model.h holds the fit that profiles/crossover_fit.json
    records (printed to 9 significant digits)."""
    fit = json.load(open(M.SUMMARY))["model"]["fit"]
    hdr = M.load_params()
    for cls in M.CLASSES:
        for name in M.CLASS_PARAMS:
            assert hdr[cls][name] == pytest.approx(fit[cls][name], rel=1e-8, abs=1e-12), (cls, name)
    for name in M.GLOBAL_PARAMS:
        assert hdr[name] == pytest.approx(fit[name], rel=1e-8, abs=1e-12), name


# shapes across both launch shapes, XCD-divisible and not, beyond the
# per-XCD job cap, ragged N, and the planner's extremes
SHAPES = [(1, 16, 16, 1024, 64), (1, 16, 16, 8192, 64), (1, 16, 16, 6144, 64),
          (1, 32, 32, 3072, 128), (8, 32, 32, 1024, 128), (1, 32, 8, 2048, 128),
          (1, 32, 8, 3072, 128), (4, 32, 8, 4096, 128), (1, 64, 8, 1536, 128),
          (3, 24, 8, 2000, 64), (1, 4, 4, 300, 64), (2, 6, 2, 4095, 128), (1, 1, 1, 1, 64),
          (64, 64, 8, 65536, 128), (20000, 16, 16, 32768, 128), (65535, 32, 8, 4096, 64),
          (0, 16, 16, 4096, 64)]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_header_cpp_times_equal_the_model(tmp_path):
    """The C++ that rac_auto_plan runs and this module's model give the same
    three path times (to the last bits: same constants, same arithmetic)."""
    src = tmp_path / "times.cpp"
    calls = "".join("    show(%d, %d, %d, %d, %d);\n" % s for s in SHAPES)
    src.write_text('#include <stdio.h>\n#include "dispatch_model.h"\n'
                   "static void show(int B, int Hq, int Hkv, int N, int D) {\n"
                   "    double f, p, s;\n"
                   "    rac_model::path_times(B, Hq, Hkv, N, D, &f, &p, &s);\n"
                   '    printf("%.17g %.17g %.17g\\n", f, p, s);\n}\n'
                   "int main() {\n" + calls + "    return 0;\n}\n")
    exe = tmp_path / "times"
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off",
                    "-I" + os.path.dirname(M.HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    p = M.load_params()
    for shape, line in zip(SHAPES, out):
        got = [float(x) for x in line.split()]
        t = M.model_us(p, *shape)
        for g, w in zip(got, (t["fused"], t["prerotate"], t["split"])):
            assert g == pytest.approx(w, rel=1e-13, abs=1e-9), shape


def _list_schedule(weights, slots):
    """Reference list scheduling: each job in order to a least-loaded slot."""
    loads = [0.0] * slots
    for w in weights:
        i = min(range(slots), key=lambda j: loads[j])
        loads[i] += w
    return max(loads)


@pytest.mark.parametrize("shape", [(1, 32, 8, 3072, 128), (1, 16, 16, 6144, 64),
                                   (1, 6, 2, 2048, 128), (2, 16, 16, 1024, 64),
                                   (1, 16, 16, 8192, 64), (1, 24, 8, 1100, 64),
                                   (1, 16, 16, 1024, 64), (1, 32, 32, 3584, 128)])
def test_makespan_is_the_per_xcd_list_schedule(shape):
    """makespan() against a plain list schedule built from the launch's own
    unit decoding (attn_fwd.hip decode_unit: XCD-aware order, GQA packs)."""
    B, Hq, Hkv, N, D = shape
    r = 2.75
    kind, units, per_head, packs, slots, base = M.launch(B, Hq, Hkv, N, D)
    div = units % M.NXCD == 0
    want = 0.0
    for x in range(M.NXCD):
        us = range(x * (units // 8), (x + 1) * (units // 8)) if div else range(x, units, 8)
        ws = [base[(u // packs) % per_head] + r for u in us]
        if ws:
            want = max(want, _list_schedule(ws, slots))
    got_kind, got = M.makespan(B, Hq, Hkv, N, D, r)
    assert got_kind == kind
    assert got == pytest.approx(want, rel=1e-12)


def test_makespan_launch_shapes_and_cap():
    # the pair launch: equal work per workgroup, one round of CUs at B = 1,
    # N = 2048, GQA 32/8: 8 pairs x 32 heads, each (len_l + len_h + 1) / 2 = 17 steps
    kind, m = M.makespan(1, 32, 8, 2048, 128, 0.0)
    assert kind == "pair" and m == 17.0
    # two rounds for MHA at exactly 512 pairs
    assert M.makespan(1, 16, 16, 8192, 64, 1.0) == ("pair", 2 * (65 + 1.0))
    # a short sequence takes the tile launch (too few pairs): the heaviest
    # query tile sets the time
    kind, m = M.makespan(1, 4, 4, 300, 64, 0.0)
    assert kind == "tile" and m == M.kv_tiles_of(2, 300) == 5
    # the launch rule of attn_fwd.hip: under half a round, pairs from 4 query
    # tiles for even GQA groups and from 12 for MHA; for MHA at D = 128 also
    # at 1.5-2 rounds, at D = 64 at exactly two
    assert M.launch(1, 8, 2, 512, 128)[0] == "pair" and M.launch(1, 8, 2, 256, 128)[0] == "tile"
    assert M.launch(1, 16, 16, 1536, 64)[0] == "pair"
    assert M.launch(1, 16, 16, 1280, 64)[0] == "tile"
    assert M.launch(1, 32, 32, 3072, 128)[0] == "pair" and M.launch(1, 32, 32, 3072, 64)[0] == "tile"
    assert M.launch(1, 32, 32, 2560, 128)[0] == "tile" and M.launch(1, 32, 8, 3072, 128)[0] == "tile"
    # past the job cap: the mean load plus half the heaviest workgroup
    B, Hq, Hkv, N = 512, 32, 8, 4096
    kind, units, per_head, packs, slots, base = M.launch(B, Hq, Hkv, N, 128)
    assert units // M.NXCD > M.JOB_CAP
    total = sum(base) * packs * (units // (per_head * packs)) + 0.5 * units
    kind, m = M.makespan(B, Hq, Hkv, N, 128, 0.5)
    assert m == pytest.approx(total / M.NXCD / slots + 0.5 * (max(base) + 0.5), rel=1e-12)
    assert M.makespan(0, 16, 16, 4096, 64, 3.0)[1] == 0.0


def _params():
    p = {"eta_bw": 0.8, "t0_us": 3.0, "t_gap_us": 1.5}
    for i, cls in enumerate(M.CLASSES):
        p[cls] = {"wg_steps": (1.5, 2.75, 4.0, 3.25)[i]}
        for j, k in enumerate(M.KERNELS):
            p[cls]["launch_us_" + k] = 0.5 + 0.25 * j + 0.1 * i
            p[cls]["pair_us_" + k] = (1.5 + 0.3 * i) * (1.0, 1.3, 1.05)[j]
            p[cls]["tile_us_" + k] = (1.2 + 0.3 * i) * (1.0, 1.25, 1.04)[j]
    return p


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
        shape, m = M.makespan(B, Hq, Hkv, N, D, c["wg_steps"])
        r = dict(B=B, Hq=Hq, Hkv=Hkv, N=N, D=D,
                 k_attn=M.kernel_us(c, "attn", shape, m),
                 k_fused=M.kernel_us(c, "fused", shape, m),
                 k_attn_q=M.kernel_us(c, "q", shape, m),
                 k_rope=M.pass_us(p, M.pass_bytes(B, Hq + Hkv, N, D)),
                 k_rope_k=M.pass_us(p, M.pass_bytes(B, Hkv, N, D)))
        r["c_fused"] = r["k_fused"] + 2.0
        r["c_prerotate"] = r["k_rope"] + r["k_attn"] + 2.0 + p["t_gap_us"]
        rows.append(r)
    return rows


def test_fit_recovers_the_parameters_that_made_the_times():
    """From times the model made, the fit finds the workgroup overhead on its
    grid and every kernel constant, and reproduces every time."""
    p = _params()
    rows = _synthetic_rows(p)
    got = M.fit(rows)
    for cls in M.CLASSES:
        assert got[cls]["wg_steps"] == p[cls]["wg_steps"], cls
        for name in M.CLASS_PARAMS[1:]:
            assert got[cls][name] == pytest.approx(p[cls][name], rel=1e-6, abs=1e-6), (cls, name)
    for k, v in M.fit_errors(got, rows).items():
        assert v["max_abs"] < 1e-6, k
    assert got["eta_bw"] == pytest.approx(0.8, rel=1e-9)
    assert got["t0_us"] == pytest.approx(3.0, rel=1e-9)
    assert got["t_gap_us"] == pytest.approx(1.5, rel=1e-9)


def test_asymptote_alphas_are_the_step_ratios():
    """Without the launch constant, the full-chip alpha is the tile launch's
    per-step ratio, and the pair figure the pair launch's."""
    p = _params()
    for cls in M.CLASSES:
        for k in M.KERNELS:
            p[cls]["launch_us_" + k] = 0.0
    a = M.asymptote(p, 32, 8, 128)
    c = p["d128_gqa"]
    assert a["alpha_qk"] == pytest.approx(c["tile_us_fused"] / c["tile_us_attn"] - 1.0, rel=1e-12)
    assert a["alpha_q"] == pytest.approx(c["tile_us_q"] / c["tile_us_attn"] - 1.0, rel=1e-12)
    assert a["alpha_qk_pair"] == pytest.approx(c["pair_us_fused"] / c["pair_us_attn"] - 1.0)
    # eta: the flop rate of a long sequence against the peak, below 1
    assert 0.0 < a["eta_attn"] < 1.0 and a["eta_fused"] < a["eta_attn"]


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 16, 64), (32, 8, 128), (64, 8, 128)])
def test_closed_form_is_the_model_crossover_when_the_chip_is_full(Hq, Hkv, D):
    """With no fixed costs and a small rotation cost (alpha = 1 %, so that N*
    lies where the chip is full), the model's fused and pre-rotation times
    meet within 2 % of the closed form ((Hq + Hkv) / Hq) * 2 * eta P /
    (eta_bw BW) / alpha."""
    p = _params()
    p["t0_us"] = p["t_gap_us"] = 0.0
    for cls in M.CLASSES:
        c = p[cls]
        c["wg_steps"] = 0.0
        for k in M.KERNELS:
            c["launch_us_" + k] = 0.0
        c["tile_us_fused"] = 1.01 * c["tile_us_attn"]
        c["pair_us_fused"] = 1.01 * c["pair_us_attn"]
    n_closed = M.n_star_closed(p, Hq, Hkv, D)
    ns = sorted({int(n_closed * 2 ** (j / 40.0)) // 128 * 128 for j in range(-40, 41)})
    n_model = M.n_star_model(p, 1, Hq, Hkv, D, ns=ns)
    assert n_model == pytest.approx(n_closed, rel=0.02)
    a = M.asymptote(p, Hq, Hkv, D)
    assert a["alpha_qk"] == pytest.approx(0.01, rel=1e-9)
    # proportional to the peak-compute to bandwidth ratio
    assert n_closed == pytest.approx(((Hq + Hkv) / Hq) * 2 * a["eta_attn"] * M.MFMA_PEAK
                                     / (0.8 * M.HBM_BW) / 0.01)


def test_locate_interpolates_the_first_sign_change():
    assert M.locate([1000, 2000, 4000], [1.0, 1.0, 3.0], [2.0, 0.5, 1.0]) == pytest.approx(
        math.exp(math.log(1000) + 0.5 / 1.5 * math.log(2)))
    assert M.locate([1, 2], [1.0, 1.0], [2.0, 2.0]) is None


def test_model_times_grow_with_the_work():
    """Twice the sequence never costs less; neither does twice the batch
    under the same launch shape (a larger batch can move a short sequence
    from the one-tile launch to the paired one, which the model prices by its
    own step time); every time is finite and positive."""
    p = M.load_params()
    for D in (64, 128):
        for Hq, Hkv in ((16, 16), (32, 8), (64, 8)):
            for N in (128, 512, 1024, 1536, 2048, 3072, 4096, 8192, 16384):
                t = M.model_us(p, 1, Hq, Hkv, N, D)
                assert all(math.isfinite(v) and v > 0 for v in t.values())
                t2n = M.model_us(p, 1, Hq, Hkv, 2 * N, D)
                same = M.launch(1, Hq, Hkv, N, D)[0] == M.launch(2, Hq, Hkv, N, D)[0]
                t2b = M.model_us(p, 2, Hq, Hkv, N, D)
                for k in t:
                    assert t2n[k] > t[k], (Hq, Hkv, N, D, k)
                    assert t2b[k] >= t[k] or not same, (Hq, Hkv, N, D, k)
