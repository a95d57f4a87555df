"""The path-cost model behind attn_rope_causal_auto, and its fit to kernel times.

"AttnFuse Makes RoPE a First-Class Attention Compilation Operation"
(tdteach paper-news, 2026-09-13), paragraph 3, states the trade-off:
pre-rotation is a memory-bandwidth cost (Q and K read and written once more),
in-kernel rotation a compute-and-tiling cost, so which one wins follows from
the GPU's compute-to-bandwidth ratio; paragraph 5 adds that the choice has to
be measured per architecture and shape. The AttnFuse abstract (arxivdaily
2609.13612) says a crossover derived that way matches measurement. The pages
print no formula; the reading written out here is the plain one:

  kernel      T = max(F / (eta * P),  t_pro + t_tile * N / 128)
              F = 2 B Hq N^2 D (causal), P = the dense MFMA peak. The first
              term is a full chip; the second an under-filled one, where too
              few workgroups run to fill it and time is one workgroup's
              prologue (Q rows, first tiles) plus its N / 128 key tiles.
              Each attention kernel has its own (eta, t_pro, t_tile): plain
              (T_attn), rotating Q and K tiles (T_fused), rotating Q rows
              only (T_q); the rotation's cost is alpha = eta_attn /
              eta_fused - 1 on a full chip and t_tile_fused / t_tile_attn
              - 1 per key tile on an under-filled one
  pass        T_pass  = t0 + bytes / (eta_bw * BW)    (BW = 8 TB/s HBM peak)
              bytes = 2 x (the rotated heads) x B N D x 2 bytes, read + write
  fused       T_fused
  pre-rotate  T_pre   = T_pass(Hq + Hkv heads) + T_attn + t_gap
  GQA split   T_split = T_pass(Hkv heads) + T_q + t_gap

t_gap is what a second launch adds to a call (0 for the kernel-level
crossover). Setting T_fused = T_pre with both kernels in the throughput
regime and t0 = t_gap = 0 gives the closed form
  N* = ((Hq + Hkv) / Hq) * 2 bytes * (eta_attn P) / (eta_bw BW) / alpha,
proportional to P / BW as paragraph 3 says.

The parameters are fitted per class of shape -- head dim 64 or 128, MHA or
GQA (Hq / Hkv >= 2) -- from kernel times measured on MI355X, and the fitted
values are the constants of csrc/dispatch_model.h, which the C dispatcher
evaluates; this module parses that header so that tests can check the C
planner against the model. Nothing here runs on the product path.
"""
from __future__ import annotations

import math
import os
import re

MFMA_PEAK = 2516.6e12   # MI355X dense bf16/fp16, FLOP/s (published)
HBM_BW = 8.0e12         # MI355X HBM3E, B/s (published)
CLASSES = ("d64_mha", "d128_mha", "d64_gqa", "d128_gqa")
KERNELS = ("attn", "fused", "q")
CLASS_PARAMS = tuple("%s_%s" % (a, k) for k in KERNELS for a in ("eta", "tpro_us", "tile_us"))
GLOBAL_PARAMS = ("eta_bw", "t0_us", "t_gap_us")
HEADER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "dispatch_model.h")


def class_key(D: int, Hq: int, Hkv: int) -> str:
    return "d%d_%s" % (D, "gqa" if Hq // Hkv >= 2 else "mha")


def load_params(path: str = HEADER) -> dict:
    """The constants of dispatch_model.h: {class: {param: v}} plus globals."""
    text = open(path).read()
    vals = {m.group(1): float(m.group(2)) for m in
            re.finditer(r"constexpr\s+double\s+(\w+)\s*=\s*([-+0-9.eE]+)\s*;", text)}
    out = {c: {p: vals["%s_%s" % (c.upper(), p.upper())] for p in CLASS_PARAMS} for c in CLASSES}
    for p in GLOBAL_PARAMS:
        out[p] = vals[p.upper()]
    return out


def flops(B, Hq, N, D) -> float:
    return 2.0 * B * Hq * float(N) * N * D


def pass_bytes(B, heads, N, D) -> float:
    return 2.0 * B * heads * float(N) * D * 2.0


def kernel_us(c: dict, kernel: str, B, Hq, N, D) -> float:
    """Modelled time of one attention kernel ("attn", "fused" or "q")."""
    thr = flops(B, Hq, N, D) / (c["eta_" + kernel] * MFMA_PEAK) * 1e6
    lat = c["tpro_us_" + kernel] + c["tile_us_" + kernel] * N / 128.0
    return max(thr, lat)


def pass_us(p: dict, nbytes: float) -> float:
    return p["t0_us"] + nbytes / (p["eta_bw"] * HBM_BW) * 1e6


def model_us(p: dict, B, Hq, Hkv, N, D, gap: bool = True) -> dict:
    """Modelled times (microseconds) of the three paths."""
    c = p[class_key(D, Hq, Hkv)]
    g = p["t_gap_us"] if gap else 0.0
    return {"fused": kernel_us(c, "fused", B, Hq, N, D),
            "prerotate": pass_us(p, pass_bytes(B, Hq + Hkv, N, D)) + kernel_us(c, "attn", B, Hq, N, D)
            + g,
            "split": pass_us(p, pass_bytes(B, Hkv, N, D)) + kernel_us(c, "q", B, Hq, N, D) + g}


def alphas(c: dict) -> dict:
    """The in-kernel rotation's cost over plain attention, full and under-filled chip."""
    def ratio(a, b):
        return a / b - 1.0 if b > 0 else None

    return {"alpha_qk": ratio(c["eta_attn"], c["eta_fused"]),
            "alpha_qk_underfilled": ratio(c["tile_us_fused"], c["tile_us_attn"]),
            "alpha_q": ratio(c["eta_attn"], c["eta_q"]),
            "alpha_q_underfilled": ratio(c["tile_us_q"], c["tile_us_attn"])}


def choose(p: dict, B, Hq, Hkv, N, D) -> str:
    """The path with the least modelled time (ties: fused, then pre-rotation)."""
    t = model_us(p, B, Hq, Hkv, N, D)
    best = "fused"
    for path in ("prerotate", "split"):
        if t[path] < t[best]:
            best = path
    return best


def n_star_model(p: dict, B, Hq, Hkv, D, other=("prerotate",), gap=False, lo=64, hi=1 << 17):
    """N where the modelled fused time first exceeds the best of `other`,
    over a fine grid in log N (None if it never does in [lo, hi])."""
    prev = None
    steps = 2000
    for i in range(steps + 1):
        n = lo * (hi / lo) ** (i / steps)
        t = model_us(p, B, Hq, Hkv, n, D, gap=gap)
        d = t["fused"] - min(t[o] for o in other)
        if prev is not None and (prev[1] <= 0) != (d <= 0):
            n0, d0 = prev
            return math.exp(math.log(n0) + d0 / (d0 - d) * (math.log(n) - math.log(n0)))
        prev = (n, d)
    return None


def n_star_closed(c: dict, p: dict, Hq, Hkv) -> float:
    """The closed form: throughput regime, no fixed pass or launch cost."""
    return ((Hq + Hkv) / Hq) * 2.0 * (c["eta_attn"] * MFMA_PEAK) / (p["eta_bw"] * HBM_BW) \
        / alphas(c)["alpha_qk"]


def family_n_star(p: dict, Hq, Hkv, D):
    """A family's modelled N* (B = 1, kernel level: no second-launch cost)
    and the closed form, from fitted parameters p."""
    cls = class_key(D, Hq, Hkv)
    full = dict(p)
    full.update({c: p[cls] for c in CLASSES})
    return n_star_model(full, 1, Hq, Hkv, D), n_star_closed(p[cls], p, Hq, Hkv)


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def fit_kernel(rows, key):
    """(eta, t_pro_us, t_tile_us) minimising the squared log error of
    max(F / (eta P), t_pro + t_tile N / 128) against the kernel times r[key]:
    a grid over t_pro in 0.25 us steps and over 1 / eta and t_tile in log
    steps of 10^(1/120), then a finer one (0.05 us, 10^(1/2400)) around the
    best point."""
    import numpy as np
    F = np.array([flops(r["B"], r["Hq"], r["N"], r["D"]) for r in rows]) * 1e6
    n = np.array([r["N"] / 128.0 for r in rows])
    t = np.array([float(r[key]) for r in rows])

    def best(tp, a, b):
        m = np.maximum(a[None, :, None, None] * F, tp[:, None, None, None] + b[None, None, :, None] * n)
        e = (np.log(t / m) ** 2).sum(-1)
        i = np.unravel_index(e.argmin(), e.shape)
        return tp[i[0]], a[i[1]], b[i[2]]

    a0 = (t / F).min()  # seconds per flop that the fastest row reaches
    b0 = (t / n).min()
    tp, a, b = best(np.arange(0.0, 20.001, 0.25), a0 * 10 ** (np.arange(-30, 91) / 120.0),
                    np.concatenate([[0.0], b0 * 10 ** (np.arange(-90, 31) / 120.0)]))
    tp, a, b = best(np.maximum(tp + np.arange(-5, 6) * 0.05, 0.0),
                    a * 10 ** (np.arange(-20, 21) / 2400.0),
                    b * 10 ** (np.arange(-20, 21) / 2400.0) if b > 0 else np.array([0.0]))
    return 1.0 / (float(a) * MFMA_PEAK), float(tp), float(b)


def fit_pass(rows):
    """(t0_us, eta_bw) by least squares of relative error over both passes."""
    pts = []
    for r in rows:
        pts.append((pass_bytes(r["B"], r["Hq"] + r["Hkv"], r["N"], r["D"]), r["k_rope"]))
        if r.get("k_rope_k") is not None:
            pts.append((pass_bytes(r["B"], r["Hkv"], r["N"], r["D"]), r["k_rope_k"]))
    # minimise sum ((t - t0 - s b) / t)^2: normal equations in (t0, s)
    s11 = sum(1.0 / t ** 2 for b, t in pts)
    s12 = sum(b / t ** 2 for b, t in pts)
    s22 = sum(b * b / t ** 2 for b, t in pts)
    r1 = sum(1.0 / t for b, t in pts)
    r2 = sum(b / t for b, t in pts)
    det = s11 * s22 - s12 * s12
    t0 = (r1 * s22 - r2 * s12) / det
    s = (s11 * r2 - s12 * r1) / det
    return t0, 1.0 / (s * 1e-6 * HBM_BW)


def fit(rows) -> dict:
    """Model parameters from measured rows. Each row: B, Hq, Hkv, N, D and the
    kernels' own times in microseconds (k_fused, k_attn, k_attn_q, k_rope,
    k_rope_k), plus call times (c_fused, c_prerotate) for t_gap."""
    p = {}
    keys = {"attn": "k_attn", "fused": "k_fused", "q": "k_attn_q"}
    for cls in CLASSES:
        rs = [r for r in rows if class_key(r["D"], r["Hq"], r["Hkv"]) == cls]
        if not rs:
            continue
        c = {}
        for kern in KERNELS:
            c["eta_" + kern], c["tpro_us_" + kern], c["tile_us_" + kern] = fit_kernel(rs, keys[kern])
        c.update(alphas(c))
        c["rows"] = len(rs)
        p[cls] = c
    t0, eta_bw = fit_pass(rows)
    p["t0_us"], p["eta_bw"] = t0, eta_bw
    # the second launch: the two-kernel path's call overhead beyond the fused one's
    p["t_gap_us"] = max(0.0, _median([(r["c_prerotate"] - r["k_rope"] - r["k_attn"])
                                      - (r["c_fused"] - r["k_fused"]) for r in rows]))
    return p


_HEADER_HEAD = """\
// dispatch_model.h -- fitted constants of the path-cost model that
// attn_rope_causal_auto evaluates to pick the fused, pre-rotation or GQA
// split path. Written by `python -m rotary_position_embedding_causal_amd.
// dispatch_fit <bench json line>` from the crossover rows of one bench run;
// the run's summary sits beside the other measurements as
// profiles/crossover_fit.json.
//
// The model reads "AttnFuse Makes RoPE a First-Class Attention Compilation
// Operation" (tdteach paper-news, 2026-09-13), paragraph 3: pre-rotation is a
// memory-bandwidth cost, in-kernel rotation a compute-and-tiling cost; per
// paragraph 5 the choice is measured per architecture and shape. In
// microseconds, with F = 2 B Hq N^2 D, P = 2516.6 TFLOP/s, BW = 8 TB/s:
//   T_k     = max(F / (ETA_k P), TPRO_US_k + TILE_US_k N / 128)  for the plain
//             attention kernel (k = ATTN), the one rotating Q and K tiles
//             (FUSED) and the one rotating Q rows (Q); the second term is an
//             under-filled chip: one workgroup's prologue and N / 128 key tiles
//   fused   = T_FUSED
//   prerot  = T0_US + 4 B (Hq + Hkv) N D / (ETA_BW BW) + T_ATTN + T_GAP_US
//   split   = T0_US + 4 B Hkv N D / (ETA_BW BW) + T_Q + T_GAP_US
// Per class of shape (head dim 64 or 128; MHA, or GQA when Hq / Hkv >= 2) the
// nine kernel constants, and the three pass/launch constants shared by all,
// are least-squares fits to kernel times measured on MI355X back to back
// (steady clocks) over the crossover families:%s
#pragma once

namespace rac_model {

constexpr double MFMA_PEAK = 2516.6e12;  // FLOP/s, dense bf16/fp16
constexpr double HBM_BW = 8.0e12;        // B/s

"""

_HEADER_TAIL = """
struct Kernel {
    double eta, tpro_us, tile_us;
};
struct Class {
    Kernel attn, fused, q;
};

#define RAC_MODEL_CLASS(P)                                                          \\
    Class {                                                                         \\
        {P##_ETA_ATTN, P##_TPRO_US_ATTN, P##_TILE_US_ATTN},                         \\
            {P##_ETA_FUSED, P##_TPRO_US_FUSED, P##_TILE_US_FUSED},                  \\
            {P##_ETA_Q, P##_TPRO_US_Q, P##_TILE_US_Q}                               \\
    }

inline Class shape_class(int D, int Hq, int Hkv) {
    const bool gqa = Hq / Hkv >= 2;
    if (D == 64) return gqa ? RAC_MODEL_CLASS(D64_GQA) : RAC_MODEL_CLASS(D64_MHA);
    return gqa ? RAC_MODEL_CLASS(D128_GQA) : RAC_MODEL_CLASS(D128_MHA);
}

#undef RAC_MODEL_CLASS

inline double kernel_us(const Kernel& k, double flops, double n) {
    const double thr = flops / (k.eta * MFMA_PEAK) * 1e6;
    const double lat = k.tpro_us + k.tile_us * n / 128.0;
    return thr > lat ? thr : lat;
}

// Modelled times in microseconds of the fused, pre-rotation and split paths.
inline void path_times(int B, int Hq, int Hkv, int N, int D, double* fused, double* prerot,
                       double* split) {
    const Class c = shape_class(D, Hq, Hkv);
    const double n = (double)N;
    const double f = 2.0 * B * (double)Hq * n * n * D;
    const double qk_bytes = 2.0 * B * ((double)Hq + Hkv) * n * D * 2.0;
    const double k_bytes = 2.0 * B * (double)Hkv * n * D * 2.0;
    const double bw = ETA_BW * HBM_BW;
    *fused = kernel_us(c.fused, f, n);
    *prerot = T0_US + qk_bytes / bw * 1e6 + kernel_us(c.attn, f, n) + T_GAP_US;
    *split = T0_US + k_bytes / bw * 1e6 + kernel_us(c.q, f, n) + T_GAP_US;
}

}  // namespace rac_model
"""


def header_text(p: dict, families: str) -> str:
    """dispatch_model.h for fitted parameters `p` (as fit() returns them)."""
    lines = [_HEADER_HEAD % families]
    for cls in CLASSES:
        for name in CLASS_PARAMS:
            lines.append("constexpr double %s_%s = %.6g;\n" % (cls.upper(), name.upper(),
                                                               p[cls][name]))
        lines.append("\n")
    for name in GLOBAL_PARAMS:
        lines.append("constexpr double %s = %.6g;\n" % (name.upper(), p[name]))
    return "".join(lines) + _HEADER_TAIL


SUMMARY = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                       "crossover_fit.json")


def summary(line: dict) -> dict:
    """The crossover part of a bench JSON line, compact: per row the median
    call and kernel times (microseconds) and the kernel-level gap's spread."""
    cx = line["crossover"]
    keep = ("workload", "auto_path", "fastest_path")
    times = ("c_fused", "c_prerotate", "c_split", "c_auto", "k_fused", "k_attn", "k_attn_q",
             "k_rope", "k_rope_k", "k_rope_cold", "k_copy", "k_copy_cold")
    rows = []
    for r in cx["rows"]:
        row = {k: r[k] for k in keep}
        row.update({k: round(r[k], 1) for k in times})
        row["gap_kernels"] = [round(r["gap_kernels"][k], 4) for k in ("min", "median", "max")]
        rows.append(row)
    out = {k: v for k, v in cx.items() if k not in ("rows", "model")}
    out["model"] = {k: v for k, v in cx["model"].items() if k != "dispatcher_constants"}
    out["rows"] = rows
    out["bench"] = {k: line[k] for k in ("metric", "value", "unit", "steps", "warmup")}
    return out


if __name__ == "__main__":
    import json
    import sys

    line = json.loads(open(sys.argv[1]).read().strip().splitlines()[-1])
    cx = line["crossover"]
    # the constants are this module's fit of the run's rows (the same fit the
    # bench reports, redone here so that header and summary always agree)
    fitted = fit(cx["rows"])
    cx["model"]["fit"] = fitted
    byname = {r["workload"]: r for r in cx["rows"]}
    from rotary_position_embedding_causal_amd import inputs
    for fam, v in cx["families"].items():
        r0 = byname[inputs.CROSSOVER_FAMILIES[fam][1][0]]
        n_model, n_closed = family_n_star(fitted, r0["Hq"], r0["Hkv"], r0["D"])
        measured = v["n_star_kernels"]["n_star"]
        v.update(n_star_model=n_model, n_star_closed_form=n_closed,
                 model_vs_measured=(n_model / measured - 1.0) if (n_model and measured) else None)
    head, c64 = cx["families"]["mha_d64_fp16"], fitted["d64_mha"]
    cx["model"].update(alpha=c64["alpha_qk"], eta_mfma=c64["eta_attn"], eta_bw=fitted["eta_bw"],
                       alpha_underfilled=c64["alpha_qk_underfilled"], t0_us=fitted["t0_us"],
                       t_gap_us=fitted["t_gap_us"], n_star_model=head["n_star_model"],
                       n_star_closed_form=head["n_star_closed_form"])
    fams = "".join("\n//   " + v["desc"] + ", N = " + ", ".join(str(n) for n in v["N"])
                   for v in cx["families"].values())
    with open(HEADER, "w") as f:
        f.write(header_text(cx["model"]["fit"], fams))
    sm = summary(line)
    rows = sm.pop("rows")
    text = json.dumps(sm, indent=1)[:-2]  # the rows last, one per line
    text += ',\n "rows": [\n' + ",\n".join("  " + json.dumps(r) for r in rows) + "\n ]\n}\n"
    with open(SUMMARY, "w") as f:
        f.write(text)
    print(HEADER)
    print(SUMMARY)
