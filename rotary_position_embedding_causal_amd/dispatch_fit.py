"""The path-cost model behind attn_rope_causal_auto, and its fit to kernel times.

"AttnFuse Makes RoPE a First-Class Attention Compilation Operation"
(tdteach paper-news, 2026-09-13), paragraph 3, states the trade-off:
pre-rotation is a memory-bandwidth cost (Q and K read and written once more),
in-kernel rotation a compute-and-tiling cost, so which one wins follows from
the GPU's compute-to-bandwidth ratio; paragraph 5 adds that the choice has to
be measured per architecture and shape. The AttnFuse abstract (arxivdaily
2609.13612) says a crossover derived that way matches measurement. The pages
print no formula; the reading written out here is the plain one, with the
attention kernels' time counted in the unit they are built from -- a
workgroup's step over one 64-key tile -- and scheduled the way the launch
runs them:

  kernel      T_k = t_launch_k + t_step_k[shape] * M
              M = the launch's makespan in steps: every workgroup costs the
              key tiles it walks plus r (its fixed work -- Q rows, the first
              tile's wait, the epilogue -- in steps, one r per class), and
              the workgroups go, in launch order, to the first free slot of
              the XCD the hardware deals them to (round robin over 8 XCDs of
              32 CUs). shape is the launch attn_fwd.hip takes: "pair" (one
              8-wave workgroup per CU, equal work per workgroup) or "tile"
              (one query tile per workgroup, heaviest first per head; two
              heads of a GQA group per 8-wave workgroup, one CU each, or one
              head per 4-wave workgroup, two per CU). Each attention kernel
              has its own (t_launch, t_step[pair], t_step[tile]): plain
              (T_attn), rotating Q and K tiles (T_fused), rotating Q rows
              only (T_q)
  pass        T_pass  = t0 + bytes / (eta_bw * BW)    (BW = 8 TB/s HBM peak)
              bytes = 2 x (the rotated heads) x B N D x 2 bytes, read + write
  fused       T_fused
  pre-rotate  T_pre   = T_pass(Hq + Hkv heads) + T_attn + t_gap
  GQA split   T_split = T_pass(Hkv heads) + T_q + t_gap

t_gap is what a second launch adds to a call (0 for the kernel-level
crossover). On a full chip (large N) M grows as N^2 and the kernels run at
a fixed fraction eta_k = F / (P T_k) of the MFMA peak P (F = 2 B Hq N^2 D,
causal); the rotation's cost is alpha = T_fused / T_attn - 1 =
t_step_fused / t_step_attn - 1 there. Setting T_fused = T_pre in that
regime with t0 = t_gap = 0 gives the closed form
  N* = ((Hq + Hkv) / Hq) * 2 bytes * (eta_attn P) / (eta_bw BW) / alpha,
proportional to P / BW as paragraph 3 says. Below it, the launch's rounds
of workgroups and their fixed work decide, which the makespan carries.

The parameters are fitted per class of shape -- head dim 64 or 128, MHA or
GQA (Hq / Hkv >= 2) -- from kernel times measured on MI355X, and the fitted
values are the constants of csrc/dispatch_model.h, whose C++ evaluates the
same makespan; this module parses that header so that tests can check the C
planner against the model. Nothing here runs on the product path.
"""
from __future__ import annotations

import heapq
import math
import os
import re

MFMA_PEAK = 2516.6e12   # MI355X dense bf16/fp16, FLOP/s (published)
HBM_BW = 8.0e12         # MI355X HBM3E, B/s (published)
NUM_CUS, NXCD, BM, BN = 256, 8, 128, 64   # as attn_fwd.hip launches
JOB_CAP = 4096          # jobs per XCD scheduled one by one; beyond, the mean load
CLASSES = ("d64_mha", "d128_mha", "d64_gqa", "d128_gqa")
KERNELS = ("attn", "fused", "q")
SHAPES = ("pair", "tile")
CLASS_PARAMS = ("wg_steps",) + tuple("%s_%s" % (a, k) for k in KERNELS
                                     for a in ("launch_us", "pair_us", "tile_us"))
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


def kv_tiles_of(qt: int, N: int) -> int:
    """64-key tiles that 128-row query tile qt walks (keys 0 .. its last row)."""
    return (min(qt * BM + BM, N) - 1) // BN + 1


def launch(B: int, Hq: int, Hkv: int, N: int, D: int):
    """The automatic launch of the attention kernels (attn_fwd.hip):
    (shape, units, per_head, packs, slots per XCD, base steps by index)."""
    nq = (N + BM - 1) // BM
    n_pairs = (nq + 1) // 2
    pair_units = n_pairs * Hq * B
    heads_ok = (Hq // Hkv) % 2 == 0
    group = Hq // Hkv
    pair = nq >= 2 and pair_units <= NUM_CUS and (
        pair_units >= NUM_CUS // 2 or nq >= (4 if heads_ok else 12))
    if not heads_ok and nq >= 2 and (pair_units == 2 * NUM_CUS or (
            D == 128 and 3 * NUM_CUS // 2 <= pair_units <= 2 * NUM_CUS)):
        pair = True
    if pair:
        base = []
        for p in range(n_pairs):
            th = nq - 1 - p
            len_h = kv_tiles_of(th, N)
            len_l = kv_tiles_of(p, N) if p < th else 0
            base.append((len_l + len_h + 1) // 2)
        return "pair", pair_units, n_pairs, group, NUM_CUS // NXCD, base
    hg = 2 if heads_ok else 1
    base = [kv_tiles_of(nq - 1 - i, N) for i in range(nq)]
    slots = (NUM_CUS // NXCD) * (1 if hg == 2 else 2)
    return "tile", nq * Hq * B // hg, nq, group // hg, slots, base


def makespan(B: int, Hq: int, Hkv: int, N: int, D: int, r: float):
    """(shape, M): the launch's makespan in 64-key steps, each workgroup
    costing its steps plus r. Workgroup u walks base[(u // packs) %
    per_head] steps; XCD x runs units x*U/8 .. (x+1)*U/8 - 1 in order when 8
    divides U (the launch's XCD-aware order), else units x, x + 8, ...; each
    goes to the XCD's least-loaded slot. Past JOB_CAP jobs per XCD the
    schedule is taken as balanced: the XCD's mean load plus half the
    heaviest workgroup."""
    shape, units, per_head, packs, slots, base = launch(B, Hq, Hkv, N, D)
    if units <= 0:
        return shape, 0.0
    wmax = max(base) + r
    pre = [0]
    for b in base:
        pre.append(pre[-1] + b)

    def weight_sum(x):  # sum of base over units 0 .. x-1
        v, rem = divmod(x, packs)
        full, part = divmod(v, per_head)
        return packs * (full * pre[-1] + pre[part]) + rem * base[part]

    best = 0.0
    div = units % NXCD == 0
    for x in range(NXCD):
        if div:
            lo, hi = x * (units // NXCD), (x + 1) * (units // NXCD)
            jobs = range(lo, hi)
        else:
            jobs = range(x, units, NXCD)
        n = len(jobs)
        if n == 0:
            continue
        if n > JOB_CAP:
            steps = weight_sum(hi) - weight_sum(lo) if div else weight_sum(units) / NXCD
            m = (steps + r * n) / slots + 0.5 * wmax
        else:
            heap = [0.0] * min(slots, n)
            for u in jobs:
                w = base[(u // packs) % per_head] + r
                heapq.heapreplace(heap, heap[0] + w)
            m = max(heap)
        best = max(best, m)
    return shape, best


def kernel_us(c: dict, kernel: str, shape: str, m: float) -> float:
    """Modelled time of one attention kernel ("attn", "fused" or "q")."""
    return c["launch_us_" + kernel] + c["%s_us_%s" % (shape, kernel)] * m


def pass_us(p: dict, nbytes: float) -> float:
    return p["t0_us"] + nbytes / (p["eta_bw"] * HBM_BW) * 1e6


def model_us(p: dict, B, Hq, Hkv, N, D, gap: bool = True) -> dict:
    """Modelled times (microseconds) of the three paths."""
    c = p[class_key(D, Hq, Hkv)]
    shape, m = makespan(B, Hq, Hkv, int(N), D, c["wg_steps"])
    g = p["t_gap_us"] if gap else 0.0
    return {"fused": kernel_us(c, "fused", shape, m),
            "prerotate": pass_us(p, pass_bytes(B, Hq + Hkv, N, D))
            + kernel_us(c, "attn", shape, m) + g,
            "split": pass_us(p, pass_bytes(B, Hkv, N, D)) + kernel_us(c, "q", shape, m) + g}


def asymptote(p: dict, Hq: int, Hkv: int, D: int, N: int = 65536) -> dict:
    """The full-chip regime at B = 1: each kernel's fraction of the MFMA peak
    (eta) and the rotation's cost over plain attention (alpha), evaluated at
    a long sequence, plus the per-step ratio of the pair launch (the
    under-filled one)."""
    c = p[class_key(D, Hq, Hkv)]
    shape, m = makespan(1, Hq, Hkv, N, D, c["wg_steps"])
    t = {k: kernel_us(c, k, shape, m) for k in KERNELS}
    f = flops(1, Hq, N, D)

    def ratio(a, b):
        return a / b - 1.0 if b > 0 else None

    out = {"eta_" + k: f / (MFMA_PEAK * t[k] * 1e-6) for k in KERNELS}
    out.update(alpha_qk=ratio(t["fused"], t["attn"]), alpha_q=ratio(t["q"], t["attn"]),
               alpha_qk_pair=ratio(c["pair_us_fused"], c["pair_us_attn"]),
               alpha_q_pair=ratio(c["pair_us_q"], c["pair_us_attn"]))
    return out


def choose(p: dict, B, Hq, Hkv, N, D) -> str:
    """The path with the least modelled time (ties: fused, then pre-rotation)."""
    t = model_us(p, B, Hq, Hkv, N, D)
    best = "fused"
    for path in ("prerotate", "split"):
        if t[path] < t[best]:
            best = path
    return best


def locate(ns, fused, other):
    """The first sign change of fused / other - 1 over ascending ns,
    interpolated log-linearly in the relative gap (None if there is none)."""
    prev = None
    for n, f, o in zip(ns, fused, other):
        d = f / o - 1.0
        if prev is not None and (prev[1] < 0) != (d < 0):
            n0, d0 = prev
            return math.exp(math.log(n0) + d0 / (d0 - d) * (math.log(n) - math.log(n0)))
        prev = (n, d)
    return None


def n_star_model(p: dict, B, Hq, Hkv, D, ns=None, other=("prerotate",), gap=False, lo=1024,
                 hi=1 << 17):
    """N* of the modelled times, fused against the best of `other`: over the
    given sequence lengths `ns` (the points a sweep measured, so that model
    and measurement are located alike), or, without them, over multiples of
    128 from `lo` stepping by ~1 % up to `hi`. None if the sign never
    changes."""
    if ns is None:
        ns, n = [], lo
        while n <= hi:
            ns.append(n)
            n = max(n + 128, int(n * 1.01) // 128 * 128)
    ts = [model_us(p, B, Hq, Hkv, n, D, gap=gap) for n in ns]
    return locate(ns, [t["fused"] for t in ts], [min(t[o] for o in other) for t in ts])


def n_star_closed(p: dict, Hq, Hkv, D) -> float:
    """The closed form: full chip, no fixed pass or launch cost."""
    a = asymptote(p, Hq, Hkv, D)
    return ((Hq + Hkv) / Hq) * 2.0 * (a["eta_attn"] * MFMA_PEAK) / (p["eta_bw"] * HBM_BW) \
        / a["alpha_qk"]


def family_n_star(p: dict, Hq, Hkv, D, ns=None):
    """A family's modelled N* (B = 1, kernel level: no second-launch cost)
    over its sweep's lengths ns, over a fine grid from its first length, and
    the closed form, from fitted parameters p."""
    return (n_star_model(p, 1, Hq, Hkv, D, ns=ns),
            n_star_model(p, 1, Hq, Hkv, D, lo=ns[0] if ns else 1024),
            n_star_closed(p, Hq, Hkv, D))


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def fit_class(rows, keys=(("attn", "k_attn"), ("fused", "k_fused"), ("q", "k_attn_q"))):
    """One class's constants: r on a grid of quarter steps (0 .. 16), and for
    each r and kernel the non-negative least-squares (t_launch, t_step[pair],
    t_step[tile]) in relative error; the r with the least total squared
    relative error over the three kernels wins. A launch shape none of the
    rows takes gets the other shape's step time."""
    import numpy as np
    from scipy.optimize import nnls
    best = None
    for r in np.arange(0.0, 16.001, 0.25):
        ms = [makespan(x["B"], x["Hq"], x["Hkv"], x["N"], x["D"], float(r)) for x in rows]
        X = np.array([[1.0] + [m if s == sh else 0.0 for sh in SHAPES] for s, m in ms])
        total, c = 0.0, {"wg_steps": float(r)}
        for kern, key in keys:
            y = np.array([float(x[key]) for x in rows])
            coef, _ = nnls(X / y[:, None], np.ones(len(rows)))
            total += float((((X @ coef) / y - 1.0) ** 2).sum())
            c["launch_us_" + kern] = float(coef[0])
            for i, sh in enumerate(SHAPES):
                c["%s_us_%s" % (sh, kern)] = float(coef[1 + i])
            seen = {s for s, _ in ms}
            for i, sh in enumerate(SHAPES):
                if sh not in seen:
                    c["%s_us_%s" % (sh, kern)] = float(coef[1 + (1 - i)])
        if best is None or total < best[0]:
            best = (total, c)
    return best[1]


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
    for cls in CLASSES:
        rs = [r for r in rows if class_key(r["D"], r["Hq"], r["Hkv"]) == cls]
        if not rs:
            continue
        c = fit_class(rs)
        c["rows"] = len(rs)
        p[cls] = c
    t0, eta_bw = fit_pass(rows)
    p["t0_us"], p["eta_bw"] = t0, eta_bw
    # the second launch: the two-kernel path's call overhead beyond the fused one's
    p["t_gap_us"] = max(0.0, _median([(r["c_prerotate"] - r["k_rope"] - r["k_attn"])
                                      - (r["c_fused"] - r["k_fused"]) for r in rows]))
    return p


def fit_errors(p: dict, rows) -> dict:
    """Per class and kernel, the fitted model's relative error on the rows:
    root mean square and largest."""
    out = {}
    for cls in CLASSES:
        rs = [r for r in rows if class_key(r["D"], r["Hq"], r["Hkv"]) == cls]
        if not rs or cls not in p:
            continue
        c = p[cls]
        for kern, key in (("attn", "k_attn"), ("fused", "k_fused"), ("q", "k_attn_q")):
            e = []
            for r in rs:
                shape, m = makespan(r["B"], r["Hq"], r["Hkv"], r["N"], r["D"], c["wg_steps"])
                e.append(kernel_us(c, kern, shape, m) / r[key] - 1.0)
            out["%s_%s" % (cls, kern)] = {"rms": math.sqrt(sum(x * x for x in e) / len(e)),
                                          "max_abs": max(abs(x) for x in e)}
    return out


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
// microseconds, with BW = 8 TB/s:
//   T_k     = LAUNCH_US_k + (PAIR_US_k or TILE_US_k) * M   for the plain
//             attention kernel (k = ATTN), the one rotating Q and K tiles
//             (FUSED) and the one rotating Q rows (Q), where M is the
//             attention launch's makespan in 64-key steps (makespan() below:
//             each workgroup's key tiles plus WG_STEPS, list-scheduled per
//             XCD) and PAIR or TILE the launch shape attn_fwd.hip takes
//   fused   = T_FUSED
//   prerot  = T0_US + 4 B (Hq + Hkv) N D / (ETA_BW BW) + T_ATTN + T_GAP_US
//   split   = T0_US + 4 B Hkv N D / (ETA_BW BW) + T_Q + T_GAP_US
// Per class of shape (head dim 64 or 128; MHA, or GQA when Hq / Hkv >= 2) the
// ten kernel constants, and the three pass/launch constants shared by all,
// are least-squares fits to kernel times measured on MI355X back to back
// (steady clocks) over the crossover families:%s
#pragma once

#include <stdint.h>

namespace rac_model {

constexpr double HBM_BW = 8.0e12;  // B/s

"""

_HEADER_TAIL = """
// The attention launch (as attn_fwd.hip takes it automatically): 128-row
// query tiles over 64-key tiles, 256 CUs in 8 XCDs.
constexpr int NUM_CUS = 256, NXCD = 8, BM = 128, BN = 64;
constexpr int64_t JOB_CAP = 4096;  // jobs per XCD scheduled one by one

struct Kernel {
    double launch_us, pair_us, tile_us;
};
struct Class {
    double wg_steps;
    Kernel attn, fused, q;
};

#define RAC_MODEL_KERNEL(P, K) Kernel{P##_LAUNCH_US_##K, P##_PAIR_US_##K, P##_TILE_US_##K}
#define RAC_MODEL_CLASS(P)                                                             \\
    Class {                                                                            \\
        P##_WG_STEPS, RAC_MODEL_KERNEL(P, ATTN), RAC_MODEL_KERNEL(P, FUSED),            \\
            RAC_MODEL_KERNEL(P, Q)                                                     \\
    }

inline Class shape_class(int D, int Hq, int Hkv) {
    const bool gqa = Hq / Hkv >= 2;
    if (D == 64) return gqa ? RAC_MODEL_CLASS(D64_GQA) : RAC_MODEL_CLASS(D64_MHA);
    return gqa ? RAC_MODEL_CLASS(D128_GQA) : RAC_MODEL_CLASS(D128_MHA);
}

#undef RAC_MODEL_CLASS
#undef RAC_MODEL_KERNEL

inline int64_t kv_tiles_of(int64_t qt, int64_t N) {
    const int64_t last = qt * BM + BM < N ? qt * BM + BM : N;
    return (last - 1) / BN + 1;
}

// The attention launch's makespan in 64-key steps (pair: whether it is the
// paired launch). Workgroup u walks base[(u / packs) % per_head] key tiles
// plus r steps of fixed work; XCD x runs units x U/8 .. (x+1) U/8 - 1 in
// order when 8 divides U (the launch's XCD-aware order), else units x,
// x + 8, ..., each on its least-loaded slot (one per CU, or two for the
// one-head tile launch's 4-wave workgroups). Past JOB_CAP jobs per XCD the
// XCD is taken as balanced: its mean load plus half the heaviest workgroup.
inline double makespan(int B, int Hq, int Hkv, int N, int D, double r, bool* pair) {
    const int64_t nq = ((int64_t)N + BM - 1) / BM;
    const int64_t n_pairs = (nq + 1) / 2;
    const int64_t pair_units = n_pairs * Hq * B;
    const int group = Hq / Hkv;
    const bool heads_ok = group % 2 == 0;
    *pair = nq >= 2 && pair_units <= NUM_CUS &&
            (pair_units >= NUM_CUS / 2 || nq >= (heads_ok ? 4 : 12));
    if (!heads_ok && nq >= 2 &&
        (pair_units == 2 * NUM_CUS ||
         (D == 128 && pair_units >= 3 * NUM_CUS / 2 && pair_units <= 2 * NUM_CUS)))
        *pair = true;
    int64_t units, per_head, packs, slots;
    if (*pair) {
        units = pair_units, per_head = n_pairs, packs = group, slots = NUM_CUS / NXCD;
    } else {
        const int hg = heads_ok ? 2 : 1;
        units = nq * Hq * B / hg, per_head = nq, packs = group / hg;
        slots = (NUM_CUS / NXCD) * (hg == 2 ? 1 : 2);
    }
    if (units <= 0) return 0.0;
    auto base = [&](int64_t i) -> int64_t {
        if (!*pair) return kv_tiles_of(nq - 1 - i, N);
        const int64_t th = nq - 1 - i;
        const int64_t len_l = i < th ? kv_tiles_of(i, N) : 0;
        return (len_l + kv_tiles_of(th, N) + 1) / 2;
    };
    // sum of base over units 0 .. x-1 (prefix over one head, then periods)
    int64_t total = 0, wmax_steps = 0;
    for (int64_t i = 0; i < per_head; ++i) {
        total += base(i);
        if (base(i) > wmax_steps) wmax_steps = base(i);
    }
    auto prefix = [&](int64_t m) {
        int64_t s = 0;
        for (int64_t i = 0; i < m; ++i) s += base(i);
        return s;
    };
    auto weight_sum = [&](int64_t x) -> double {
        const int64_t v = x / packs, rem = x % packs;
        const int64_t full = v / per_head, part = v % per_head;
        return (double)packs * ((double)full * total + prefix(part)) +
               (double)rem * (part < per_head ? base(part) : 0);
    };
    const double wmax = (double)wmax_steps + r;
    const bool div = units % NXCD == 0;
    double best = 0.0;
    double heap[64];
    for (int x = 0; x < NXCD; ++x) {
        const int64_t lo = div ? x * (units / NXCD) : x;
        const int64_t hi = div ? (x + 1) * (units / NXCD) : units;
        const int64_t step = div ? 1 : NXCD;
        const int64_t n = hi > lo ? (hi - lo + step - 1) / step : 0;
        if (n == 0) continue;
        double m;
        if (n > JOB_CAP) {
            const double steps = div ? weight_sum(hi) - weight_sum(lo) : weight_sum(units) / NXCD;
            m = (steps + r * (double)n) / (double)slots + 0.5 * wmax;
        } else {
            // list scheduling: a binary min-heap of the slots' loads
            const int k = (int)(n < slots ? n : slots);
            for (int i = 0; i < k; ++i) heap[i] = 0.0;
            for (int64_t u = lo; u < hi; u += step) {
                const double w = (double)base((u / packs) % per_head) + r;
                double v = heap[0] + w;  // the least-loaded slot takes it
                int i = 0;
                for (;;) {
                    int c = 2 * i + 1;
                    if (c >= k) break;
                    if (c + 1 < k && heap[c + 1] < heap[c]) ++c;
                    if (heap[c] >= v) break;
                    heap[i] = heap[c];
                    i = c;
                }
                heap[i] = v;
            }
            m = 0.0;
            for (int i = 0; i < k; ++i) m = heap[i] > m ? heap[i] : m;
        }
        if (m > best) best = m;
    }
    return best;
}

inline double kernel_us(const Kernel& k, bool pair, double m) {
    return k.launch_us + (pair ? k.pair_us : k.tile_us) * m;
}

// Modelled times in microseconds of the fused, pre-rotation and split paths.
inline void path_times(int B, int Hq, int Hkv, int N, int D, double* fused, double* prerot,
                       double* split) {
    const Class c = shape_class(D, Hq, Hkv);
    bool pair = false;
    const double m = makespan(B, Hq, Hkv, N, D, c.wg_steps, &pair);
    const double n = (double)N;
    const double qk_bytes = 2.0 * B * ((double)Hq + Hkv) * n * D * 2.0;
    const double k_bytes = 2.0 * B * (double)Hkv * n * D * 2.0;
    const double bw = ETA_BW * HBM_BW;
    *fused = kernel_us(c.fused, pair, m);
    *prerot = T0_US + qk_bytes / bw * 1e6 + kernel_us(c.attn, pair, m) + T_GAP_US;
    *split = T0_US + k_bytes / bw * 1e6 + kernel_us(c.q, pair, m) + T_GAP_US;
}

}  // namespace rac_model
"""


def header_text(p: dict, families: str) -> str:
    """dispatch_model.h for fitted parameters `p` (as fit() returns them)."""
    lines = [_HEADER_HEAD % families]
    for cls in CLASSES:
        for name in CLASS_PARAMS:
            lines.append("constexpr double %s_%s = %.9g;\n" % (cls.upper(), name.upper(),
                                                               p[cls][name]))
        lines.append("\n")
    for name in GLOBAL_PARAMS:
        lines.append("constexpr double %s = %.9g;\n" % (name.upper(), p[name]))
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


def family_models(p: dict, families: dict, byname: dict) -> None:
    """Adds to each family of a crossover summary its modelled N* (over the
    sweep's own lengths, and over a fine grid), the closed form and the
    modelled-over-measured ratio of the sweep-located values."""
    from rotary_position_embedding_causal_amd import inputs
    for fam, v in families.items():
        r0 = byname[inputs.CROSSOVER_FAMILIES[fam][1][0]]
        n_model, n_fine, n_closed = family_n_star(p, r0["Hq"], r0["Hkv"], r0["D"], ns=v["N"])
        measured = v["n_star_kernels"]["n_star"]
        v.update(n_star_model=n_model, n_star_model_fine=n_fine, n_star_closed_form=n_closed,
                 model_vs_measured=(n_model / measured - 1.0) if (n_model and measured) else None,
                 closed_vs_measured=(n_closed / measured - 1.0) if measured else None)


def headline_model(p: dict, families: dict) -> dict:
    """The model's headline figures: the D = 64 MHA family's asymptotic
    eta and alpha (full chip) and the pair launch's per-step alpha, the
    pass constants, the family's modelled and closed-form N*."""
    head = families["mha_d64_fp16"]
    a = asymptote(p, 16, 16, 64)
    return {"alpha": a["alpha_qk"], "eta_mfma": a["eta_attn"], "eta_bw": p["eta_bw"],
            "alpha_underfilled": a["alpha_qk_pair"], "t0_us": p["t0_us"],
            "t_gap_us": p["t_gap_us"], "n_star_model": head["n_star_model"],
            "n_star_model_fine": head["n_star_model_fine"],
            "n_star_closed_form": head["n_star_closed_form"]}


FORM = ("T_k = t_launch_k + t_step_k[pair|tile] * M, M = the attention launch's makespan in "
        "64-key steps (each workgroup's key tiles + wg_steps, list-scheduled per XCD); "
        "alpha = T_fused/T_attn - 1 and eta_k = F/(P T_k) at N = 65536; pre = t0 + "
        "4B(Hq+Hkv)ND/(eta_bw BW) + T_attn; N* where T_fused = pre")


if __name__ == "__main__":
    import json
    import sys

    line = json.loads(open(sys.argv[1]).read().strip().splitlines()[-1])
    cx = line["crossover"]
    # the constants are this module's fit of the run's rows (the same fit the
    # bench reports, redone here so that header and summary always agree)
    fitted = fit(cx["rows"])
    byname = {r["workload"]: r for r in cx["rows"]}
    family_models(fitted, cx["families"], byname)
    cx["model"] = dict(headline_model(fitted, cx["families"]), fit=fitted,
                       fit_errors=fit_errors(fitted, cx["rows"]), form=FORM)
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
