"""Benchmark: causal RoPE attention forward on one MI355X, fused vs pre-rotated.

One step = the whole hot path over one batch of the Llama-3-8B-shaped GQA
attention layer (B=1, Hq=32, Hkv=8, N=2048, D=128, bf16, RoPE base 500000):
  * the fused path: attn_rope_causal_fwd (one kernel), and
  * the pre-rotation path: rope_prerotate then attn_causal_fwd.
`value` = causal attention FLOPs of both paths (2 * 2*B*Hq*N^2*D per step)
divided by the measured step time, in TFLOP/s. Inputs are resident in HBM
before timing starts; steps run back to back on torch's current stream.

Also printed in the same JSON line:
  * roofline: the fused attention kernel (the dominant kernel), achieved
    TFLOP/s from a pair of HIP events that each of its launches in the timed
    region records at the kernel's own start and end (rac.time_next_kernel,
    hipExtLaunchKernel on the launch stream), against the dense bf16 MFMA
    peak;
  * paths: per-kernel times taken the same way (warm, and cold after a
    512 MiB cache flush) and their sums per path, TFLOP/s, % of MFMA peak,
    rope_prerotate GB/s vs 8 TB/s;
    also the GQA split path (rope_prerotate_k then attn_rope_q_causal_fwd),
    timed after the step loop and not part of `value`;
  * crossover: fused vs pre-rotation (and split) times over the D=64 fp16
    MHA sweep (N = 2048 .. 32768) and the GQA shapes, with the measured
    crossover N* of fused vs pre-rotation;
  * variants: the half-split RoPE pairing (fused and pre-rotated) and the
    ALiBi score modification (alone and with fused RoPE), timed after the
    step loop and not part of `value`;
  * cpu_baseline: the fp64 CPU oracle timed on this host over the full
    workload (rotation + causal attention), in the same unit.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
       [--no-cpu] [--only fused|prerotate|rope|attn|split|rope_k|attn_q
       [--workload NAME]]
       [--copy-calib]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6}  # MI355X dense, published
CSRC = os.path.join(ROOT, "rotary_position_embedding_causal_amd", "csrc")
ATTN_SOURCES = ("attn_fwd.hip", "rac_device.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fused_traffic_llama3_8b_gqa_n2048.json")


def rotation_mode(kernel_name):
    """Rotation-mode template argument of an attention kernel name
    (attn_*_kernel<dtype, head dim, mode, ...>): 0 none, 1 Q and K, 2 Q only."""
    args = kernel_name.split("(")[0].split("<", 1)[1].rsplit(">", 1)[0].split(",")
    return int(args[2])

HBM_PEAK_GBS = 8000.0
WARM_SECONDS = 0.2  # minimum warm-up before any timed region
MAIN = "llama3_8b_gqa_n2048"
METRIC = "causal RoPE-attn fwd TFLOP/s (fused & pre-rotate) + % of MFMA peak; N*"


def attn_source_hash():
    """sha256 over the attention kernel sources (counters are tied to it)."""
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per fused-kernel launch from the committed counter summary,
    or None when the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != attn_source_hash():
        return None
    return t["read_bytes"] + t["write_bytes"]


def ingest_counters(fetch_dir, write_dir, calib_fetch_dir, calib_write_dir):
    """Turns rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE CSVs of a `--only fused`
    run and of a `--copy-calib` run into the traffic summary under profiles/."""
    import csv
    import glob

    def per_dispatch(d, pick):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(f[0])) if pick(r["Kernel_Name"])]
        return sum(vals) / len(vals), len(vals)

    fused = lambda k: "attn_" in k and "<" in k and rotation_mode(k) == 1  # noqa: E731
    copy = lambda k: "copyBuffer" in k or "elementwise" in k  # noqa: E731
    fetch, nf = per_dispatch(fetch_dir, fused)
    write, nw = per_dispatch(write_dir, fused)
    cfetch, _ = per_dispatch(calib_fetch_dir, lambda k: "copyBuffer" in k)
    cwrite, _ = per_dispatch(calib_write_dir, lambda k: "copyBuffer" in k)
    copy_bytes = 256 << 20
    rscale = copy_bytes / (cfetch * 1024.0)
    wscale = copy_bytes / (cwrite * 1024.0)
    out = {"kernel": "attn fused (RoPE) forward", "workload": MAIN,
           "source_sha256": attn_source_hash(),
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "dispatches": [nf, nw],
           "calibration": {"copy_bytes": copy_bytes, "fetch_kib": cfetch, "write_kib": cwrite,
                           "read_scale": rscale, "write_scale": wscale},
           "read_bytes": fetch * 1024.0 * rscale, "write_bytes": write * 1024.0 * wscale}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def warm(fn, calls, min_seconds, sync):
    """Runs fn at least `calls` times and for at least `min_seconds` (GPU clocks
    settle only after tens of milliseconds of work), then synchronizes."""
    t0 = time.perf_counter()
    done = 0
    while done < calls or time.perf_counter() - t0 < min_seconds:
        for _ in range(max(1, min(calls, 10))):
            fn()
        done += max(1, min(calls, 10))
        sync()


def attn_flops(w):
    return 2.0 * w["B"] * w["Hq"] * w["N"] ** 2 * w["D"]


def prerot_bytes(w):
    return 2.0 * w["B"] * (w["Hq"] + w["Hkv"]) * w["N"] * w["D"] * 2


def prerot_k_bytes(w):
    return 2.0 * w["B"] * w["Hkv"] * w["N"] * w["D"] * 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["fused", "prerotate", "rope", "attn", "split", "rope_k",
                                       "attn_q"], default=None,
                    help="time one kernel/path alone (for profiler runs)")
    ap.add_argument("--workload", default=MAIN,
                    help="workload of the --only runs (a name from inputs.WORKLOADS)")
    ap.add_argument("--ingest-counters", nargs=4, metavar="DIR",
                    help="FETCH_SIZE and WRITE_SIZE counter dirs of a --only fused run, then of "
                         "a --copy-calib run: write the traffic summary under profiles/ and exit")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run a plain 256 MiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import rotary_position_embedding_causal_amd as rac
    from rotary_position_embedding_causal_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rac.lib()

    if args.copy_calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": 256 << 20, "launches": 5}))
        return

    name = args.workload if args.only else MAIN
    w = inputs.WORKLOADS[name]
    B, Hq, Hkv, N, D, base = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["base"]
    q, k, v = inputs.workload_qkv(name)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out_f = torch.empty_like(qd)
    out_p = torch.empty_like(qd)
    lse_f = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    lse_p = torch.empty_like(lse_f)
    qr = torch.empty_like(qd)
    kr = torch.empty_like(kd)
    kr_s = torch.empty_like(kd)
    out_s = torch.empty_like(qd)
    lse_s = torch.empty_like(lse_f)

    def fused():
        rac.attn_rope_causal_fwd(qd, kd, vd, base, out=out_f, lse=lse_f)

    def rope():
        rac.rope_prerotate(qd, kd, base, q_rot=qr, k_rot=kr)

    def attn():
        rac.attn_causal_fwd(qr, kr, vd, out=out_p, lse=lse_p)

    # the GQA split path: K alone through the streaming pass, Q rotated in the kernel
    def rope_k():
        rac.rope_prerotate_k(kd, base, k_rot=kr_s)

    def attn_q():
        rac.attn_rope_q_causal_fwd(qd, kr_s, vd, base, out=out_s, lse=lse_s)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    if args.only:
        fn = {"fused": fused, "rope": rope, "attn": attn,
              "prerotate": lambda: (rope(), attn()), "rope_k": rope_k, "attn_q": attn_q,
              "split": lambda: (rope_k(), attn_q())}[args.only]
        warm(fn, args.warmup, 0.0, torch.cuda.synchronize)  # counter runs: few dispatches
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"only": args.only, "workload": name, "ms_per_call": dt * 1e3}))
        return

    def made(pairs):
        """Creates the events up front (torch creates one at its first record)."""
        for a, b in pairs:
            a.record(); b.record()
        torch.cuda.synchronize()
        return pairs

    # ---- the timed region: K steps of the whole hot path ----
    # warm-up: W steps, and at least WARM_SECONDS of them
    warm(lambda: (fused(), rope(), attn()), args.warmup, WARM_SECONDS, torch.cuda.synchronize)
    # each fused launch (the roofline kernel) records a pair of HIP events at
    # its own start and end (rac.time_next_kernel: hipExtLaunchKernel on the
    # launch stream), so no event packet of its own enters the queue and the
    # time excludes the dispatch latency
    fused_ev = made([(ev(), ev()) for _ in range(args.steps)])
    t0 = time.perf_counter()
    for i in range(args.steps):
        rac.time_next_kernel(*fused_ev[i]); fused()
        rope()
        attn()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps

    def avg_ms(pairs):
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)

    # the pre-rotation path's two kernels, timed the same way after the step loop
    rope_ev = made([(ev(), ev()) for _ in range(args.steps)])
    attn_ev = made([(ev(), ev()) for _ in range(args.steps)])
    for i in range(args.steps):
        rac.time_next_kernel(*rope_ev[i]); rope()
        rac.time_next_kernel(*attn_ev[i]); attn()
    torch.cuda.synchronize()

    fl = attn_flops(w)
    t_fused = avg_ms(fused_ev)
    t_rope = avg_ms(rope_ev)
    t_attn = avg_ms(attn_ev)
    value = 2 * fl / step_s / 1e12
    peak = MFMA_PEAK_TFLOPS[w["dtype"]]
    achieved = fl / (t_fused * 1e-3) / 1e12

    # ---- cold-cache kernel times (512 MiB flush before each rep) ----
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def cold(fn, reps=20):
        """Median kernel time of fn's (single) kernel after a cache flush."""
        ts = []
        for a, b in made([(ev(), ev()) for _ in range(reps)]):
            flush.zero_()
            rac.time_next_kernel(a, b); fn()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        return ts[len(ts) // 2]

    c_fused, c_rope, c_attn = cold(fused), cold(rope), cold(attn)
    pb = prerot_bytes(w)

    # ---- the GQA split path, timed the same way after the timed region ----
    warm(lambda: (rope_k(), attn_q()), args.warmup, WARM_SECONDS, torch.cuda.synchronize)
    rk_ev = made([(ev(), ev()) for _ in range(args.steps)])
    aq_ev = made([(ev(), ev()) for _ in range(args.steps)])
    for i in range(args.steps):
        rac.time_next_kernel(*rk_ev[i]); rope_k()
        rac.time_next_kernel(*aq_ev[i]); attn_q()
    torch.cuda.synchronize()
    t_rk, t_aq = avg_ms(rk_ev), avg_ms(aq_ev)
    c_rk, c_aq = cold(rope_k), cold(attn_q)
    kb = prerot_k_bytes(w)
    paths = {
        "fused": {"ms": t_fused, "tflops": fl / t_fused / 1e9, "mfma_frac": fl / t_fused / 1e9 / peak,
                  "cold_ms": c_fused, "cold_tflops": fl / c_fused / 1e9},
        "prerotate": {"ms": t_rope + t_attn, "tflops": fl / (t_rope + t_attn) / 1e9,
                      "mfma_frac": fl / (t_rope + t_attn) / 1e9 / peak,
                      "cold_ms": c_rope + c_attn},
        "attn_causal_fwd": {"ms": t_attn, "tflops": fl / t_attn / 1e9,
                            "mfma_frac": fl / t_attn / 1e9 / peak, "cold_ms": c_attn},
        "rope_prerotate": {"ms": t_rope, "gbs": pb / t_rope / 1e6,
                           "hbm_frac": pb / t_rope / 1e6 / HBM_PEAK_GBS, "cold_ms": c_rope,
                           "cold_gbs": pb / c_rope / 1e6,
                           "cold_hbm_frac": pb / c_rope / 1e6 / HBM_PEAK_GBS, "bytes": pb},
        "split": {"ms": t_rk + t_aq, "tflops": fl / (t_rk + t_aq) / 1e9,
                  "mfma_frac": fl / (t_rk + t_aq) / 1e9 / peak, "cold_ms": c_rk + c_aq},
        "attn_rope_q_causal_fwd": {"ms": t_aq, "tflops": fl / t_aq / 1e9,
                                   "mfma_frac": fl / t_aq / 1e9 / peak, "cold_ms": c_aq},
        "rope_prerotate_k": {"ms": t_rk, "gbs": kb / t_rk / 1e6,
                             "hbm_frac": kb / t_rk / 1e6 / HBM_PEAK_GBS, "cold_ms": c_rk,
                             "cold_gbs": kb / c_rk / 1e6, "bytes": kb},
    }

    result = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": MAIN, "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "D": D,
                   "rope_base": base, "causal": True,
                   "step": "attn_rope_causal_fwd + (rope_prerotate -> attn_causal_fwd)",
                   "flops_per_path": fl},
        "roofline": {"kernel": "attn_rope_causal_fwd kernel (bf16, D=128)", "bound": "mfma",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": measured_traffic()},
        "paths": paths,
    }

    result["variants"] = variants(torch, rac, w, qd, kd, vd, ev, args.steps)
    result["backward"] = backward(torch, rac, w, qd, kd, vd, out_f, lse_f, ev, args.steps)
    if not args.no_sweep:
        result["crossover"] = crossover(torch, rac, inputs, dev, ev)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(inputs, w)
    print(json.dumps(result), flush=True)


def variants(torch, rac, w, qd, kd, vd, ev, reps):
    """The other RoPE pairing and the ALiBi score modification on the bench
    workload, after the timed region (not part of `value`): half-split pairs
    fused and pre-rotated, ALiBi alone and composed with fused RoPE (slopes
    2^(-8(h+1)/Hq)). Median of `reps` warm calls each, as the kernel's own
    start-to-end time (rac.time_next_kernel)."""
    base = w["base"]
    Hq = w["Hq"]
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)],
                          dtype=torch.float32, device=qd.device)
    fns = {
        "fused_half_pairs": lambda: rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half"),
        "rope_prerotate_half_pairs": lambda: rac.rope_prerotate_ex(qd, kd, base, "half"),
        "alibi": lambda: rac.attn_alibi_causal_fwd(qd, kd, vd, slopes),
        "alibi_fused_rope": lambda: rac.attn_alibi_causal_fwd(qd, kd, vd, slopes, rope_base=base),
    }
    fl = attn_flops(w)
    res = {}
    for key, fn in fns.items():
        warm(fn, 3, WARM_SECONDS, torch.cuda.synchronize)
        pairs = [(ev(), ev()) for _ in range(reps)]
        for a, b in pairs:
            a.record(); b.record()
        torch.cuda.synchronize()
        for a, b in pairs:  # each call is one kernel: its own start and end
            rac.time_next_kernel(a, b); fn()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in pairs)
        ms = ts[len(ts) // 2]
        if key.startswith("rope_"):
            pb = prerot_bytes(w)
            res[key] = {"ms": ms, "gbs": pb / ms / 1e6, "hbm_frac": pb / ms / 1e6 / HBM_PEAK_GBS}
        else:
            res[key] = {"ms": ms, "tflops": fl / ms / 1e9,
                        "mfma_frac": fl / ms / 1e9 / MFMA_PEAK_TFLOPS[w["dtype"]]}
    return res


def backward(torch, rac, w, qd, kd, vd, out, lse, ev, reps):
    """The backward of both paths on the bench workload, after the timed region
    (not part of `value`): fused (attn_rope_causal_bwd) and pre-rotation
    (rope_prerotate, attn_causal_bwd, rope_prerotate_bwd). TFLOP/s count the
    algorithmic backward work, 2.5 x the forward's (five N^2 products: S, dP,
    dV, dK, dQ); the two-pass kernels rebuild S and dP once more."""
    gen = torch.Generator(device=qd.device).manual_seed(20260913)
    dout = torch.randn(qd.shape, generator=gen, device=qd.device, dtype=torch.float32).to(qd.dtype)
    base = w["base"]
    fns = {"fused": lambda: rac.attn_rope_causal_bwd(qd, kd, vd, out, lse, dout, base),
           "prerotate": lambda: rac.prerotate_path_bwd(qd, kd, vd, out, lse, dout, base)}
    res = {"flops_per_call": 2.5 * attn_flops(w), "dout": "N(0,1) from a seeded torch generator"}
    for key, fn in fns.items():
        warm(fn, 3, WARM_SECONDS, torch.cuda.synchronize)
        pairs = [(ev(), ev()) for _ in range(reps)]
        for a, b in pairs:
            a.record(); fn(); b.record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in pairs)
        ms = ts[len(ts) // 2]
        res[key] = {"ms": ms, "tflops": res["flops_per_call"] / ms / 1e9,
                    "mfma_frac": res["flops_per_call"] / ms / 1e9 / MFMA_PEAK_TFLOPS[w["dtype"]]}
    return res


def crossover(torch, rac, inputs, dev, ev, reps=15):
    """Fused vs pre-rotation path time per shape; N* where their order flips.

    Each path is warmed up for 50 ms, then timed as the median of `reps`
    back-to-back calls, each bracketed by HIP events on the launch stream
    (so both paths' times include their launches). Also per shape: the GQA
    split path, the dispatcher (with a workspace for its preferred path), and
    rope_prerotate bandwidth warm and cold (after a 512 MiB cache flush,
    larger than the 256 MB MALL) from its kernel's own start and end. N* is
    located twice: over the call times, and over the kernels' own times
    (fused kernel vs the pass plus plain attention), which leave out the
    pre-rotation path's second launch."""
    rows = []
    names = ["mha_d64_fp16_n%d" % n for n in inputs.CROSSOVER_NS] + [
        "llama3_8b_gqa_n2048", "llama3_8b_gqa_b4_n4096", "llama3_8b_gqa_n8192"]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for name in names:
        w = inputs.WORKLOADS[name]
        q, k, v = inputs.workload_qkv(name)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        del q, k, v
        base = w["base"]
        o = torch.empty_like(qd)
        lse = torch.empty(qd.shape[:-1], dtype=torch.float32, device=dev)
        qr, kr = torch.empty_like(qd), torch.empty_like(kd)
        krs = torch.empty_like(kd)
        path, need = rac.auto_plan(w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], qd.dtype, 1 << 62)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        fns = {
            "fused": lambda: rac.attn_rope_causal_fwd(qd, kd, vd, base, out=o, lse=lse),
            "prerotate": lambda: (rac.rope_prerotate(qd, kd, base, q_rot=qr, k_rot=kr),
                                  rac.attn_causal_fwd(qr, kr, vd, out=o, lse=lse)),
            "attn": lambda: rac.attn_causal_fwd(qr, kr, vd, out=o, lse=lse),
            "rope": lambda: rac.rope_prerotate(qd, kd, base, q_rot=qr, k_rot=kr),
            "split": lambda: (rac.rope_prerotate_k(kd, base, k_rot=krs),
                              rac.attn_rope_q_causal_fwd(qd, krs, vd, base, out=o, lse=lse)),
            "auto": lambda: rac.attn_rope_causal_auto(qd, kd, vd, base, workspace=ws, out=o,
                                                      lse=lse),
        }
        t = {}
        for key, fn in fns.items():
            warm(fn, 3, 0.05, torch.cuda.synchronize)
            pairs = [(ev(), ev()) for _ in range(reps)]
            for a, b in pairs:
                a.record(); fn(); b.record()
            torch.cuda.synchronize()
            ts = sorted(a.elapsed_time(b) for a, b in pairs)
            t[key] = ts[len(ts) // 2]
        # kernel-only times: each kernel's own start-to-end time
        # (rac.time_next_kernel), warm, and for the streaming pass also after
        # a cache flush; these leave out launches and host work
        def kernel_ms(fn, flushed=False):
            out_ = []
            for _ in range(reps):
                a, b = ev(), ev()
                a.record(); b.record()
                if flushed:
                    flush.zero_()
                rac.time_next_kernel(a, b); fn()
                torch.cuda.synchronize()
                out_.append(a.elapsed_time(b))
            out_.sort()
            return out_[len(out_) // 2]
        t["rope"] = kernel_ms(fns["rope"])
        t_rope_cold = kernel_ms(fns["rope"], flushed=True)
        tk = {key: kernel_ms(fns[key]) for key in ("fused", "attn")}
        fl = attn_flops(w)
        pb = prerot_bytes(w)
        fastest = min(("fused", "prerotate", "split"), key=lambda p: t[p])
        rows.append({"workload": name, "N": w["N"], "fused_ms": t["fused"],
                     "prerotate_ms": t["prerotate"], "attn_only_ms": t["attn"],
                     "split_ms": t["split"], "auto_ms": t["auto"],
                     "auto_path": rac.PATH_NAMES[path], "fastest_path": fastest,
                     "fused_tflops": fl / t["fused"] / 1e9,
                     "prerotate_tflops": fl / t["prerotate"] / 1e9,
                     "attn_only_tflops": fl / t["attn"] / 1e9,
                     "fused_overhead_vs_plain": t["fused"] / t["attn"] - 1.0,
                     "fused_vs_prerotate_gap": t["fused"] / t["prerotate"] - 1.0,
                     "fused_kernel_ms": tk["fused"], "attn_kernel_ms": tk["attn"],
                     "prerotate_kernels_ms": t["rope"] + tk["attn"],
                     "fused_vs_prerotate_kernel_gap": tk["fused"] / (t["rope"] + tk["attn"]) - 1.0,
                     "rope_prerotate_ms": t["rope"], "rope_prerotate_gbs": pb / t["rope"] / 1e6,
                     "rope_prerotate_cold_ms": t_rope_cold,
                     "rope_prerotate_cold_gbs": pb / t_rope_cold / 1e6,
                     "rope_prerotate_cold_hbm_frac": pb / t_rope_cold / 1e6 / HBM_PEAK_GBS})
        del qd, kd, vd, o, lse, qr, kr, krs, ws
        torch.cuda.empty_cache()
    sweep = [r for r in rows if r["workload"].startswith("mha_d64")]
    calls = locate_crossover(sweep, "fused_ms", "prerotate_ms")
    kernels = locate_crossover(sweep, "fused_kernel_ms", "prerotate_kernels_ms")
    return {"n_star": calls["n_star"], "bracket": calls["bracket"],
            "gaps_at_bracket": calls["gaps_at_bracket"],
            "winner_if_no_crossing": calls["winner_if_no_crossing"],
            "kernels": kernels,
            "sweep": "mha_d64_fp16 N=1024..32768 (B=1, H=16)", "rows": rows}


def locate_crossover(sweep, fused_key, pre_key):
    """N* over the sweep rows (ascending N): the first sign change of
    t_fused − t_prerotate, log-linearly interpolated in the relative gap;
    with no change, which path won at every N ("mixed" if neither)."""
    n_star = bracket = gaps = winner = None
    for a, b in zip(sweep, sweep[1:]):
        da = a[fused_key] - a[pre_key]
        db = b[fused_key] - b[pre_key]
        if (da < 0) != (db < 0):
            ga, gb = da / a[pre_key], db / b[pre_key]
            x = ga / (ga - gb)
            n_star = math.exp(math.log(a["N"]) + x * (math.log(b["N"]) - math.log(a["N"])))
            bracket = [a["N"], b["N"]]
            # the relative gaps at the bracket's ends: a sign change between
            # gaps of a few percent is within the run-to-run spread
            gaps = [r[fused_key] / r[pre_key] - 1.0 for r in (a, b)]
            break
    if n_star is None and sweep:
        winner = "fused" if all(r[fused_key] < r[pre_key] for r in sweep) else (
            "prerotate" if all(r[fused_key] > r[pre_key] for r in sweep) else "mixed")
    return {"n_star": n_star, "bracket": bracket, "gaps_at_bracket": gaps,
            "winner_if_no_crossing": winner}


def cpu_baseline(inputs, w, min_seconds=10.0):
    """The fp64 oracle on this host over the full workload (one pass)."""
    import oracle
    q, k, v = inputs.workload_qkv(MAIN)
    qb, kb, vb = inputs.bits(q), inputs.bits(k), inputs.bits(v)
    passes = 0
    t0 = time.perf_counter()
    while True:  # whole passes until at least min_seconds of CPU work
        oracle.rope_attention(qb, kb, vb, w["dtype"], w["base"], variant="rounded")
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 200:
            break
    return {"value": passes * attn_flops(w) / dt / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "seconds": dt, "passes": passes,
            "sample": "the full %s workload, %d pass(es): fp64 RoPE of Q and K, then "
                      "two-pass causal attention over every query row; FLOPs counted as "
                      "2*B*Hq*N^2*D per pass, as for the GPU" % (MAIN, passes)}


if __name__ == "__main__":
    main()
