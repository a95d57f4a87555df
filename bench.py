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
    peak; warm (the timed steps) and cold (after a 512 MiB flush); and
    against that peak scaled to the GFX clock sampled (amd-smi) while the
    kernel runs back to back (`frac_at_sclk`);
  * paths: per-kernel times taken the same way (warm, and cold after a
    512 MiB cache flush) and their sums per path, TFLOP/s, % of MFMA peak,
    rope_prerotate GB/s vs 8 TB/s and vs a plain copy of the same bytes
    with the same access pattern (rac.stream_copy), warm and cold;
    also the GQA split path (rope_prerotate_k then attn_rope_q_causal_fwd),
    timed after the step loop and not part of `value`;
  * crossover: fused vs pre-rotation (and split) times over six families
    (D=64 fp16 MHA N = 1024 .. 32768; D=128 bf16 MHA; GQA 4:1 at D=64 bf16
    and D=128 bf16/fp16; GQA 8:1 at D=128 bf16), three interleaved repeats,
    the measured N* per family (kernel level, the headline; and call level),
    and the Rotation Calculus model fitted to the same rows with its N*;
  * variants: the half-split RoPE pairing (fused and pre-rotated) and the
    ALiBi score modification (alone and with fused RoPE), timed after the
    step loop and not part of `value`;
  * cpu_baseline: the fp64 CPU oracle timed on this host over the full
    workload (rotation + causal attention), in the same unit.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
       [--no-cpu] [--only fused|prerotate|rope|attn|split|rope_k|attn_q|bwd|bwd_prerotate
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


NOMINAL_SCLK_MHZ = 2400.0  # the clock the published MFMA peak is quoted at


def parse_gfx_clocks(text):
    """The GFX clocks (MHz) in the JSON that `amd-smi metric -c --json` prints:
    one value per XCD ("gfx_0" ...) of every GPU listed, leaving out XCDs
    caught below their lowest clock level (min_clk, else 500 MHz), which are
    in deep sleep at that instant rather than running slower. Empty if none."""
    try:
        data = json.loads(text)
    except ValueError:
        return []
    gpus = data.get("gpu_data", []) if isinstance(data, dict) else data
    mhz = []

    def value(c, key):
        v = c.get(key, {})
        v = v.get("value") if isinstance(v, dict) else v
        return float(v) if isinstance(v, (int, float)) else None

    for g in gpus if isinstance(gpus, list) else []:
        clocks = g.get("clock", {}) if isinstance(g, dict) else {}
        for key, c in sorted(clocks.items()):
            if key.startswith("gfx_") and isinstance(c, dict):
                v, lo = value(c, "clk"), value(c, "min_clk")
                if v is not None and v >= (lo if lo else 500.0):
                    mhz.append(v)
    return mhz


def gfx_clock_under(fn, sync, seconds=1.0):
    """Per-XCD GFX clocks while fn runs back to back for about `seconds`: a
    helper thread samples `amd-smi metric -c --json` (a child process that
    reads the driver's metrics) while this thread keeps the GPU busy.
    Returns the median, min and max MHz over all samples and XCDs, or None
    when amd-smi is unavailable or reports nothing."""
    import subprocess
    import threading
    samples, done = [], threading.Event()

    def sampler():
        while not done.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True,
                                   text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            if r.returncode != 0:
                return
            samples.append(parse_gfx_clocks(r.stdout))
            done.wait(0.05)

    warm(fn, 20, 0.1, sync)  # clocks up before the first sample
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and th.is_alive():
        for _ in range(100):
            fn()
        sync()
    done.set()
    th.join()
    mhz = sorted(m for smp in samples for m in smp)
    if not mhz:
        return None
    return {"median_mhz": _median(mhz), "min_mhz": mhz[0], "max_mhz": mhz[-1],
            "readings": len(mhz), "samples": len(samples),
            "source": "amd-smi metric -c (per-XCD GFX clock, XCDs in deep sleep left out), "
                      "sampled while the kernel runs back to back"}


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
                                       "attn_q", "bwd", "bwd_prerotate"], default=None,
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
        fns = {"fused": fused, "rope": rope, "attn": attn,
               "prerotate": lambda: (rope(), attn()), "rope_k": rope_k, "attn_q": attn_q,
               "split": lambda: (rope_k(), attn_q())}
        if args.only.startswith("bwd"):
            # the backward of the fused path or of the pre-rotation path, from the
            # fused forward's out and lse and a seeded dO
            fused()
            gen = torch.Generator(device=dev).manual_seed(20260913)
            dout = torch.randn(qd.shape, generator=gen, device=dev,
                               dtype=torch.float32).to(qd.dtype)
            fns["bwd"] = lambda: rac.attn_rope_causal_bwd(qd, kd, vd, out_f, lse_f, dout, base)
            fns["bwd_prerotate"] = lambda: rac.prerotate_path_bwd(qd, kd, vd, out_f, lse_f, dout,
                                                                  base)
        if args.only == "attn":
            rope()  # the plain kernel reads the rotated operands: write them first
        if args.only == "attn_q":
            rope_k()
        fn = fns[args.only]
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

    # the GFX clock while the roofline kernel runs: its peak at that clock
    sclk = gfx_clock_under(fused, torch.cuda.synchronize)

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
    # the pass's ceiling: a plain copy of as many bytes as it reads (then
    # writes), with its access pattern, warm and cold, in this same run
    csrc = torch.empty(int(pb // 2), dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    copy = lambda: rac.stream_copy(csrc, cdst)  # noqa: E731
    warm(copy, args.warmup, WARM_SECONDS / 4, torch.cuda.synchronize)
    copy_ev = made([(ev(), ev()) for _ in range(args.steps)])
    for a, b in copy_ev:
        rac.time_next_kernel(a, b); copy()
    torch.cuda.synchronize()
    t_copy, c_copy = avg_ms(copy_ev), cold(copy)
    del csrc, cdst

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
                           "cold_hbm_frac": pb / c_rope / 1e6 / HBM_PEAK_GBS, "bytes": pb,
                           "copy_ceiling": {"ms": t_copy, "gbs": pb / t_copy / 1e6,
                                            "cold_ms": c_copy, "cold_gbs": pb / c_copy / 1e6,
                                            "cold_hbm_frac": pb / c_copy / 1e6 / HBM_PEAK_GBS},
                           "frac_of_copy": t_copy / t_rope, "cold_frac_of_copy": c_copy / c_rope},
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
                     "frac": achieved / peak, "traffic": measured_traffic(),
                     "achieved_cold": fl / (c_fused * 1e-3) / 1e12,
                     "frac_cold": fl / (c_fused * 1e-3) / 1e12 / peak,
                     "cold": "median of 20 launches, each after a 512 MiB cache flush"},
        "paths": paths,
    }
    if sclk is not None:
        # the published peak scaled to the clock measured under this kernel
        result["roofline"]["sclk"] = sclk
        result["roofline"]["frac_at_sclk"] = achieved / (peak * sclk["median_mhz"] / NOMINAL_SCLK_MHZ)

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
    (rope_prerotate, attn_causal_bwd, rope_prerotate_bwd), both again with the
    half-split RoPE pairing (from the half-split forward's out and lse), and
    the fused backward with the ALiBi penalty (slopes 2^(-8(h+1)/Hq)) after
    adjacent-pair RoPE.
    TFLOP/s count the algorithmic backward work, 2.5 x the forward's (five N^2
    products: S, dP, dV, dK, dQ); the two-pass kernels rebuild S and dP once
    more."""
    gen = torch.Generator(device=qd.device).manual_seed(20260913)
    dout = torch.randn(qd.shape, generator=gen, device=qd.device, dtype=torch.float32).to(qd.dtype)
    base = w["base"]
    out_h, lse_h = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / w["Hq"]) for h in range(w["Hq"])],
                          dtype=torch.float32, device=qd.device)
    out_a, lse_a = rac.attn_alibi_causal_fwd(qd, kd, vd, slopes, rope_base=base)
    fns = {"fused": lambda: rac.attn_rope_causal_bwd(qd, kd, vd, out, lse, dout, base),
           "prerotate": lambda: rac.prerotate_path_bwd(qd, kd, vd, out, lse, dout, base),
           "fused_half": lambda: rac.attn_rope_causal_bwd_ex(qd, kd, vd, out_h, lse_h, dout, base,
                                                             "half"),
           "prerotate_half": lambda: rac.prerotate_path_bwd(qd, kd, vd, out_h, lse_h, dout, base,
                                                            "half"),
           "fused_alibi": lambda: rac.attn_alibi_causal_bwd(qd, kd, vd, out_a, lse_a, dout, slopes,
                                                            rope_base=base)}
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


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _stage_row(torch, rac, inputs, name, dev):
    """Device tensors of one crossover row (timing-only inputs drawn on the
    device) and the callables that time each path and kernel."""
    w = inputs.WORKLOADS[name]
    qd, kd, vd = inputs.device_qkv(name, dev)
    base = w["base"]
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:-1], dtype=torch.float32, device=dev)
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    krs = torch.empty_like(kd)
    path, need = rac.auto_plan(w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], qd.dtype, 1 << 62)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    # the copy ceiling: as many bytes as the pass reads (and then writes)
    pb = prerot_bytes(w)
    csrc = torch.empty(int(pb // 2), dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    fns = {
        "fused": lambda: rac.attn_rope_causal_fwd(qd, kd, vd, base, out=o, lse=lse),
        "rope": lambda: rac.rope_prerotate(qd, kd, base, q_rot=qr, k_rot=kr),
        "attn": lambda: rac.attn_causal_fwd(qr, kr, vd, out=o, lse=lse),
        "rope_k": lambda: rac.rope_prerotate_k(kd, base, k_rot=krs),
        "attn_q": lambda: rac.attn_rope_q_causal_fwd(qd, krs, vd, base, out=o, lse=lse),
        "copy": lambda: rac.stream_copy(csrc, cdst),
        "auto": lambda: rac.attn_rope_causal_auto(qd, kd, vd, base, workspace=ws, out=o,
                                                  lse=lse),
    }
    fns["prerotate"] = lambda: (fns["rope"](), fns["attn"]())  # noqa: E731
    fns["split"] = lambda: (fns["rope_k"](), fns["attn_q"]())
    return {"w": w, "fns": fns, "auto_path": rac.PATH_NAMES[path],
            "keep": (qd, kd, vd, o, lse, qr, kr, krs, ws, csrc, cdst)}


def _events(torch, n):
    """n pairs of timing events, created up front (torch creates the HIP
    event at its first record)."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for a, b in pairs:
        a.record(); b.record()
    torch.cuda.synchronize()
    return pairs


def _time_row(torch, rac, st, flush, reps, warm_s):
    """One repeat of one row. Each path is warmed up, then called `reps`
    times back to back (steady clocks, as in a model's step) with events
    around each call, then `reps` times more with each of its kernels timed
    by the events it records at its own start and end (rac.time_next_kernel;
    those records lengthen the calls, so the two are kept apart); medians.
    The pass and the copy are also timed cold, one launch at a time after a
    512 MiB flush written (zero_) or only read (max)."""
    fns = st["fns"]
    t = {}
    plans = (("fused", ("fused",)), ("prerotate", ("rope", "attn")),
             ("split", ("rope_k", "attn_q")), ("auto", ()), ("copy", ("copy",)))
    for path, kernels in plans:
        warm(fns[path], 3, warm_s, torch.cuda.synchronize)
        if path != "copy":
            # calls alone: the kernel timer's events are not recorded here
            calls = _events(torch, reps)
            for a, b in calls:
                a.record(); fns[path](); b.record()
            torch.cuda.synchronize()
            t["c_" + path] = _median([a.elapsed_time(b) for a, b in calls]) * 1e3
        kev = {k: _events(torch, reps) for k in kernels}
        for i in range(reps):
            for k in kernels:
                rac.time_next_kernel(*kev[k][i]); fns[k]()
        torch.cuda.synchronize()
        for k in kernels:
            t["k_" + k] = _median([a.elapsed_time(b) for a, b in kev[k]]) * 1e3

    def cold_us(fn, how):
        out_ = []
        for a, b in _events(torch, reps):
            if how == "write":
                flush.zero_()
            else:
                flush.max()
            rac.time_next_kernel(a, b); fn()
            torch.cuda.synchronize()
            out_.append(a.elapsed_time(b))
        return _median(out_) * 1e3

    for key in ("rope", "copy"):
        t["k_%s_cold" % key] = cold_us(fns[key], "write")
        t["k_%s_cold_read" % key] = cold_us(fns[key], "read")
    return t


def crossover(torch, rac, inputs, dev, ev, repeats=3, reps=11):
    """Fused vs pre-rotation (and GQA split) over the crossover families,
    each row timed `repeats` times (interleaved: one pass over every row,
    then the next), and the Rotation Calculus model fitted to the same rows.

    Per row and time: the median over repeats (each repeat's own figure is
    the median of `reps` calls), and the min/median/max of the fused vs
    pre-rotation gap over repeats. N* per family is located twice: over the
    kernels' own times (the fused kernel vs the pass plus plain attention;
    the headline) and over call times (which add the pre-rotation path's
    second launch). The model (rotary_position_embedding_causal_amd.
    dispatch_fit) is fitted to the median kernel times of all rows, and its
    N* per family set beside the measured one; the dispatcher's own constants
    (csrc/dispatch_model.h) are checked against the call times: auto_ms vs
    the fastest path per row."""
    from rotary_position_embedding_causal_amd import dispatch_fit
    fams = inputs.CROSSOVER_FAMILIES
    names = [n for _, rows in fams.values() for n in rows] + list(inputs.CROSSOVER_EXTRA)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    staged = {name: _stage_row(torch, rac, inputs, name, dev) for name in names}
    samples = {name: [] for name in names}
    for r in range(repeats):
        for name in names:
            samples[name].append(_time_row(torch, rac, staged[name], flush, reps,
                                           0.05 if r == 0 else 0.02))
        print("crossover repeat %d/%d done" % (r + 1, repeats), file=sys.stderr, flush=True)
    rows = []
    for name in names:
        st, ts = staged[name], samples[name]
        w = st["w"]
        med = {key: _median([t[key] for t in ts]) for key in ts[0]}
        fl, pb, kb = attn_flops(w), prerot_bytes(w), prerot_k_bytes(w)
        gk = sorted(t["k_fused"] / (t["k_rope"] + t["k_attn"]) - 1.0 for t in ts)
        gc = sorted(t["c_fused"] / t["c_prerotate"] - 1.0 for t in ts)
        calls = {p: med["c_" + p] for p in ("fused", "prerotate", "split")}
        fastest = min(calls, key=calls.get)
        row = {"workload": name, "B": w["B"], "Hq": w["Hq"], "Hkv": w["Hkv"], "N": w["N"],
               "D": w["D"], "dtype": w["dtype"]}
        row.update({k_: v_ for k_, v_ in med.items()})
        row.update({
            "auto_path": st["auto_path"], "fastest_path": fastest,
            "auto_vs_fastest": med["c_auto"] / calls[fastest] - 1.0,
            "gap_kernels": {"min": gk[0], "median": _median(gk), "max": gk[-1]},
            "gap_calls": {"min": gc[0], "median": _median(gc), "max": gc[-1]},
            "fused_tflops": fl / med["k_fused"] / 1e6,
            "attn_tflops": fl / med["k_attn"] / 1e6,
            "attn_q_tflops": fl / med["k_attn_q"] / 1e6,
            "fused_mfma_frac": fl / med["k_fused"] / 1e6 / MFMA_PEAK_TFLOPS[w["dtype"]],
            "attn_mfma_frac": fl / med["k_attn"] / 1e6 / MFMA_PEAK_TFLOPS[w["dtype"]],
            "rope_gbs": pb / med["k_rope"] / 1e3,
            "rope_cold_gbs": pb / med["k_rope_cold"] / 1e3,
            "rope_cold_hbm_frac": pb / med["k_rope_cold"] / 1e3 / HBM_PEAK_GBS,
            "rope_cold_read_hbm_frac": pb / med["k_rope_cold_read"] / 1e3 / HBM_PEAK_GBS,
            "copy_gbs": pb / med["k_copy"] / 1e3,
            "copy_cold_hbm_frac": pb / med["k_copy_cold"] / 1e3 / HBM_PEAK_GBS,
            "copy_cold_read_hbm_frac": pb / med["k_copy_cold_read"] / 1e3 / HBM_PEAK_GBS,
            "rope_k_gbs": kb / med["k_rope_k"] / 1e3,
            "samples": ts})
        rows.append(row)
    del staged
    torch.cuda.empty_cache()

    # the model, fitted to this run's rows
    fit = dispatch_fit.fit(rows)
    header = dispatch_fit.load_params()
    byname = {r["workload"]: r for r in rows}
    families = {}
    for fam, (desc, fam_rows) in fams.items():
        sweep = [byname[n] for n in fam_rows]
        w0 = sweep[0]
        cls = dispatch_fit.class_key(w0["D"], w0["Hq"], w0["Hkv"])
        kern = locate_crossover(sweep, "k_fused", None, pre_fn=lambda r: r["k_rope"] + r["k_attn"])
        per_rep = []
        for i in range(repeats):
            reps_i = [dict(N=r["N"], f=r["samples"][i]["k_fused"],
                           p=r["samples"][i]["k_rope"] + r["samples"][i]["k_attn"]) for r in sweep]
            per_rep.append(locate_crossover(reps_i, "f", "p")["n_star"])
        callx = locate_crossover(sweep, "c_fused", "c_prerotate")
        worst = max(r["auto_vs_fastest"] for r in sweep)
        families[fam] = {
            "desc": desc, "class": cls, "N": [r["N"] for r in sweep],
            "n_star_kernels": kern, "n_star_kernels_per_repeat": per_rep,
            "n_star_calls": callx,
            "auto_worst_vs_fastest": worst, "auto_within_2pct": worst <= 0.02}
    dispatch_fit.family_models(fit, families, byname)
    for r in rows:
        del r["samples"]  # per-repeat figures: summarised above
    head = families["mha_d64_fp16"]
    model = dict(dispatch_fit.headline_model(fit, families), fit=fit,
                 fit_errors=dispatch_fit.fit_errors(fit, rows),
                 dispatcher_constants=header, form=dispatch_fit.FORM)
    return {"n_star": head["n_star_kernels"]["n_star"],
            "level": "kernels (the fused kernel vs the pass plus plain attention)",
            "bracket": head["n_star_kernels"]["bracket"],
            "gaps_at_bracket": head["n_star_kernels"]["gaps_at_bracket"],
            "n_star_per_repeat": head["n_star_kernels_per_repeat"],
            "n_star_calls": head["n_star_calls"]["n_star"],
            "winner_if_no_crossing": head["n_star_kernels"]["winner_if_no_crossing"],
            "model": model, "families": families, "repeats": repeats,
            "sweep": "mha_d64_fp16 N=1024..32768 (B=1, H=16)", "rows": rows}


def locate_crossover(sweep, fused_key, pre_key, pre_fn=None):
    """N* over the sweep rows (ascending N): the first sign change of
    t_fused - t_prerotate, log-linearly interpolated in the relative gap;
    with no change, which path won at every N ("mixed" if neither)."""
    pre = pre_fn or (lambda r: r[pre_key])
    n_star = bracket = gaps = winner = None
    for a, b in zip(sweep, sweep[1:]):
        da = a[fused_key] - pre(a)
        db = b[fused_key] - pre(b)
        if (da < 0) != (db < 0):
            ga, gb = da / pre(a), db / pre(b)
            x = ga / (ga - gb)
            n_star = math.exp(math.log(a["N"]) + x * (math.log(b["N"]) - math.log(a["N"])))
            bracket = [a["N"], b["N"]]
            # the relative gaps at the bracket's ends: a sign change between
            # gaps of a few percent is within the run-to-run spread
            gaps = [r[fused_key] / pre(r) - 1.0 for r in (a, b)]
            break
    if n_star is None and sweep:
        winner = "fused" if all(r[fused_key] < pre(r) for r in sweep) else (
            "prerotate" if all(r[fused_key] > pre(r) for r in sweep) else "mixed")
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
