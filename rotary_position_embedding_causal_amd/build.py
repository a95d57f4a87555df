"""Builds librac.so (the C ABI of include/rac.h) for gfx950 with hipcc.

Every HIP source is compiled with packed-FP32 instructions disabled and no
floating-point contraction beyond the fused multiply-adds written out in the
source, so that the RoPE rotation is evaluated identically in every kernel.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
CSRC = os.path.join(_HERE, "csrc")
LIB = os.path.join(_HERE, "librac.so")
SOURCES = ["rac_api.hip", "attn_fwd.hip", "attn_bwd.hip", "rope_prerotate.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=" + ARCH, "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-result"]


# Extra flags per source. The attention kernels never see NaNs from finite
# inputs (masking uses -inf), so fmax needs no NaN-quieting canonicalisation.
EXTRA = {"attn_fwd.hip": ["-fno-honor-nans"], "attn_bwd.hip": ["-fno-honor-nans"]}


# The forward attention kernels compile as one object per (dtype, head dim,
# rotation mode), in parallel, plus the dispatcher (the same source with no
# part selected); see the end of attn_fwd.hip.
FWD_MODES = (0, 1, 2, 3, 4, 5, 7)  # ROT_* | MOD_ALIBI combinations the dispatcher uses
FWD_PARTS = [(dt, d, m) for dt in (0, 1) for d in (64, 128) for m in FWD_MODES]


def _jobs(objdir):
    """(source, object, extra flags) for every object of the library."""
    jobs = []
    for src in SOURCES:
        if src == "attn_fwd.hip":
            for dt, d, m in FWD_PARTS:
                jobs.append((src, os.path.join(objdir, "attn_fwd_%d_%d_%d.o" % (dt, d, m)),
                             ["-DRAC_FWD_DT=%d" % dt, "-DRAC_FWD_D=%d" % d, "-DRAC_FWD_MODE=%d" % m]))
        jobs.append((src, os.path.join(objdir, src.replace(".hip", ".o")), []))
    return jobs


def _compile(src, obj, verbose, defs=()):
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + list(defs) + ["-c", os.path.join(CSRC, src),
                                                                "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip() and verbose:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build", "rac")
    os.makedirs(objdir, exist_ok=True)
    jobs = _jobs(objdir)
    objs = [j[1] for j in jobs]
    # largest parts first, so the long compiles start early
    order = sorted(jobs, key=lambda j: ("_128_" not in j[1], j[1]))
    with ThreadPoolExecutor(max_workers=max(2, os.cpu_count() or 2)) as ex:
        list(ex.map(lambda j: _compile(j[0], j[1], verbose, j[2]), order))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """The same library with its host code (the C ABI: validation, the table
    cache, the path planner) built with AddressSanitizer and
    UndefinedBehaviorSanitizer (-Xarch_host: the device code is unchanged),
    into _build/asan/librac.so, for the CPU tests with the ROCm clang's ASan
    runtime preloaded (see tests/conftest.py). The kernels' objects come from
    the regular build."""
    objdir = os.path.join(ROOT, "_build", "rac")
    asandir = os.path.join(ROOT, "_build", "asan")
    os.makedirs(asandir, exist_ok=True)
    jobs = _jobs(objdir)
    if not all(os.path.exists(j[1]) for j in jobs):
        build(verbose)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    api_obj = os.path.join(asandir, "rac_api.o")
    _compile("rac_api.hip", api_obj, verbose, san)
    objs = [api_obj if os.path.basename(j[1]) == "rac_api.o" else j[1] for j in jobs]
    out = os.path.join(asandir, "librac.so")
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-shared-libsan",
           "-fsanitize=address,undefined", "-o", out] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
