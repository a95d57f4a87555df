"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module holds no arithmetic of the method: it only draws Q, K, V and
rounds them to the storage dtype, so that the GPU path and the oracle read
the very same bits.

Recipe: each tensor is drawn i.i.d. N(0, sigma^2) in fp32 by numpy's PCG64
generator seeded with ``SeedSequence([20260913, *key, t])`` (t = 0 for q,
1 for k, 2 for v), then rounded to bf16/fp16 round-to-nearest-even by torch
on the CPU. Layout is contiguous [B, H, N, D].

The workloads below are the attention-layer shapes the measurements use:
a tiny MHA case, Llama-3-8B-shaped GQA layers (32 query heads sharing 8 key/
value heads, head dim 128, RoPE base 500000) at N = 2048, 4096 (batch 4) and
8192, a D = 64 fp16 MHA sweep over N (1024 to 32768) for the
fused/pre-rotate crossover, and the crossover's other families (MHA at
D = 128, GQA 4:1 and 8:1 at D = 64 and 128, bf16 and fp16).
No trained weights or real activations are available, so N(0,1) tensors of
these shapes stand in for them.
"""
from __future__ import annotations

import numpy as np
import torch

SEED_ROOT = 20260913

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}

# name -> shape dictionary
WORKLOADS = {
    "tiny_mha_n512_d64": dict(B=1, Hq=4, Hkv=4, N=512, D=64, dtype="bf16", base=10000.0),
    "llama3_8b_gqa_n2048": dict(B=1, Hq=32, Hkv=8, N=2048, D=128, dtype="bf16", base=500000.0),
    "llama3_8b_gqa_b4_n4096": dict(B=4, Hq=32, Hkv=8, N=4096, D=128, dtype="bf16",
                                   base=500000.0),
    "llama3_8b_gqa_n8192": dict(B=1, Hq=32, Hkv=8, N=8192, D=128, dtype="bf16", base=500000.0),
}
SWEEP_NS = (2048, 4096, 6144, 8192, 16384, 32768)
for _n in SWEEP_NS:
    WORKLOADS["mha_d64_fp16_n%d" % _n] = dict(B=1, Hq=16, Hkv=16, N=_n, D=64, dtype="fp16",
                                              base=10000.0)
# one point below the sweep, where the fused kernel is expected to lead
# (appended after the others so that their seed keys stay as they were)
CROSSOVER_NS = (1024,) + SWEEP_NS
WORKLOADS["mha_d64_fp16_n1024"] = dict(B=1, Hq=16, Hkv=16, N=1024, D=64, dtype="fp16",
                                       base=10000.0)
# the crossover envelope beyond the D = 64 fp16 MHA sweep: MHA at D = 128
# (bf16, 32 heads; one batch-8 row of the same layer), GQA 4:1 at D = 64
# bf16 and at D = 128 fp16, GQA 8:1 at D = 128 bf16 (64 query heads over 8
# key/value heads), and more lengths of the Llama-3-8B layer (appended)
for _n in (1024, 2048, 4096, 8192, 16384):
    WORKLOADS["mha_d128_bf16_n%d" % _n] = dict(B=1, Hq=32, Hkv=32, N=_n, D=128, dtype="bf16",
                                               base=10000.0)
WORKLOADS["mha_d128_bf16_b8_n1024"] = dict(B=8, Hq=32, Hkv=32, N=1024, D=128, dtype="bf16",
                                           base=10000.0)
for _n in (1024, 2048, 4096, 8192, 16384):
    WORKLOADS["gqa4_d64_bf16_n%d" % _n] = dict(B=1, Hq=32, Hkv=8, N=_n, D=64, dtype="bf16",
                                               base=10000.0)
for _n in (1024, 2048, 4096, 8192):
    WORKLOADS["gqa4_d128_fp16_n%d" % _n] = dict(B=1, Hq=32, Hkv=8, N=_n, D=128, dtype="fp16",
                                                base=500000.0)
for _n in (1024, 2048, 4096, 8192):
    WORKLOADS["gqa8_d128_bf16_n%d" % _n] = dict(B=1, Hq=64, Hkv=8, N=_n, D=128, dtype="bf16",
                                                base=500000.0)
for _n in (1024, 4096, 16384):
    WORKLOADS["llama3_8b_gqa_n%d" % _n] = dict(B=1, Hq=32, Hkv=8, N=_n, D=128, dtype="bf16",
                                               base=500000.0)

# midpoints around the crossovers (1.5K, 3K) for every family
for _n in (1536, 3072):
    WORKLOADS["mha_d64_fp16_n%d" % _n] = dict(B=1, Hq=16, Hkv=16, N=_n, D=64, dtype="fp16",
                                              base=10000.0)
    WORKLOADS["mha_d128_bf16_n%d" % _n] = dict(B=1, Hq=32, Hkv=32, N=_n, D=128, dtype="bf16",
                                               base=10000.0)
    WORKLOADS["gqa4_d64_bf16_n%d" % _n] = dict(B=1, Hq=32, Hkv=8, N=_n, D=64, dtype="bf16",
                                               base=10000.0)
    WORKLOADS["llama3_8b_gqa_n%d" % _n] = dict(B=1, Hq=32, Hkv=8, N=_n, D=128, dtype="bf16",
                                               base=500000.0)
    WORKLOADS["gqa4_d128_fp16_n%d" % _n] = dict(B=1, Hq=32, Hkv=8, N=_n, D=128, dtype="fp16",
                                                base=500000.0)
    WORKLOADS["gqa8_d128_bf16_n%d" % _n] = dict(B=1, Hq=64, Hkv=8, N=_n, D=128, dtype="bf16",
                                                base=500000.0)

# crossover families: (description, row names in ascending N); one family
# shares D, dtype and Hq/Hkv, and within it only N changes (B = 1)
CROSSOVER_FAMILIES = {
    "mha_d64_fp16": ("MHA D=64 fp16, B=1 H=16",
                     ["mha_d64_fp16_n%d" % n for n in (1024, 1536, 2048, 3072, 4096, 6144, 8192,
                                                       16384, 32768)]),
    "mha_d128_bf16": ("MHA D=128 bf16, B=1 H=32",
                      ["mha_d128_bf16_n%d" % n for n in (1024, 1536, 2048, 3072, 4096, 8192,
                                                         16384)]),
    "gqa4_d64_bf16": ("GQA 4:1 D=64 bf16, B=1 Hq=32 Hkv=8",
                      ["gqa4_d64_bf16_n%d" % n for n in (1024, 1536, 2048, 3072, 4096, 8192,
                                                         16384)]),
    "gqa4_d128_bf16": ("GQA 4:1 D=128 bf16 (Llama-3-8B layer), B=1 Hq=32 Hkv=8",
                       ["llama3_8b_gqa_n%d" % n for n in (1024, 1536, 2048, 3072, 4096, 8192,
                                                          16384)]),
    "gqa4_d128_fp16": ("GQA 4:1 D=128 fp16, B=1 Hq=32 Hkv=8",
                       ["gqa4_d128_fp16_n%d" % n for n in (1024, 1536, 2048, 3072, 4096, 8192)]),
    "gqa8_d128_bf16": ("GQA 8:1 D=128 bf16, B=1 Hq=64 Hkv=8",
                       ["gqa8_d128_bf16_n%d" % n for n in (1024, 1536, 2048, 3072, 4096, 8192)]),
}
# rows outside the families: other batch sizes of a family's layer
CROSSOVER_EXTRA = ["mha_d128_bf16_b8_n1024", "llama3_8b_gqa_b4_n4096"]

# seed keys: a workload's position in this table (stable: append only)
SEED_KEYS = {name: (i + 1,) for i, name in enumerate(WORKLOADS)}


def draw(shape, dtype: str, key, tensor_index: int, sigma: float = 1.0) -> torch.Tensor:
    """One seeded N(0, sigma^2) tensor, rounded to ``dtype``, on the CPU."""
    ss = np.random.SeedSequence([SEED_ROOT, *[int(x) for x in key], int(tensor_index)])
    rng = np.random.default_rng(ss)
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype])


def qkv(B: int, Hq: int, Hkv: int, N: int, D: int, dtype: str, key, sigma: float = 1.0):
    """Seeded (q, k, v) CPU tensors: q [B,Hq,N,D]; k, v [B,Hkv,N,D]."""
    q = draw((B, Hq, N, D), dtype, key, 0, sigma)
    k = draw((B, Hkv, N, D), dtype, key, 1, sigma)
    v = draw((B, Hkv, N, D), dtype, key, 2, sigma)
    return q, k, v


def workload_qkv(name: str, sigma: float = 1.0):
    w = WORKLOADS[name]
    return qkv(w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["dtype"], SEED_KEYS[name], sigma)


def device_qkv(name: str, device):
    """Timing-only inputs: (q, k, v) of a workload drawn i.i.d. N(0, 1) on the
    device by torch's generator seeded with SEED_ROOT and the workload's key,
    then rounded to its dtype -- the same shapes and distribution as
    workload_qkv without the CPU draw. Not bit-equal to workload_qkv: nothing
    checks values against them."""
    w = WORKLOADS[name]
    g = torch.Generator(device=device).manual_seed(SEED_ROOT * 1000 + SEED_KEYS[name][0])
    out = []
    for h in (w["Hq"], w["Hkv"], w["Hkv"]):
        x = torch.randn((w["B"], h, w["N"], w["D"]), generator=g, device=device,
                        dtype=torch.float32)
        out.append(x.to(TORCH_DTYPES[w["dtype"]]))
        del x
    return tuple(out)


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16/fp16 CPU tensor, as uint16 numpy."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
