"""attn_rope_causal_fwd_noalloc, the entry point for callers that cannot
allocate device memory, against attn_rope_causal_fwd (the entry point it is a
variant of): four calls in a row through the C ABI into preallocated outputs,
each with a smaller input than the one before -- the first two fill the
static table to its capacity, at D = 64 and D = 128 -- and the rope_base
changing along the way (each call rebuilds its table rows in the static
array), to the parity bounds (O max-abs 2e-2, rel-L2 1e-2; LSE 1e-3)."""
import ctypes

import numpy as np
import pytest
import torch

import rotary_position_embedding_causal_amd as rac
from rotary_position_embedding_causal_amd import inputs
from parity import assert_lse, assert_o, to_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(q, k, v, out, lse, base, stream):
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    dt = rac.RAC_BF16 if q.dtype == torch.bfloat16 else rac.RAC_FP16
    return rac.lib().attn_rope_causal_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                 B, Hq, Hkv, N, D, base, dt, stream)


def test_noalloc_matches_fused_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    cases = [  # (B, Hq, Hkv, N, D, dtype, base, key): each call smaller than the one before
        # the static table's full capacity: N * D = RAC_NOALLOC_MAX_N * 128 at D = 64 and 128
        (1, 1, 1, 2 * rac.RAC_NOALLOC_MAX_N, 64, "fp16", 10000.0, (503,)),
        (1, 2, 1, rac.RAC_NOALLOC_MAX_N, 128, "bf16", 500000.0, (504,)),
        (1, 32, 8, 2048, 128, "bf16", 500000.0, (501,)),
        (2, 4, 2, 300, 64, "fp16", 10000.0, (502,)),
    ]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    prepared = []
    for B, Hq, Hkv, N, D, dt, base, key in cases:
        q, k, v = (t.to(DEV) for t in inputs.qkv(B, Hq, Hkv, N, D, dt, key=key))
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
        ref_o, ref_l = rac.attn_rope_causal_fwd(q, k, v, base)
        prepared.append((q, k, v, out, lse, base, ref_o, ref_l))
    torch.cuda.synchronize()
    # the two calls back to back on one stream, outputs preallocated above
    for q, k, v, out, lse, base, _, _ in prepared:
        assert _noalloc(q, k, v, out, lse, base, stream) == rac.RAC_OK, rac.last_error()
    torch.cuda.synchronize()
    for (q, k, v, out, lse, base, ref_o, ref_l), case in zip(prepared, cases):
        what = "noalloc B%d Hq%d Hkv%d N%d D%d %s" % case[:6]
        mx, rel = assert_o(to_f64(out), to_f64(ref_o), what)
        lerr = assert_lse(to_f64(lse), to_f64(ref_l), what)
        same = bool(torch.equal(out, ref_o) and torch.equal(lse, ref_l))
        print("%s: max|dO|=%.3e relL2=%.3e max|dLSE|=%.3e bit-identical=%s" %
              (what, mx, rel, lerr, same))


def test_noalloc_rejects_lengths_beyond_its_table():
    """N * D above the static table's capacity is an argument error, found
    before anything is enqueued (the pointers are never used)."""
    p = ctypes.c_void_p(1 << 20)
    args = lambda N, D: (p, ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20),  # noqa: E731
                         ctypes.c_void_p(4 << 20), None, 1, 1, 1, N, D, 1e4, 0, None)
    L = rac.lib()
    assert L.attn_rope_causal_fwd_noalloc(*args(rac.RAC_NOALLOC_MAX_N + 1, 128)) == rac.RAC_ERR_ARG
    assert "static table" in rac.last_error()
    assert L.attn_rope_causal_fwd_noalloc(*args(2 * rac.RAC_NOALLOC_MAX_N + 1, 64)) == rac.RAC_ERR_ARG
