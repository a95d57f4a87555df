"""GPU parity of the half-split RoPE pairing (coordinates i and i + D/2 turn
together) against the fp64 oracle's half-split rotation, and the contract of
the pairing entry points: pairing "adjacent" reproduces the plain entry points
bit for bit, and the fused kernel equals pre-rotation + plain attention bit for
bit under either pairing.
"""
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_causal_amd as rac
from rotary_position_embedding_causal_amd import inputs
from parity import (assert_grad, assert_lse, assert_o, bits, o_errors, oracle_rows, sampled_rows,
                    to_f64)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rac.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(params=["auto", "pair", "tile", "pairheads"])
def launch_shape(request, monkeypatch):
    monkeypatch.setenv("RAC_ATTN_SHAPE", request.param)
    return request.param


SMALL = [  # B, Hq, Hkv, N, D, dtype, base
    (1, 4, 4, 512, 64, "bf16", 10000.0),
    (1, 8, 2, 300, 128, "bf16", 500000.0),
    (2, 4, 1, 129, 64, "fp16", 10000.0),
    (1, 8, 1, 65, 128, "fp16", 500000.0),
    (1, 2, 2, 1, 64, "bf16", 10000.0),
    (1, 6, 3, 17, 128, "bf16", 10000.0),
]


def _id(s):
    return "B%d_Hq%d_Hkv%d_N%d_D%d_%s" % s[:6]


def _inputs(B, Hq, Hkv, N, D, dtype, key):
    q, k, v = inputs.qkv(B, Hq, Hkv, N, D, dtype, key=key)
    return (q, k, v), (q.to(DEV), k.to(DEV), v.to(DEV))


def _check_half_rotation(g, src_bits, N, dt, base):
    """Rotated bits vs the oracle's half-split rotation: >= 99.9 % bit-exact,
    and every element within one ulp or within the fp32 evaluation error of
    its pair, 8 * 2^-24 * (|x_i| + |x_(i+D/2)|)."""
    x = oracle.decode(src_bits, dt)
    y = oracle.rope(x, np.arange(N, dtype=np.int64), base, "half")
    ref = oracle.encode(y, dt)
    exact = float(np.mean(g == ref))
    assert exact >= 0.999, "bit-exact fraction %.5f" % exact
    gv = oracle.decode(g, dt)
    h = x.shape[-1] // 2
    pair = np.abs(x[..., :h]) + np.abs(x[..., h:])
    pair = np.concatenate([pair, pair], axis=-1)
    ulp = np.spacing(np.abs(gv).astype(np.float16 if dt == "fp16" else np.float32))
    ulp = ulp.astype(np.float64) * (65536.0 if dt == "bf16" else 1.0)
    bad = np.abs(gv - y) > ulp + 8 * 2.0 ** -24 * pair
    assert not bad.any(), "%d elements outside the fp32 rotation error model" % int(bad.sum())


@pytest.mark.parametrize("shape", SMALL + [(1, 16, 16, 4096, 64, "fp16", 10000.0),
                                          (2, 32, 8, 1000, 128, "bf16", 500000.0)], ids=_id)
def test_half_prerotate_matches_oracle(shape):
    B, Hq, Hkv, N, D, dt, base = shape
    (q, k, _), (qd, kd, _) = _inputs(B, Hq, Hkv, N, D, dt, key=(301, N, D))
    qr, kr = rac.rope_prerotate_ex(qd, kd, base, "half")
    torch.cuda.synchronize()
    for src, got in ((q, qr), (k, kr)):
        _check_half_rotation(bits(got), inputs.bits(src), N, dt, base)


def test_half_prerotate_in_place():
    _, (qd, kd, _) = _inputs(1, 4, 2, 257, 128, "bf16", key=(302,))
    qr, kr = rac.rope_prerotate_ex(qd, kd, 500000.0, "half")
    q2, k2 = qd.clone(), kd.clone()
    rac.rope_prerotate_ex(q2, k2, 500000.0, "half", q_rot=q2, k_rot=k2)
    torch.cuda.synchronize()
    assert torch.equal(q2, qr) and torch.equal(k2, kr)


@pytest.mark.parametrize("shape", SMALL, ids=_id)
@pytest.mark.parametrize("path", ["fused", "prerotate"])
def test_half_pairing_matches_oracle(shape, path, launch_shape):
    B, Hq, Hkv, N, D, dt, base = shape
    (q, k, v), (qd, kd, vd) = _inputs(B, Hq, Hkv, N, D, dt, key=(303, N, D))
    if path == "fused":
        o, l = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    else:
        o, l = rac.prerotate_path(qd, kd, vd, base, pairing="half")
    torch.cuda.synchronize()
    qb, kb, vb = inputs.bits(q), inputs.bits(k), inputs.bits(v)
    ro, rl, _, _ = oracle.rope_attention(qb, kb, vb, dt, base, variant="rounded",
                                         pairing="half")
    eo, el, _, _ = oracle.rope_attention(qb, kb, vb, dt, base, variant="exact", pairing="half")
    og, lg = to_f64(o), to_f64(l)
    assert_o(og, ro, path + " half vs rounded-rotation oracle")
    assert_o(og, eo, path + " half vs exact-rotation oracle")
    assert_lse(lg, rl, path + " half LSE")
    assert float(np.max(np.abs(lg - el))) < 2e-2
    if N >= 64:
        # the pairing matters: the adjacent-pair oracle is a different result
        ao, _, _, _ = oracle.rope_attention(qb, kb, vb, dt, base, variant="rounded")
        assert o_errors(og, ao)[0] > 10 * o_errors(og, ro)[0]


@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_half_fused_equals_prerotate_path(shape, launch_shape):
    B, Hq, Hkv, N, D, dt, base = shape
    _, (qd, kd, vd) = _inputs(B, Hq, Hkv, N, D, dt, key=(304, N, D))
    of, lf = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    op, lp = rac.prerotate_path(qd, kd, vd, base, pairing="half")
    torch.cuda.synchronize()
    assert torch.equal(of, op) and torch.equal(lf, lp)


@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_adjacent_pairing_reproduces_plain_entry_points(shape):
    B, Hq, Hkv, N, D, dt, base = shape
    _, (qd, kd, vd) = _inputs(B, Hq, Hkv, N, D, dt, key=(305, N, D))
    of, lf = rac.attn_rope_causal_fwd(qd, kd, vd, base)
    ox, lx = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "adjacent")
    qr, kr = rac.rope_prerotate(qd, kd, base)
    qx, kx = rac.rope_prerotate_ex(qd, kd, base, rac.RAC_PAIR_ADJACENT)
    torch.cuda.synchronize()
    assert torch.equal(of, ox) and torch.equal(lf, lx)
    assert torch.equal(qr, qx) and torch.equal(kr, kx)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("D,dt,ratio", [(64, "bf16", 1), (128, "fp16", 4), (128, "bf16", 8)])
def test_half_ragged_lengths_and_gqa(N, D, dt, ratio, launch_shape):
    Hkv = 2
    Hq = Hkv * ratio
    (q, k, v), (qd, kd, vd) = _inputs(1, Hq, Hkv, N, D, dt, key=(306, N, D, ratio))
    o, l = rac.attn_rope_causal_fwd_ex(qd, kd, vd, 10000.0, "half")
    torch.cuda.synchronize()
    ro, rl, _, _ = oracle.rope_attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), dt,
                                         10000.0, variant="rounded", pairing="half")
    assert_o(to_f64(o), ro, "ragged half")
    assert_lse(to_f64(l), rl, "ragged half")


def test_half_full_size_sampled_rows():
    """The Llama-3-8B-shaped layer (32 query / 8 key heads, D = 128, N = 2048,
    bf16) under the half-split pairing, on sampled rows."""
    name = "llama3_8b_gqa_n2048"
    w = inputs.WORKLOADS[name]
    B, Hq, Hkv, N, D, dt, base = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["dtype"], w["base"]
    print("full-size half-split case %s" % name, flush=True)
    q, k, v = inputs.workload_qkv(name)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    of, lf = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    op, lp = rac.prerotate_path(qd, kd, vd, base, pairing="half")
    torch.cuda.synchronize()
    assert torch.equal(of, op) and torch.equal(lf, lp)
    rows = sampled_rows(B, Hq, N, np.random.default_rng(7), per_head=12)
    qb, kb, vb = inputs.bits(q), inputs.bits(k), inputs.bits(v)
    ref = oracle_rows(qb, kb, vb, dt, base, Hq, Hkv, rows, "rounded", pairing="half")
    og, lg = to_f64(of), to_f64(lf)
    got = np.concatenate([og[b, h, r] for (b, h), r in rows.items()])
    gl = np.concatenate([lg[b, h, r] for (b, h), r in rows.items()])
    assert_o(got, np.concatenate([ref[bh][0] for bh in rows]), name + " half")
    assert_lse(gl, np.concatenate([ref[bh][1] for bh in rows]), name + " half LSE")


def test_half_largest_batch_short_sequences():
    """B = 65535 (the largest batch accepted), GQA 2:1, N = 3, D = 128, fp16:
    the half-split fused kernel and pre-rotation path give the same bits and
    O matches the oracle; the backward of both paths against the oracle's
    gradients."""
    B, Hq, Hkv, N, D, dt, base = 65535, 2, 1, 3, 128, "fp16", 10000.0
    (q, k, v), (qd, kd, vd) = _inputs(B, Hq, Hkv, N, D, dt, key=(330,))
    of, lf = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    op, lp = rac.prerotate_path(qd, kd, vd, base, pairing="half")
    torch.cuda.synchronize()
    assert torch.equal(of, op) and torch.equal(lf, lp)
    qb, kb, vb = inputs.bits(q), inputs.bits(k), inputs.bits(v)
    ro, _, _, _ = oracle.rope_attention(qb, kb, vb, dt, base, variant="rounded", pairing="half")
    assert_o(to_f64(of), ro, "half at B = 65535")
    do = inputs.draw((B, Hq, N, D), dt, (330,), 3)
    dod = do.to(DEV)
    res = {"fused": rac.attn_rope_causal_bwd_ex(qd, kd, vd, of, lf, dod, base, "half"),
           "prerotate": rac.prerotate_path_bwd(qd, kd, vd, of, lf, dod, base, "half")}
    torch.cuda.synchronize()
    rdq, rdk, rdv, _, _ = oracle.rope_attention_bwd(qb, kb, vb, inputs.bits(do), dt, base,
                                                    "rounded", pairing="half")
    for path, (dq, dk, dv, _) in res.items():
        for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            assert_grad(to_f64(got), ref, "half %s %s at B = 65535" % (path, name))


def test_half_empty_inputs():
    for shape in ((1, 4, 0, 64), (0, 4, 16, 64)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        o, l = rac.attn_rope_causal_fwd_ex(x, x, x, 10000.0, "half")
        qr, kr = rac.rope_prerotate_ex(x, x, 10000.0, "half")
        assert o.shape == shape and l.shape == shape[:3] and qr.shape == shape
