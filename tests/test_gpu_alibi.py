"""GPU parity of causal attention with the ALiBi distance penalty (scores
q_i . k_j / sqrt(D) - slopes[h] * (i - j)), alone and composed with RoPE of
either pairing, against the fp64 oracle's ALiBi attention; and the contract
that zero slopes reproduce the penalty-free entry points bit for bit. The
same for the backward (attn_alibi_causal_bwd) against the oracle's ALiBi
gradients.
"""
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_causal_amd as rac
from rotary_position_embedding_causal_amd import inputs
from parity import assert_grad, assert_lse, assert_o, oracle_rows, sampled_rows, to_f64

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


def geometric_slopes(H):
    """The ALiBi method's slope sequence 2^(-8(h+1)/H), as fp32 values."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def _run(qd, kd, vd, slopes, base, pairing):
    sd = torch.from_numpy(slopes).to(DEV)
    if pairing == "none":
        return rac.attn_alibi_causal_fwd(qd, kd, vd, sd)
    return rac.attn_alibi_causal_fwd(qd, kd, vd, sd, rope_base=base, pairing=pairing)


def _oracle(q, k, v, dt, base, pairing, slopes, variant="rounded", rows=None):
    return oracle.rope_attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), dt,
                                 None if pairing == "none" else base, rows=rows, variant=variant,
                                 pairing="adjacent" if pairing == "none" else pairing,
                                 slopes=slopes.astype(np.float64))


@pytest.mark.parametrize("shape", SMALL, ids=_id)
@pytest.mark.parametrize("pairing", ["none", "adjacent", "half"])
def test_alibi_matches_oracle(shape, pairing, launch_shape):
    B, Hq, Hkv, N, D, dt, base = shape
    q, k, v = inputs.qkv(B, Hq, Hkv, N, D, dt, key=(401, N, D))
    slopes = geometric_slopes(Hq)
    o, l = _run(q.to(DEV), k.to(DEV), v.to(DEV), slopes, base, pairing)
    torch.cuda.synchronize()
    ro, rl, _, _ = _oracle(q, k, v, dt, base, pairing, slopes)
    og, lg = to_f64(o), to_f64(l)
    assert_o(og, ro, "alibi %s" % pairing)
    assert_lse(lg, rl, "alibi %s LSE" % pairing)
    if pairing != "none":
        eo, _, _, _ = _oracle(q, k, v, dt, base, pairing, slopes, variant="exact")
        assert_o(og, eo, "alibi %s vs exact rotation" % pairing)


@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_zero_slopes_reproduce_penalty_free_kernels(shape, launch_shape):
    B, Hq, Hkv, N, D, dt, base = shape
    qd, kd, vd = [t.to(DEV) for t in inputs.qkv(B, Hq, Hkv, N, D, dt, key=(402, N, D))]
    zero = np.zeros(Hq, dtype=np.float32)
    o0, l0 = _run(qd, kd, vd, zero, base, "none")
    o1, l1 = _run(qd, kd, vd, zero, base, "adjacent")
    o2, l2 = _run(qd, kd, vd, zero, base, "half")
    p0, m0 = rac.attn_causal_fwd(qd, kd, vd)
    p1, m1 = rac.attn_rope_causal_fwd(qd, kd, vd, base)
    p2, m2 = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    torch.cuda.synchronize()
    assert torch.equal(o0, p0) and torch.equal(l0, m0)
    assert torch.equal(o1, p1) and torch.equal(l1, m1)
    assert torch.equal(o2, p2) and torch.equal(l2, m2)


@pytest.mark.parametrize("scale", [0.0, 0.05, 1.0, 8.0])
def test_alibi_slope_range(scale, launch_shape):
    """From no penalty to one that leaves only the diagonal (out_i ~ v_i),
    with distinct slopes per query head of a GQA group."""
    B, Hq, Hkv, N, D, dt = 1, 8, 2, 200, 128, "bf16"
    q, k, v = inputs.qkv(B, Hq, Hkv, N, D, dt, key=(403, int(scale * 100)))
    slopes = (scale * np.linspace(0.25, 1.0, Hq)).astype(np.float32)
    o, l = _run(q.to(DEV), k.to(DEV), v.to(DEV), slopes, None, "none")
    torch.cuda.synchronize()
    ro, rl, _, _ = _oracle(q, k, v, dt, None, "none", slopes)
    assert_o(to_f64(o), ro, "alibi scale %g" % scale)
    assert_lse(to_f64(l), rl, "alibi scale %g LSE" % scale)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("D,dt,ratio", [(64, "bf16", 1), (128, "fp16", 4), (128, "bf16", 8)])
def test_alibi_ragged_lengths_and_gqa(N, D, dt, ratio, launch_shape):
    Hkv = 2
    Hq = Hkv * ratio
    q, k, v = inputs.qkv(1, Hq, Hkv, N, D, dt, key=(404, N, D, ratio))
    slopes = geometric_slopes(Hq)
    o, l = _run(q.to(DEV), k.to(DEV), v.to(DEV), slopes, 10000.0, "adjacent")
    torch.cuda.synchronize()
    ro, rl, _, _ = _oracle(q, k, v, dt, 10000.0, "adjacent", slopes)
    assert_o(to_f64(o), ro, "ragged alibi")
    assert_lse(to_f64(l), rl, "ragged alibi LSE")


def test_alibi_full_size_sampled_rows():
    """The Llama-3-8B-shaped layer (32 query / 8 key heads, D = 128, N = 2048,
    bf16) with ALiBi and adjacent-pair RoPE, on sampled rows."""
    name = "llama3_8b_gqa_n2048"
    w = inputs.WORKLOADS[name]
    B, Hq, Hkv, N, D, dt, base = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["dtype"], w["base"]
    print("full-size ALiBi case %s" % name, flush=True)
    q, k, v = inputs.workload_qkv(name)
    slopes = geometric_slopes(Hq)
    o, l = _run(q.to(DEV), k.to(DEV), v.to(DEV), slopes, base, "adjacent")
    torch.cuda.synchronize()
    rows = sampled_rows(B, Hq, N, np.random.default_rng(11), per_head=12)
    flat = np.concatenate([(b * Hq + h) * N + r for (b, h), r in rows.items()])
    ro, rl, _, _ = _oracle(q, k, v, dt, base, "adjacent", slopes, rows=flat)
    og, lg = to_f64(o), to_f64(l)
    got = np.concatenate([og[b, h, r] for (b, h), r in rows.items()])
    gl = np.concatenate([lg[b, h, r] for (b, h), r in rows.items()])
    assert_o(got, ro, name + " alibi")
    assert_lse(gl, rl, name + " alibi LSE")


def test_alibi_largest_batch_short_sequences():
    """B = 65535 (the largest batch accepted), GQA 2:1, N = 3, D = 128: ALiBi
    alone (O and LSE against the oracle) and after RoPE of either pairing (O
    against the oracle; a one-key row's LSE would carry a rotated operand's
    rounding unaveraged), and the backward without RoPE against the
    oracle's gradients."""
    B, Hq, Hkv, N, D, dt, base = 65535, 2, 1, 3, 128, "bf16", 10000.0
    q, k, v = inputs.qkv(B, Hq, Hkv, N, D, dt, key=(430,))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    slopes = geometric_slopes(Hq)
    for pairing in ("none", "adjacent", "half"):
        o, l = _run(qd, kd, vd, slopes, base, pairing)
        torch.cuda.synchronize()
        ro, rl, _, _ = _oracle(q, k, v, dt, base, pairing, slopes)
        assert_o(to_f64(o), ro, "alibi %s at B = 65535" % pairing)
        if pairing == "none":
            assert_lse(to_f64(l), rl, "alibi LSE at B = 65535")
    o, l = _run(qd, kd, vd, slopes, base, "none")
    do = inputs.draw((B, Hq, N, D), dt, (430,), 3)
    dq, dk, dv, _ = rac.attn_alibi_causal_bwd(qd, kd, vd, o, l, do.to(DEV),
                                              torch.from_numpy(slopes).to(DEV))
    torch.cuda.synchronize()
    rdq, rdk, rdv, _, _ = oracle.rope_attention_bwd(
        inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), dt, None,
        slopes=slopes.astype(np.float64))
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert_grad(to_f64(got), ref, "alibi %s at B = 65535" % name)


def test_alibi_empty_inputs():
    for shape in ((1, 4, 0, 64), (0, 4, 16, 64)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        sl = torch.zeros(4, dtype=torch.float32, device=DEV)
        o, l = rac.attn_alibi_causal_fwd(x, x, x, sl, rope_base=10000.0)
        assert o.shape == shape and l.shape == shape[:3]


# ---- the backward ------------------------------------------------------------

@pytest.fixture(params=["auto", "k128", "k64x2", "k64x2h"])
def bwd_shape(request, monkeypatch):
    monkeypatch.setenv("RAC_BWD_SHAPE", request.param)
    return request.param


def _bwd_case(B, Hq, Hkv, N, D, dt, base, pairing, slopes, key):
    q, k, v = inputs.qkv(B, Hq, Hkv, N, D, dt, key=key)
    do = inputs.draw((B, Hq, N, D), dt, key, 3)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    sd = torch.from_numpy(slopes).to(DEV)
    o, lse = _run(qd, kd, vd, slopes, base, pairing)
    rb = None if pairing == "none" else base
    grads = rac.attn_alibi_causal_bwd(qd, kd, vd, o, lse, dod, sd, rope_base=rb,
                                      pairing="adjacent" if pairing == "none" else pairing)
    return (q, k, v, do), (qd, kd, vd, dod, o, lse, sd), grads


@pytest.mark.parametrize("shape", SMALL, ids=_id)
@pytest.mark.parametrize("pairing", ["none", "adjacent", "half"])
def test_alibi_backward_matches_oracle(shape, pairing):
    """The gradients with the ALiBi penalty (alone or after RoPE of either
    pairing) against the oracle's ALiBi backward, both oracle variants."""
    from parity import assert_grad
    B, Hq, Hkv, N, D, dt, base = shape
    print("alibi backward %s %s" % (pairing, _id(shape)), flush=True)
    slopes = geometric_slopes(Hq)
    (q, k, v, do), _, (dq, dk, dv, delta) = _bwd_case(B, Hq, Hkv, N, D, dt, base, pairing,
                                                      slopes, (405, N, D))
    torch.cuda.synchronize()
    for variant in (("rounded", "exact") if pairing != "none" else ("rounded",)):
        rdq, rdk, rdv, rdelta, _ = oracle.rope_attention_bwd(
            inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), dt,
            None if pairing == "none" else base, variant,
            "adjacent" if pairing == "none" else pairing, slopes.astype(np.float64))
        for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            assert_grad(to_f64(got), ref, "alibi %s %s vs %s oracle" % (pairing, name, variant))
        assert_grad(delta.cpu().double().numpy(), rdelta, "alibi %s delta" % pairing)


@pytest.mark.parametrize("shape", SMALL[:4], ids=_id)
def test_alibi_backward_zero_slopes_and_shapes(shape, bwd_shape):
    """Zero slopes give the penalty-free backward bit for bit (same operands,
    same arithmetic), under every key-parallel workgroup shape; and the
    ALiBi backward is deterministic."""
    B, Hq, Hkv, N, D, dt, base = shape
    zero = np.zeros(Hq, dtype=np.float32)
    for pairing in ("none", "adjacent", "half"):
        _, (qd, kd, vd, dod, o, lse, sd), g = _bwd_case(B, Hq, Hkv, N, D, dt, base, pairing,
                                                        zero, (406, N, D))
        if pairing == "none":
            ref = rac.attn_causal_bwd(qd, kd, vd, o, lse, dod)
        else:
            ref = rac.attn_rope_causal_bwd_ex(qd, kd, vd, o, lse, dod, base, pairing)
        torch.cuda.synchronize()
        for a, b, name in zip(g, ref, ("dq", "dk", "dv", "delta")):
            assert torch.equal(a, b), (pairing, name)
    slopes = geometric_slopes(Hq)
    _, (qd, kd, vd, dod, o, lse, sd), g1 = _bwd_case(B, Hq, Hkv, N, D, dt, base, "adjacent",
                                                     slopes, (407, N, D))
    g2 = rac.attn_alibi_causal_bwd(qd, kd, vd, o, lse, dod, sd, rope_base=base)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("N", [2, 65, 129])
@pytest.mark.parametrize("scale", [0.0, 1.0, 4.0, 8.0])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_alibi_backward_slopes_and_ragged(N, scale, dt):
    """From no penalty to one that leaves only the diagonal, distinct slopes
    per query head of a GQA 4:1 group, ragged lengths. Where the penalty is at
    least one unit of score per position (scale >= 4: slopes 1 .. 8) a bf16
    row's P is nearly one-hot, and dq, dk are held to the peaked-softmax
    bound (parity.G_RELL2_PEAKED; measured 1.1-1.3e-2 rel-L2, fp16 1.5e-3);
    dv, which has no dS, keeps the standard one."""
    from parity import G_RELL2, G_RELL2_PEAKED, assert_grad
    B, Hq, Hkv, D = 1, 8, 2, 128
    slopes = (scale * np.linspace(0.25, 1.0, Hq)).astype(np.float32)
    (q, k, v, do), _, (dq, dk, dv, _) = _bwd_case(B, Hq, Hkv, N, D, dt, None, "none", slopes,
                                                  (408, N, int(scale)))
    torch.cuda.synchronize()
    rdq, rdk, rdv, _, _ = oracle.rope_attention_bwd(
        inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), dt, None, "rounded",
        "adjacent", slopes.astype(np.float64))
    peaked = G_RELL2_PEAKED if (dt == "bf16" and scale >= 4.0) else G_RELL2
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        _, rel = assert_grad(to_f64(got), ref, "alibi N=%d scale=%g %s" % (N, scale, name),
                             peaked if name != "dv" else G_RELL2)
        print("alibi %s N=%d scale=%g %s rel-L2 %.2e" % (dt, N, scale, name, rel))


def test_alibi_backward_full_length_one_group():
    """The Llama-3-8B-shaped layer at N = 2048 with ALiBi after adjacent-pair
    RoPE, one key/value group in full against the oracle."""
    from parity import assert_grad
    name = "llama3_8b_gqa_n2048"
    w = inputs.WORKLOADS[name]
    B, Hq, Hkv, N, D, dt, base = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["dtype"], w["base"]
    q, k, v = inputs.workload_qkv(name)
    do = inputs.draw((B, Hq, N, D), dt, (409,), 3)
    slopes = geometric_slopes(Hq)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    sd = torch.from_numpy(slopes).to(DEV)
    o, lse = rac.attn_alibi_causal_fwd(qd, kd, vd, sd, rope_base=base)
    dq, dk, dv, _ = rac.attn_alibi_causal_bwd(qd, kd, vd, o, lse, dod, sd, rope_base=base)
    torch.cuda.synchronize()
    group = Hq // Hkv
    g = 2
    hs = slice(g * group, (g + 1) * group)
    rdq, rdk, rdv, _, _ = oracle.rope_attention_bwd(
        inputs.bits(q)[:, hs], inputs.bits(k)[:, g:g + 1], inputs.bits(v)[:, g:g + 1],
        inputs.bits(do)[:, hs], dt, base, "rounded", "adjacent",
        slopes[hs].astype(np.float64))
    assert_grad(to_f64(dq[:, hs]), rdq, "%s alibi dq" % name)
    assert_grad(to_f64(dk[:, g:g + 1]), rdk, "%s alibi dk" % name)
    assert_grad(to_f64(dv[:, g:g + 1]), rdv, "%s alibi dv" % name)


def test_alibi_backward_empty_inputs():
    for shape in ((1, 4, 0, 64), (0, 4, 16, 64)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        l = torch.empty(shape[:3], dtype=torch.float32, device=DEV)
        sl = torch.zeros(4, dtype=torch.float32, device=DEV)
        dq, dk, dv, delta = rac.attn_alibi_causal_bwd(x, x, x, x, l, x, sl, rope_base=10000.0)
        assert dq.shape == shape and delta.shape == shape[:3]
