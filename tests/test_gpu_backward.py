"""GPU parity of the backward: the HIP kernels, called through the C ABI,
against the fp64 oracle's gradients on the same seeded inputs.

Cases: the fused backward (attn_rope_causal_bwd) and the pre-rotation path's
backward (rope_prerotate, attn_causal_bwd, rope_prerotate_bwd), with adjacent
and with half-split RoPE pairs (the _ex entry points), on small shapes
spanning several tiles with ragged tails, GQA ratios 1-8, D = 64 and 128,
bf16 and fp16; the inverse rotation pass on its own; determinism; and one key/
value group of the Llama-3-8B-shaped layer at full length (N = 2048 and 8192)
in the launch configuration the bench times. The small cases run under every
key-parallel workgroup shape (RAC_BWD_SHAPE). Bounds: parity.assert_grad.
"""
import numpy as np
import pytest
import torch

import oracle
import rotary_position_embedding_causal_amd as rac
from rotary_position_embedding_causal_amd import inputs
from parity import assert_grad, assert_o, bits, to_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rac.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(params=["auto", "k128", "k64", "k64x2", "k64x2h", "dqtile"])
def bwd_shape(request, monkeypatch):
    """Runs a test under each key-parallel workgroup shape (RAC_BWD_SHAPE),
    and once with the dQ pass's one-tile-per-workgroup launch (RAC_BWD_DQ;
    small problems otherwise take its paired launch)."""
    if request.param == "dqtile":
        monkeypatch.setenv("RAC_BWD_DQ", "tile")
    else:
        monkeypatch.setenv("RAC_BWD_SHAPE", request.param)
    return request.param


SHAPES = [  # B, Hq, Hkv, N, D, dtype, base
    (1, 4, 4, 512, 64, "bf16", 10000.0),
    (1, 8, 2, 300, 128, "bf16", 500000.0),
    (2, 4, 1, 129, 64, "fp16", 10000.0),
    (1, 8, 1, 65, 128, "fp16", 500000.0),
    (1, 2, 2, 1, 64, "bf16", 10000.0),
    (1, 6, 3, 17, 128, "bf16", 10000.0),
    (1, 4, 2, 1000, 128, "bf16", 500000.0),
]


def _id(s):
    return "B%d_Hq%d_Hkv%d_N%d_D%d_%s" % s[:6]


def _case(B, Hq, Hkv, N, D, dt, base, key):
    q, k, v = inputs.qkv(B, Hq, Hkv, N, D, dt, key=key)
    do = inputs.draw((B, Hq, N, D), dt, key, 3)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = rac.attn_rope_causal_fwd(qd, kd, vd, base)
    return (q, k, v, do), (qd, kd, vd, dod, o, lse)


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
@pytest.mark.parametrize("path", ["fused", "prerotate"])
def test_backward_matches_oracle(shape, path, bwd_shape):
    B, Hq, Hkv, N, D, dt, base = shape
    print("backward %s %s %s" % (path, _id(shape), bwd_shape), flush=True)
    (q, k, v, do), (qd, kd, vd, dod, o, lse) = _case(B, Hq, Hkv, N, D, dt, base, (401, N, D))
    fn = rac.attn_rope_causal_bwd if path == "fused" else rac.prerotate_path_bwd
    dq, dk, dv, delta = fn(qd, kd, vd, o, lse, dod, base)
    torch.cuda.synchronize()
    for variant in ("rounded", "exact"):
        rdq, rdk, rdv, rdelta, _ = oracle.rope_attention_bwd(
            inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), dt, base, variant)
        for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            assert_grad(to_f64(got), ref, "%s %s vs %s oracle" % (path, name, variant))
        assert_grad(delta.cpu().double().numpy(), rdelta, "%s delta" % path)


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_fused_backward_rotation_once_or_per_tile_agree(shape, bwd_shape, monkeypatch):
    """The fused backward rotates q and k once through the streaming pass
    (default) or inside its kernels at every tile visit (RAC_BWD_ROT=kernel):
    the same rotated operands reach the same arithmetic, so every output is
    bit for bit the same."""
    B, Hq, Hkv, N, D, dt, base = shape
    _, (qd, kd, vd, dod, o, lse) = _case(B, Hq, Hkv, N, D, dt, base, (403, N, D))
    once = rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base)
    monkeypatch.setenv("RAC_BWD_ROT", "kernel")
    per_tile = rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base)
    torch.cuda.synchronize()
    for a, b, name in zip(once, per_tile, ("dq", "dk", "dv", "delta")):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("shape", SHAPES[:4], ids=_id)
def test_paths_agree_and_are_deterministic(shape, bwd_shape):
    B, Hq, Hkv, N, D, dt, base = shape
    _, (qd, kd, vd, dod, o, lse) = _case(B, Hq, Hkv, N, D, dt, base, (402, N, D))
    f1 = rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base)
    f2 = rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base)
    p = rac.prerotate_path_bwd(qd, kd, vd, o, lse, dod, base)
    torch.cuda.synchronize()
    for a, b in zip(f1, f2):
        assert torch.equal(a, b)  # one writer per element: no run-to-run variation
    # dv and delta see the same rotated operands on both paths; dq and dk
    # differ by the pre-rotation path's extra rounding of dq', dk'
    assert torch.equal(f1[2], p[2]) and torch.equal(f1[3], p[3])
    for a, b, name in ((f1[0], p[0], "dq"), (f1[1], p[1], "dk")):
        assert_grad(to_f64(b), to_f64(a), "prerotate vs fused " + name)


@pytest.mark.parametrize("shape", SHAPES[1:4], ids=_id)
def test_attn_causal_bwd_on_rotated_inputs(shape):
    B, Hq, Hkv, N, D, dt, base = shape
    (q, k, v, do), (qd, kd, vd, dod, _, _) = _case(B, Hq, Hkv, N, D, dt, base, (403, N, D))
    qr, kr = rac.rope_prerotate(qd, kd, base)
    o, lse = rac.attn_causal_fwd(qr, kr, vd)
    dq, dk, dv, delta = rac.attn_causal_bwd(qr, kr, vd, o, lse, dod)
    torch.cuda.synchronize()
    dec = lambda t: oracle.decode(bits(t), dt)  # noqa: E731
    rdq, rdk, rdv, _, rdelta = oracle.attention_bwd(dec(qr), dec(kr), dec(vd), dec(dod))
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert_grad(to_f64(got), ref, "attn_causal_bwd " + name)


@pytest.mark.parametrize("shape", [(1, 4, 2, 300, 128, "bf16", 500000.0),
                                   (2, 2, 2, 4096, 64, "fp16", 10000.0)], ids=_id)
def test_rope_prerotate_bwd_is_the_inverse_rotation(shape):
    B, Hq, Hkv, N, D, dt, base = shape
    gq = inputs.draw((B, Hq, N, D), dt, (404, N), 0)
    gk = inputs.draw((B, Hkv, N, D), dt, (404, N), 1)
    dq, dk = rac.rope_prerotate_bwd(gq.to(DEV), gk.to(DEV), base)
    g2 = gq.to(DEV).clone()
    rac.rope_prerotate_bwd(g2, gk.to(DEV), base, dq=g2, dk=torch.empty_like(gk, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(g2, dq)  # in place
    neg = -np.arange(N)
    for src, got in ((gq, dq), (gk, dk)):
        y = oracle.rope(oracle.decode(inputs.bits(src), dt), neg, base)
        ref = oracle.encode(y, dt)
        g = bits(got)
        exact = float(np.mean(g == ref))
        assert exact >= 0.999, "bit-exact fraction %.5f" % exact
        x = oracle.decode(inputs.bits(src), dt)
        pair = np.repeat(np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]), 2, axis=-1)
        gv = oracle.decode(g, dt)
        spacing = np.spacing(np.abs(gv).astype(np.float16 if dt == "fp16" else np.float32))
        ulp = spacing.astype(np.float64) * (65536.0 if dt == "bf16" else 1.0)
        assert np.all(np.abs(gv - y) <= ulp + 8 * 2.0 ** -24 * pair)


@pytest.mark.parametrize("N", [2, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("ratio", [1, 4, 8])
def test_ragged_lengths_and_gqa(N, ratio, bwd_shape):
    B, Hkv, D, dt, base = 1, 1, 128, "bf16", 10000.0
    Hq = Hkv * ratio
    (q, k, v, do), (qd, kd, vd, dod, o, lse) = _case(B, Hq, Hkv, N, D, dt, base, (405, N, ratio))
    dq, dk, dv, delta = rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base)
    torch.cuda.synchronize()
    rdq, rdk, rdv, rdelta, _ = oracle.rope_attention_bwd(
        inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), dt, base, "rounded")
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert_grad(to_f64(got), ref, "N=%d ratio=%d %s" % (N, ratio, name))


@pytest.mark.parametrize("name,key", [("llama3_8b_gqa_n2048", 406), ("llama3_8b_gqa_n8192", 407),
                                      ("gqa8_d128_bf16_n2048", 408), ("mha_d64_fp16_n8192", 409)])
def test_full_length_one_group(name, key):
    """The Llama-3-8B-shaped layer at N = 2048 and 8192 in the bench's launch
    configuration, a GQA 8:1 layer (two workgroups per key tile, paired dQ
    launch) and a D = 64 fp16 MHA layer at N = 8192; the oracle checks one
    key/value group (its query heads and their key/value head) in full,
    which the other groups do not influence (about 15 s of oracle time at
    N = 8192 on 16 cores)."""
    w = inputs.WORKLOADS[name]
    B, Hq, Hkv, N, D, dt, base = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["dtype"], w["base"]
    q, k, v = inputs.workload_qkv(name)
    do = inputs.draw((B, Hq, N, D), dt, (key,), 3)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = rac.attn_rope_causal_fwd(qd, kd, vd, base)
    dq, dk, dv, _ = rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base)
    torch.cuda.synchronize()
    group = Hq // Hkv
    g = 5
    hs = slice(g * group, (g + 1) * group)
    rdq, rdk, rdv, _, _ = oracle.rope_attention_bwd(
        inputs.bits(q)[:, hs], inputs.bits(k)[:, g:g + 1], inputs.bits(v)[:, g:g + 1],
        inputs.bits(do)[:, hs], dt, base, "rounded")
    assert_grad(to_f64(dq[:, hs]), rdq, "%s dq" % name)
    assert_grad(to_f64(dk[:, g:g + 1]), rdk, "%s dk" % name)
    assert_grad(to_f64(dv[:, g:g + 1]), rdv, "%s dv" % name)


# ---- the half-split pairing (i, i + D/2) ----------------------------------

def _case_half(B, Hq, Hkv, N, D, dt, base, key):
    q, k, v = inputs.qkv(B, Hq, Hkv, N, D, dt, key=key)
    do = inputs.draw((B, Hq, N, D), dt, key, 3)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    return (q, k, v, do), (qd, kd, vd, dod, o, lse)


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
@pytest.mark.parametrize("path", ["fused", "prerotate"])
def test_half_split_backward_matches_oracle(shape, path):
    """The gradients through the half-split pairing's RoPE against the
    oracle's (its inverse turn of pairs (i, i + D/2)), both oracle variants."""
    B, Hq, Hkv, N, D, dt, base = shape
    print("half-split backward %s %s" % (path, _id(shape)), flush=True)
    (q, k, v, do), (qd, kd, vd, dod, o, lse) = _case_half(B, Hq, Hkv, N, D, dt, base,
                                                          (411, N, D))
    if path == "fused":
        dq, dk, dv, delta = rac.attn_rope_causal_bwd_ex(qd, kd, vd, o, lse, dod, base, "half")
    else:
        dq, dk, dv, delta = rac.prerotate_path_bwd(qd, kd, vd, o, lse, dod, base, "half")
    torch.cuda.synchronize()
    for variant in ("rounded", "exact"):
        rdq, rdk, rdv, rdelta, _ = oracle.rope_attention_bwd(
            inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), dt, base, variant,
            "half")
        for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            assert_grad(to_f64(got), ref, "half %s %s vs %s oracle" % (path, name, variant))
        assert_grad(delta.cpu().double().numpy(), rdelta, "half %s delta" % path)


@pytest.mark.parametrize("shape", SHAPES[:4] + SHAPES[6:], ids=_id)
def test_half_split_backward_paths_agree_bit_for_bit(shape, bwd_shape):
    """The fused half-split backward is the pre-rotation path's three calls
    (the same passes and kernels in the same order), so every output is
    bit for bit the same, and it is deterministic; under every key-parallel
    workgroup shape."""
    B, Hq, Hkv, N, D, dt, base = shape
    _, (qd, kd, vd, dod, o, lse) = _case_half(B, Hq, Hkv, N, D, dt, base, (412, N, D))
    f1 = rac.attn_rope_causal_bwd_ex(qd, kd, vd, o, lse, dod, base, "half")
    f2 = rac.attn_rope_causal_bwd_ex(qd, kd, vd, o, lse, dod, base, "half")
    p = rac.prerotate_path_bwd(qd, kd, vd, o, lse, dod, base, "half")
    a = rac.attn_rope_causal_bwd_ex(qd, kd, vd, o, lse, dod, base, "adjacent")
    b = rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base)
    torch.cuda.synchronize()
    for x, y, z, name in zip(f1, f2, p, ("dq", "dk", "dv", "delta")):
        assert torch.equal(x, y) and torch.equal(x, z), name
    for x, y in zip(a, b):  # the _ex entry with adjacent pairs is the plain one
        assert torch.equal(x, y)


@pytest.mark.parametrize("shape", [(1, 4, 2, 300, 128, "bf16", 500000.0),
                                   (2, 2, 2, 4096, 64, "fp16", 10000.0)], ids=_id)
def test_rope_prerotate_bwd_ex_half_is_the_inverse_rotation(shape):
    B, Hq, Hkv, N, D, dt, base = shape
    gq = inputs.draw((B, Hq, N, D), dt, (413, N), 0)
    gk = inputs.draw((B, Hkv, N, D), dt, (413, N), 1)
    dq, dk = rac.rope_prerotate_bwd_ex(gq.to(DEV), gk.to(DEV), base, "half")
    g2 = gq.to(DEV).clone()
    rac.rope_prerotate_bwd_ex(g2, gk.to(DEV), base, "half", dq=g2,
                              dk=torch.empty_like(gk, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(g2, dq)  # in place
    neg = -np.arange(N)
    for src, got in ((gq, dq), (gk, dk)):
        y = oracle.rope(oracle.decode(inputs.bits(src), dt), neg, base, "half")
        ref = oracle.encode(y, dt)
        g = bits(got)
        exact = float(np.mean(g == ref))
        assert exact >= 0.999, "bit-exact fraction %.5f" % exact
        x = oracle.decode(inputs.bits(src), dt)
        h = D // 2
        pair = np.abs(x[..., :h]) + np.abs(x[..., h:])
        pair = np.concatenate([pair, pair], axis=-1)
        gv = oracle.decode(g, dt)
        spacing = np.spacing(np.abs(gv).astype(np.float16 if dt == "fp16" else np.float32))
        ulp = spacing.astype(np.float64) * (65536.0 if dt == "bf16" else 1.0)
        assert np.all(np.abs(gv - y) <= ulp + 8 * 2.0 ** -24 * pair)


def test_half_split_backward_full_length_one_group():
    """The Llama-3-8B-shaped layer at N = 2048 with the half-split pairing
    (the layout its checkpoints use), one key/value group against the
    oracle, as test_full_length_one_group."""
    name, key = "llama3_8b_gqa_n2048", 414
    w = inputs.WORKLOADS[name]
    B, Hq, Hkv, N, D, dt, base = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["dtype"], w["base"]
    q, k, v = inputs.workload_qkv(name)
    do = inputs.draw((B, Hq, N, D), dt, (key,), 3)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = rac.attn_rope_causal_fwd_ex(qd, kd, vd, base, "half")
    dq, dk, dv, _ = rac.attn_rope_causal_bwd_ex(qd, kd, vd, o, lse, dod, base, "half")
    torch.cuda.synchronize()
    group = Hq // Hkv
    g = 3
    hs = slice(g * group, (g + 1) * group)
    rdq, rdk, rdv, _, _ = oracle.rope_attention_bwd(
        inputs.bits(q)[:, hs], inputs.bits(k)[:, g:g + 1], inputs.bits(v)[:, g:g + 1],
        inputs.bits(do)[:, hs], dt, base, "rounded", "half")
    assert_grad(to_f64(dq[:, hs]), rdq, "%s half dq" % name)
    assert_grad(to_f64(dk[:, g:g + 1]), rdk, "%s half dk" % name)
    assert_grad(to_f64(dv[:, g:g + 1]), rdv, "%s half dv" % name)


def test_largest_batch_short_sequences():
    """B = 65535 (the largest batch accepted), GQA 2:1, N = 3: the dQ pass's
    131070 and the dK/dV pass's 65535 work units, both paths against the
    oracle's gradients."""
    B, Hq, Hkv, N, D, dt, base = 65535, 2, 1, 3, 64, "bf16", 10000.0
    (q, k, v, do), (qd, kd, vd, dod, o, lse) = _case(B, Hq, Hkv, N, D, dt, base, (402,))
    res = {"fused": rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base),
           "prerotate": rac.prerotate_path_bwd(qd, kd, vd, o, lse, dod, base)}
    torch.cuda.synchronize()
    rdq, rdk, rdv, rdelta, _ = oracle.rope_attention_bwd(
        inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), dt, base, "rounded")
    for path, (dq, dk, dv, delta) in res.items():
        for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            assert_grad(to_f64(got), ref, "%s %s at B = 65535" % (path, name))
        assert_grad(delta.cpu().double().numpy(), rdelta, "%s delta at B = 65535" % path)


def test_most_query_heads_in_one_group():
    """Hq = 65535 (the most query heads accepted) sharing one key/value head,
    N = 3: a GQA group of 65535 heads, odd, so neither pass splits it; the
    dK/dV pass walks all of them for its one key tile. The forward's O and
    both backwards against the oracle."""
    B, Hq, Hkv, N, D, dt, base = 1, 65535, 1, 3, 64, "bf16", 10000.0
    (q, k, v, do), (qd, kd, vd, dod, o, lse) = _case(B, Hq, Hkv, N, D, dt, base, (403,))
    res = {"fused": rac.attn_rope_causal_bwd(qd, kd, vd, o, lse, dod, base),
           "prerotate": rac.prerotate_path_bwd(qd, kd, vd, o, lse, dod, base)}
    torch.cuda.synchronize()
    qb, kb, vb = inputs.bits(q), inputs.bits(k), inputs.bits(v)
    ro, _, _, _ = oracle.rope_attention(qb, kb, vb, dt, base, variant="rounded")
    assert_o(to_f64(o), ro, "forward with Hq = 65535")
    rdq, rdk, rdv, rdelta, _ = oracle.rope_attention_bwd(qb, kb, vb, inputs.bits(do), dt, base,
                                                         "rounded")
    for path, (dq, dk, dv, delta) in res.items():
        for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            assert_grad(to_f64(got), ref, "%s %s with Hq = 65535" % (path, name))
        assert_grad(delta.cpu().double().numpy(), rdelta, "%s delta with Hq = 65535" % path)


def test_empty_inputs():
    for shape in ((0, 2, 8, 64), (1, 2, 0, 64)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        l = torch.empty(shape[:3], dtype=torch.float32, device=DEV)
        dq, dk, dv, delta = rac.attn_rope_causal_bwd(x, x, x, x, l, x, 10000.0)
        dq2, dk2, dv2, _ = rac.attn_causal_bwd(x, x, x, x, l, x)
        a, b = rac.rope_prerotate_bwd(x, x, 10000.0)
        dq3, _, _, _ = rac.attn_rope_causal_bwd_ex(x, x, x, x, l, x, 10000.0, "half")
        c, _ = rac.rope_prerotate_bwd_ex(x, x, 10000.0, "half")
        assert dq.shape == shape and dv2.shape == shape and a.shape == shape
        assert dq3.shape == shape and c.shape == shape
