"""Pins for the fp64 oracle: checks against what the definition and the
mathematics fix, never against the oracle itself.

Each pin is a function of an ``oracle.Oracle`` instance that raises
AssertionError when the oracle is wrong. ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on oracle builds with a
planted mistake and requires that some pin fails for every mistake.

The pages print no worked numeric example (no tensor, output or LSE value),
so the pins are: bit-level agreement of the storage-format routines with
torch/numpy, RoPE invariants (position 0 is the identity, pair norms are
kept, dot products depend only on the position difference, rotations
compose), an independent complex-number form of RoPE, a D = 2 closed form,
explicit N x N brute force and torch's fp64 scaled_dot_product_attention for
attention, and special cases with closed forms (row 0 returns v_0, zero
queries average the visible values, softmax rows sum to one).
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch

RNG_SEED = 1234


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([RNG_SEED, *key]))


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def pin_decode_bf16_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_decode_fp16_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _wide_fp32_sample(rng, n):
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-140, 128, n)
    sign = rng.choice([-1.0, 1.0], n)
    x = (sign * np.ldexp(mant, expo)).astype(np.float32)
    # exact ties: one bit past the bf16 grid, for both parities of the last kept bit
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3 * 2 ** -9 + 2 ** -16,
                     2 ** -130 + 2 ** -134], dtype=np.float32)
    return np.concatenate([x, ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])


def pin_encode_bf16_matches_torch(orc):
    x = _wide_fp32_sample(_rng(1), 200000)
    got = orc.encode(x.astype(np.float64), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def pin_encode_fp16_matches_numpy(orc):
    rng = _rng(2)
    n = 200000
    x = rng.uniform(1.0, 2.0, n) * np.exp2(rng.integers(-27, 18, n)) * rng.choice([-1, 1], n)
    ties = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65504.0, 65519.99, 65520.0, 2 ** -25,
                     3 * 2 ** -26, 2 ** -24 * 1.5, 2 ** -14 - 2 ** -25, 0.0, -0.0])
    x = np.concatenate([x, ties, -ties])
    got = orc.encode(x, "fp16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def pin_encode_decode_roundtrip(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in ("bf16", "fp16"):
        vals = orc.decode(bits, dt)
        keep = ~np.isnan(vals)
        assert np.array_equal(orc.encode(vals[keep], dt), bits[keep])


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def _rope_complex(x, pos, base):
    """RoPE written as complex multiplication: pair (x_2i, x_2i+1) is the
    complex number x_2i + 1j*x_2i+1, multiplied by exp(1j * p * base**(-2i/D))."""
    D = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freq = np.power(float(base), -np.arange(0, D, 2, dtype=np.float64) / D)
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * freq)
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def pin_rope_position_zero_identity(orc):
    x = _rng(3).standard_normal((7, 128))
    assert np.array_equal(orc.rope(x, np.zeros(7, np.int64), 500000.0), x)


def pin_rope_preserves_pair_norms(orc):
    rng = _rng(4)
    x = rng.standard_normal((64, 128))
    pos = rng.integers(0, 32768, 64)
    y = orc.rope(x, pos, 10000.0)
    nx = np.hypot(x[:, 0::2], x[:, 1::2])
    ny = np.hypot(y[:, 0::2], y[:, 1::2])
    assert np.max(np.abs(ny - nx) / nx) < 1e-14


def pin_rope_complex_form(orc):
    rng = _rng(5)
    for D in (2, 8, 64, 128):
        for base in (10000.0, 500000.0):
            x = rng.standard_normal((50, D))
            pos = np.concatenate([np.arange(10), rng.integers(0, 32768, 40)])
            got = orc.rope(x, pos, base)
            ref = _rope_complex(x, pos, base)
            assert np.max(np.abs(got - ref)) < 1e-10, (D, base)


def pin_rope_d2_rotates_by_position_radians(orc):
    # D = 2: the only frequency is base**0 = 1, so position p turns the pair by
    # p radians, counter-clockwise, whatever the base.
    pos = np.arange(0, 40, dtype=np.int64)
    x = np.tile(np.array([[1.0, 0.0]]), (40, 1))
    for base in (10000.0, 3.0):
        y = orc.rope(x, pos, base)
        assert np.allclose(y[:, 0], np.cos(pos), atol=1e-15, rtol=0)
        assert np.allclose(y[:, 1], np.sin(pos), atol=1e-15, rtol=0)


def pin_rope_first_and_last_frequency(orc):
    # unit vector on pair i at position 1 turns by exactly theta_i: theta_0 = 1
    # and theta_{D/2-1} = base**(-(D-2)/D).
    D, base = 64, 10000.0
    x = np.zeros((2, D))
    x[0, 0] = 1.0
    x[1, D - 2] = 1.0
    y = orc.rope(x, np.array([1, 1]), base)
    assert abs(math.atan2(y[0, 1], y[0, 0]) - 1.0) < 1e-15
    assert abs(math.atan2(y[1, D - 1], y[1, D - 2]) - base ** (-(D - 2) / D)) < 1e-15


def pin_rope_pairs_are_adjacent(orc):
    # a unit vector on coordinate c only ever mixes with its partner c ^ 1
    D = 16
    x = np.eye(D)
    y = orc.rope(x, np.full(D, 5), 100.0)
    for c in range(D):
        support = set(np.nonzero(np.abs(y[c]) > 1e-300)[0].tolist())
        assert support <= {c, c ^ 1}, (c, support)
        assert len(support) == 2


def pin_rope_shift_invariance(orc):
    # (R(m) q) . (R(n) k) depends only on m - n
    rng = _rng(6)
    for D, base in ((64, 10000.0), (128, 500000.0)):
        q = rng.standard_normal((30, D))
        k = rng.standard_normal((30, D))
        m = rng.integers(0, 16384, 30)
        n = rng.integers(0, 16384, 30)
        t = rng.integers(0, 16384, 30)
        d0 = np.sum(orc.rope(q, m, base) * orc.rope(k, n, base), axis=1)
        d1 = np.sum(orc.rope(q, m + t, base) * orc.rope(k, n + t, base), axis=1)
        scale = np.linalg.norm(q, axis=1) * np.linalg.norm(k, axis=1)
        assert np.max(np.abs(d0 - d1) / scale) < 1e-11


def pin_rope_composition(orc):
    rng = _rng(7)
    x = rng.standard_normal((40, 64))
    a = rng.integers(0, 16384, 40)
    b = rng.integers(0, 16384, 40)
    y = orc.rope(orc.rope(x, a, 10000.0), b, 10000.0)
    z = orc.rope(x, a + b, 10000.0)
    assert np.max(np.abs(y - z)) < 1e-10


# --------------------------------------------------------------------------
# causal attention
# --------------------------------------------------------------------------

def _brute_attention(q, k, v):
    """Explicit N x N score matrix, -inf above the diagonal, scipy softmax."""
    B, Hq, N, D = q.shape
    rep = Hq // k.shape[1]
    kk = np.repeat(k, rep, axis=1)
    vv = np.repeat(v, rep, axis=1)
    S = np.matmul(q, np.swapaxes(kk, -1, -2)) / np.sqrt(D)
    S[..., np.triu(np.ones((N, N), dtype=bool), 1)] = -np.inf
    lse = scipy.special.logsumexp(S, axis=-1)
    P = scipy.special.softmax(S, axis=-1)
    return np.matmul(P, vv), lse


def _qkv(rng, B, Hq, Hkv, N, D, sigma=1.0):
    return (sigma * rng.standard_normal((B, Hq, N, D)), sigma * rng.standard_normal((B, Hkv, N, D)),
            rng.standard_normal((B, Hkv, N, D)))


def pin_attention_bruteforce(orc):
    rng = _rng(8)
    for (B, Hq, Hkv, N, D) in ((1, 1, 1, 1, 2), (1, 2, 2, 5, 8), (2, 4, 1, 17, 16),
                               (1, 8, 2, 64, 64), (1, 6, 3, 33, 128)):
        q, k, v = _qkv(rng, B, Hq, Hkv, N, D, sigma=2.0)
        o, lse = orc.attention(q, k, v)
        ro, rlse = _brute_attention(q, k, v)
        assert np.max(np.abs(o - ro)) < 1e-12
        assert np.max(np.abs(lse - rlse)) < 1e-12


def pin_attention_torch_sdpa(orc):
    rng = _rng(9)
    B, Hq, Hkv, N, D = 2, 8, 2, 48, 32
    q, k, v = _qkv(rng, B, Hq, Hkv, N, D)
    o, _ = orc.attention(q, k, v)
    rep = Hq // Hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(rep, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def pin_attention_row0_is_v0(orc):
    rng = _rng(10)
    q, k, v = _qkv(rng, 1, 4, 2, 9, 64, sigma=3.0)
    o, lse = orc.attention(q, k, v)
    for h in range(4):
        g = h // 2
        assert np.array_equal(o[0, h, 0], v[0, g, 0])
        s00 = float(np.dot(q[0, h, 0], k[0, g, 0])) / 8.0
        assert abs(lse[0, h, 0] - s00) < 1e-13 * max(1.0, abs(s00))


def pin_attention_zero_query_mean(orc):
    rng = _rng(11)
    B, H, N, D = 1, 2, 40, 16
    q = np.zeros((B, H, N, D))
    _, k, v = _qkv(rng, B, H, H, N, D)
    o, lse = orc.attention(q, k, v)
    mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.max(np.abs(o - mean)) < 1e-14
    assert np.max(np.abs(lse - np.log(np.arange(1, N + 1))[None, None, :])) < 1e-14


def pin_attention_probabilities(orc):
    # with v_j = e_j the output row i is the probability row P_i.
    rng = _rng(12)
    N, D = 24, 32
    q = 2.0 * rng.standard_normal((1, 1, N, D))
    k = 2.0 * rng.standard_normal((1, 1, N, D))
    v = np.zeros((1, 1, N, D))
    v[0, 0, np.arange(N), np.arange(N)] = 1.0
    o, lse = orc.attention(q, k, v)
    P = o[0, 0, :, :N]
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-14
    assert np.all(P[np.triu(np.ones((N, N), dtype=bool), 1)] == 0.0)
    assert np.all(P[np.tril(np.ones((N, N), dtype=bool))] > 0.0)
    S = (q[0, 0] @ k[0, 0].T) / np.sqrt(D)
    for i in range(N):
        # log P_ij = s_ij - L_i on the visible keys
        assert np.max(np.abs(np.log(P[i, :i + 1]) - (S[i, :i + 1] - lse[0, 0, i]))) < 1e-12


def pin_attention_prefix_invariance(orc):
    rng = _rng(13)
    q, k, v = _qkv(rng, 1, 4, 4, 50, 16)
    o, lse = orc.attention(q, k, v)
    n2 = 21
    o2, lse2 = orc.attention(q[:, :, :n2], k[:, :, :n2], v[:, :, :n2])
    assert np.array_equal(o[:, :, :n2], o2)
    assert np.array_equal(lse[:, :, :n2], lse2)


def pin_attention_gqa_equals_repeated_mha(orc):
    rng = _rng(14)
    q, k, v = _qkv(rng, 2, 8, 2, 20, 16)
    o, lse = orc.attention(q, k, v)
    o2, lse2 = orc.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_attention_rows_subset(orc):
    rng = _rng(15)
    q, k, v = _qkv(rng, 2, 4, 2, 30, 16)
    o, lse = orc.attention(q, k, v)
    rows = rng.choice(2 * 4 * 30, 37, replace=False)
    o2, lse2 = orc.attention(q, k, v, rows=rows)
    assert np.array_equal(o.reshape(-1, 16)[rows], o2)
    assert np.array_equal(lse.reshape(-1)[rows], lse2)


def pin_attention_large_sigma_finite(orc):
    rng = _rng(16)
    q, k, v = _qkv(rng, 1, 2, 2, 64, 64, sigma=8.0)
    o, lse = orc.attention(q, k, v)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # each output row is a convex combination of the visible values
    vmax = np.maximum.accumulate(np.max(np.abs(v), axis=-1), axis=-1)
    assert np.all(np.max(np.abs(o), axis=-1) <= vmax + 1e-12)


# --------------------------------------------------------------------------
# RoPE then attention
# --------------------------------------------------------------------------

def pin_rope_attention_relative_position(orc):
    # rotating every query and key by position + t leaves attention unchanged
    rng = _rng(17)
    B, Hq, Hkv, N, D = 1, 4, 2, 32, 64
    q, k, v = _qkv(rng, B, Hq, Hkv, N, D)
    pos = np.arange(N)
    o1, l1 = orc.attention(orc.rope(q, pos, 10000.0), orc.rope(k, pos, 10000.0), v)
    o2, l2 = orc.attention(orc.rope(q, pos + 9000, 10000.0), orc.rope(k, pos + 9000, 10000.0), v)
    assert np.max(np.abs(o1 - o2)) < 1e-10 and np.max(np.abs(l1 - l2)) < 1e-10


def pin_rope_attention_closed_form_d2(orc):
    # D = 2, every q and k equal to (1, 0): after RoPE q_i = (cos i, sin i) and
    # k_j = (cos j, sin j), so s_ij = cos(i - j) / sqrt(2); v_j = (j, 1).
    N = 5
    one = np.array([[1.0, 0.0]] * N)
    bits = orc.encode(one, "bf16")[None, None]
    v = np.stack([np.arange(N, dtype=np.float64), np.ones(N)], axis=1)[None, None]
    o, lse, _, _ = orc.rope_attention(bits, bits, orc.encode(v, "bf16"), "bf16", 10000.0,
                                      variant="exact")
    for i in range(N):
        w = [math.exp(math.cos(i - j) / math.sqrt(2.0)) for j in range(i + 1)]
        z = math.fsum(w)
        assert abs(o[0, 0, i, 0] - math.fsum(j * w[j] for j in range(i + 1)) / z) < 1e-14
        assert abs(o[0, 0, i, 1] - 1.0) < 1e-15
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-14


def pin_rope_attention_variants(orc):
    rng = _rng(18)
    B, Hq, Hkv, N, D = 1, 2, 1, 40, 64
    q = torch.from_numpy(rng.standard_normal((B, Hq, N, D)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, N, D)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, N, D)).astype(np.float32)).to(torch.bfloat16)

    def b(t):
        return t.view(torch.int16).numpy().view(np.uint16)

    oe, le, qe, ke = orc.rope_attention(b(q), b(k), b(v), "bf16", 10000.0, variant="exact")
    orr, lr, qr, kr = orc.rope_attention(b(q), b(k), b(v), "bf16", 10000.0, variant="rounded")
    # the rounded operands are the exact ones rounded to bf16 (torch rounding
    # from fp64 via fp32 agrees except on double-rounding ties, absent here)
    ref_q = torch.from_numpy(qe).float().to(torch.bfloat16).double().numpy()
    assert np.mean(qr == ref_q) > 0.999
    assert np.max(np.abs(qr - qe) / np.maximum(np.abs(qe), 1e-30)) <= 2.0 ** -8 + 1e-12
    # rounding the operands perturbs the result only slightly
    assert np.max(np.abs(oe - orr)) < 2e-2 and np.max(np.abs(le - lr)) < 2e-2
    # the first row is exact in both: rotation by 0 is the identity
    assert np.array_equal(qe[:, :, 0], qr[:, :, 0])


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def pin_attention_bwd_torch_autograd(orc):
    # library special case: torch's fp64 autograd through scaled_dot_product_attention
    rng = _rng(19)
    for (B, Hq, Hkv, N, D) in ((1, 2, 2, 7, 8), (2, 4, 2, 33, 16), (1, 8, 1, 20, 64)):
        q, k, v = _qkv(rng, B, Hq, Hkv, N, D)
        do = rng.standard_normal(q.shape)
        dq, dk, dv, lse, delta = orc.attention_bwd(q, k, v, do)
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        rep = Hq // Hkv
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.repeat_interleave(rep, 1), vt.repeat_interleave(rep, 1), is_causal=True)
        o.backward(torch.from_numpy(do))
        for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
            ref = ref.numpy()
            assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        # Delta_i = sum_j P_ij dP_ij equals dO_i . o_i
        assert np.max(np.abs(delta - np.sum(do * o.detach().numpy(), axis=-1))) < 1e-12
        _, lse_f = orc.attention(q, k, v)
        assert np.max(np.abs(lse - lse_f)) < 1e-13


def pin_attention_bwd_finite_differences(orc):
    # central differences of L = sum(dO * o) through the oracle's forward
    rng = _rng(20)
    B, Hq, Hkv, N, D = 1, 4, 2, 9, 6
    q, k, v = _qkv(rng, B, Hq, Hkv, N, D)
    do = rng.standard_normal(q.shape)
    dq, dk, dv, _, _ = orc.attention_bwd(q, k, v, do)

    def loss(q_, k_, v_):
        return float(np.sum(do * orc.attention(q_, k_, v_)[0]))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [tuple(rng.integers(0, s) for s in x.shape) for _ in range(12)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def pin_attention_bwd_special_cases(orc):
    rng = _rng(21)
    B, Hq, Hkv, N, D = 1, 4, 2, 24, 16
    q, k, v = _qkv(rng, B, Hq, Hkv, N, D)
    do = rng.standard_normal(q.shape)
    # every key equal: the scores of a row are all equal, softmax is flat in
    # them, so the query gradient vanishes
    kc = np.broadcast_to(k[:, :, :1], k.shape).copy()
    dq, _, _, _, _ = orc.attention_bwd(q, kc, v, do)
    assert np.max(np.abs(dq)) < 1e-12
    # probabilities of a row sum to one: the value gradients of a key head sum
    # to the output gradients of its query heads
    _, dk, dv, _, _ = orc.attention_bwd(q, k, v, do)
    ref = do.reshape(B, Hkv, Hq // Hkv, N, D).sum(axis=(2, 3))
    assert np.max(np.abs(dv.sum(axis=2) - ref)) < 1e-11
    # dS rows sum to zero, so sum_j dk_j = tau sum_i (sum_j dS_ij) q_i = 0
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-11
    # row 0 sees only key 0: its P is 1 and dS is 0, so dO_0 reaches only v_0
    do0 = np.zeros_like(do)
    do0[:, :, 0] = do[:, :, 0]
    dq0, dk0, dv0, _, _ = orc.attention_bwd(q, k, v, do0)
    assert np.max(np.abs(dq0)) == 0.0 and np.max(np.abs(dk0)) == 0.0
    assert np.max(np.abs(dv0[:, :, 1:])) == 0.0


def _rope_attention_bwd_fd(orc, pairing, seed, slopes=None, base=10000.0):
    # gradients with respect to the unrotated q and k (the inverse rotation),
    # against central differences of the RoPE-then-attention forward (with
    # the ALiBi penalty when slopes are given, without RoPE when base is None)
    rng = _rng(seed)
    B, Hq, Hkv, N, D = 1, 2, 1, 12, 8

    def bf16_bits(shape):
        x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
        return x.view(torch.int16).numpy().view(np.uint16)

    qb, kb, vb, dob = (bf16_bits(s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D),
                                              (B, Hq, N, D)))
    q, k, v, do = (orc.decode(b, "bf16") for b in (qb, kb, vb, dob))
    dq, dk, dv, delta, lse = orc.rope_attention_bwd(qb, kb, vb, dob, "bf16", base,
                                                    variant="exact", pairing=pairing,
                                                    slopes=slopes)
    pos = np.arange(N)

    def rot(x):
        return x if base is None else orc.rope(x, pos, base, pairing)

    def loss(q_, k_, v_):
        o, _ = orc.attention(rot(q_), rot(k_), v_, slopes=slopes)
        return float(np.sum(do * o))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [tuple(rng.integers(0, s) for s in x.shape) for _ in range(12)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def pin_rope_attention_bwd_finite_differences(orc):
    _rope_attention_bwd_fd(orc, "adjacent", 22)


def pin_rope_half_attention_bwd_finite_differences(orc):
    # the half-split pairing's gradient: the inverse turn of pairs (i, i + D/2)
    _rope_attention_bwd_fd(orc, "half", 26)


def pin_alibi_attention_bwd_finite_differences(orc):
    # the ALiBi backward: P carries the penalty (one slope per query head,
    # steep enough to matter over 12 positions), with and without RoPE
    slopes = np.array([0.5, 0.125])
    _rope_attention_bwd_fd(orc, "adjacent", 27, slopes=slopes, base=None)
    _rope_attention_bwd_fd(orc, "adjacent", 28, slopes=slopes)
    _rope_attention_bwd_fd(orc, "half", 29, slopes=slopes)


def pin_alibi_bwd_zero_slopes_is_plain_backward(orc):
    rng = _rng(30)
    q, k, v, do = (rng.standard_normal(s) for s in ((1, 4, 9, 8), (1, 2, 9, 8), (1, 2, 9, 8),
                                                     (1, 4, 9, 8)))
    plain = orc.attention_bwd(q, k, v, do)
    alibi = orc.attention_bwd(q, k, v, do, slopes=np.zeros(4))
    for a, b in zip(plain, alibi):
        assert np.array_equal(a, b)
    # and the forward's L is the backward's
    _, lse = orc.attention(q, k, v, slopes=np.array([0.3, 0.0, 0.7, 1.5]))
    assert np.max(np.abs(orc.attention_bwd(q, k, v, do, slopes=np.array([0.3, 0.0, 0.7, 1.5]))[3]
                         - lse)) < 1e-12


# --------------------------------------------------------------------------
# RoPE, half-split pairing (i, i + D/2)
# --------------------------------------------------------------------------

def pin_rope_half_complex_form(orc):
    # pair i is the complex number x_i + 1j*x_{i+D/2}, turned by p * base**(-2i/D)
    rng = _rng(23)
    for D in (2, 8, 64, 128):
        for base in (10000.0, 500000.0):
            x = rng.standard_normal((40, D))
            pos = np.concatenate([np.arange(8), rng.integers(0, 32768, 32)])
            freq = np.power(base, -np.arange(0, D, 2, dtype=np.float64) / D)
            z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * pos[:, None] * freq)
            ref = np.concatenate([z.real, z.imag], axis=1)
            got = orc.rope(x, pos, base, "half")
            assert np.max(np.abs(got - ref)) < 1e-10, (D, base)


def pin_rope_half_is_permuted_adjacent(orc):
    # interleaving the two halves turns pairs (i, i+D/2) into (2i, 2i+1)
    rng = _rng(24)
    D = 128
    x = rng.standard_normal((30, D))
    pos = rng.integers(0, 32768, 30)
    perm = np.empty(D, dtype=np.int64)
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    inv = np.argsort(perm)
    via_adjacent = orc.rope(x[:, perm], pos, 500000.0)[:, inv]
    assert np.max(np.abs(orc.rope(x, pos, 500000.0, "half") - via_adjacent)) < 1e-13


def pin_rope_half_invariants(orc):
    rng = _rng(25)
    D = 64
    x = rng.standard_normal((16, D))
    assert np.array_equal(orc.rope(x, np.zeros(16, np.int64), 10000.0, "half"), x)
    pos = rng.integers(0, 32768, 16)
    y = orc.rope(x, pos, 10000.0, "half")
    nx = np.hypot(x[:, :D // 2], x[:, D // 2:])
    ny = np.hypot(y[:, :D // 2], y[:, D // 2:])
    assert np.max(np.abs(ny - nx) / nx) < 1e-14
    # dot products after rotation depend only on the position difference
    q, k = rng.standard_normal((2, D))
    scale = np.linalg.norm(q) * np.linalg.norm(k)
    for m, n, t in ((5, 3, 1000), (100, 7, 16000), (0, 0, 16384)):
        a = orc.rope(q, m, 10000.0, "half") @ orc.rope(k, n, 10000.0, "half")
        b = orc.rope(q, m + t, 10000.0, "half") @ orc.rope(k, n + t, 10000.0, "half")
        assert abs(a - b) / scale < 1e-11


# --------------------------------------------------------------------------
# ALiBi: a linear penalty by distance added to the scaled scores
# --------------------------------------------------------------------------

def _alibi_slopes(H):
    """The geometric slope sequence 2^(-8(h+1)/H) of the ALiBi method."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)])


def pin_alibi_torch_sdpa_float_mask(orc):
    # torch adds a float attn_mask to the scaled scores: the bias -m_h (i - j)
    # with -inf above the diagonal, one slope per query head, GQA by repeat
    rng = _rng(40)
    for (B, Hq, Hkv, N, D) in ((1, 4, 4, 33, 16), (2, 8, 2, 48, 32), (1, 6, 3, 17, 64)):
        q, k, v = _qkv(rng, B, Hq, Hkv, N, D, sigma=1.5)
        slopes = _alibi_slopes(Hq) * rng.uniform(0.5, 2.0, Hq)
        o, lse = orc.attention(q, k, v, slopes=slopes)
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        bias = -slopes[:, None, None] * (i - j)[None].astype(np.float64)
        bias = np.where((j > i)[None], -np.inf, bias)
        rep = Hq // Hkv
        tk = torch.from_numpy(k).repeat_interleave(rep, dim=1)
        tv = torch.from_numpy(v).repeat_interleave(rep, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), tk, tv, attn_mask=torch.from_numpy(bias)[None]).numpy()
        assert np.max(np.abs(o - ref)) < 1e-12
        S = np.matmul(q, np.swapaxes(tk.numpy(), -1, -2)) / np.sqrt(D) + bias[None]
        assert np.max(np.abs(lse - scipy.special.logsumexp(S, axis=-1))) < 1e-12


def pin_alibi_zero_queries_geometric(orc):
    # q = 0: every score is the penalty alone, so the weights of keys t back
    # are e^(-m t): a geometric series with closed-form sums
    N, D, H = 60, 16, 4
    q = np.zeros((1, H, N, D))
    k = _rng(41).standard_normal((1, H, N, D))
    v = np.zeros((1, H, N, D))
    v[0, :, 0, 0] = 1.0                      # picks out key 0's weight
    v[0, :, :, 1] = np.arange(N)             # the mean key position
    slopes = _alibi_slopes(H)
    o, lse = orc.attention(q, k, v, slopes=slopes)
    i = np.arange(N, dtype=np.float64)
    for h, m in enumerate(slopes):
        r = math.exp(-m)
        total = (1.0 - r ** (i + 1)) / (1.0 - r)          # sum_{t=0..i} r^t
        assert np.max(np.abs(lse[0, h] - np.log(total))) < 1e-13
        assert np.max(np.abs(o[0, h, :, 0] - r ** i / total)) < 1e-14
        # mean position i - E[t], E[t] = sum t r^t / sum r^t
        et = (r * (1 - (i + 1) * r ** i + i * r ** (i + 1)) / (1 - r) ** 2) / total
        assert np.max(np.abs(o[0, h, :, 1] - (i - et))) < 1e-11


def pin_alibi_zero_slopes_is_plain_attention(orc):
    rng = _rng(42)
    q, k, v = _qkv(rng, 2, 4, 2, 31, 32, sigma=2.0)
    o, lse = orc.attention(q, k, v)
    o2, lse2 = orc.attention(q, k, v, slopes=np.zeros(4))
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


def pin_alibi_steep_slope_keeps_the_diagonal(orc):
    # a slope far above the spread of the scores leaves only key j = i
    rng = _rng(43)
    q, k, v = _qkv(rng, 1, 2, 1, 20, 16, sigma=0.5)
    o, lse = orc.attention(q, k, v, slopes=np.array([80.0, 120.0]))
    for h in range(2):
        assert np.max(np.abs(o[0, h] - v[0, 0])) < 1e-20 + 1e-25
        sii = np.einsum("nd,nd->n", q[0, h], k[0, 0]) / 4.0
        assert np.max(np.abs(lse[0, h] - sii)) < 1e-14


ALL_PINS = [obj for name, obj in sorted(globals().items()) if name.startswith("pin_")]
