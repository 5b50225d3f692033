"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test fixes one part of the oracle with something independent of it: a
closed form, an invariant of the mathematics, a library routine used as a
special case, or brute force on small inputs.  The pages print no worked
example, so there is no stored value from them.  A plausible mistake in the
oracle (a dropped term, a wrong sign, a transposed operand, a wrong flatten
order, the wrong Sinkhorn order, a different rounding) fails at least one
of these tests.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O

EPS = 1e-6
S = 2.0


def _kw(**over):
    kw = dict(hc_norm_eps=EPS, hc_post_scale=S, sinkhorn_eps=EPS, sinkhorn_iters=20)
    kw.update(over)
    return kw


def _bf16_values(shape, rng, scale=1.0):
    a = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return a.to(torch.bfloat16).to(torch.float64).numpy()


def _logit(p):
    return math.log(p / (1.0 - p))


# ----------------------------------------------------------------------------
# number formats against torch's casts
# ----------------------------------------------------------------------------

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),    # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
    ])
    # exact ties: bf16 value + half a bf16 ulp
    base = torch.from_numpy(rng.standard_normal(20000).astype(np.float32)).to(torch.bfloat16)
    bits = base.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
    ties = (bits | 0x8000).view(np.float32)
    f = np.concatenate([f, ties])
    ours = O.bf16_round(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_round_fixes_every_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]   # drop inf/NaN
    v = O.bf16_bits_to_f64(bits.astype(np.uint16))
    assert np.array_equal(O.bf16_round(v), v)
    assert np.array_equal(O.f64_to_bf16_bits(v), bits.astype(np.uint16))


def _all_bf16_in(lo, hi):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f64(bits)
    return v[np.isfinite(v) & (v >= lo) & (v <= hi)]


def test_e4m3_encode_matches_torch_exhaustive_over_bf16():
    v = _all_bf16_in(-448.0, 448.0)
    ours = O.e4m3_encode(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_matches_torch_on_scaled_values():
    # the quantizer sees bf16 values times powers of two, including ties
    rng = np.random.default_rng(2)
    v = _all_bf16_in(-448.0, 448.0)
    k = rng.integers(-8, 9, size=v.shape)
    w = v * np.ldexp(1.0, k)
    w = w[np.abs(w) <= 448.0]
    ours = O.e4m3_encode(w)
    ref = torch.from_numpy(w.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert O.e4m3_decode(np.array([0x7E]))[0] == 448.0


def test_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([449.0]))


# ----------------------------------------------------------------------------
# MXFP8 scale rule
# ----------------------------------------------------------------------------

def _brute_e(a):
    if a == 0:
        return -127
    for e in range(-127, 128):
        if a <= 448.0 * 2.0 ** e:
            return e
    return 127


def test_scale_exponent_brute_force():
    v = np.abs(_all_bf16_in(0.0, 3e38))
    v = np.concatenate([v, np.ldexp(448.0, np.arange(-130, 120)), np.ldexp(448.0, np.arange(-130, 120)) * (1 + 2.0 ** -7)])
    ours = O.mxfp8_scale_exponent(v)
    ref = np.array([max(-127, min(127, _brute_e(a))) for a in v])
    assert np.array_equal(ours, ref)


def test_scale_exponent_from_bf16_bits():
    # independent derivation from the bf16 encoding: amax = (1 + f/128) 2^E,
    # 448 = 1.75 * 2^8, so e = E - 8 when f <= 96 and E - 7 otherwise.
    bits = np.arange(1 << 15, dtype=np.uint32)          # positive values
    expf = (bits >> 7) & 0xFF
    keep = (expf > 0) & (expf < 0xFF)
    bits, expf = bits[keep], expf[keep]
    frac = bits & 0x7F
    E = expf.astype(np.int64) - 127
    e_rule = np.clip(np.where(frac > 96, E - 7, E - 8), -127, 127)
    v = O.bf16_bits_to_f64(bits.astype(np.uint16))
    assert np.array_equal(O.mxfp8_scale_exponent(v), e_rule)


def test_mxfp8_invariants_over_decades():
    rng = np.random.default_rng(3)
    T, C = 64, 256
    h = O.bf16_round(rng.standard_normal((T, C)) * (10.0 ** rng.uniform(-2, 3, size=(T, 1))))
    h[0, :32] = 0.0                      # a zero block
    h[1, 32:64] = 1e-38                  # tiny block: clamped exponent
    q, sc = O.mxfp8(h)
    e = sc.astype(np.int64) - 127
    blk = h.reshape(T, C // 32, 32)
    amax = np.abs(blk).max(-1)
    assert sc[0, 0] == 0 and np.all(q[0, :32] == 0)
    unclamped = (amax > 0) & (e > -127)
    r = amax[unclamped] * np.ldexp(1.0, -e[unclamped])
    assert np.all((r > 224.0) & (r <= 448.0))
    dec = O.e4m3_decode(q).reshape(T, C // 32, 32) * np.ldexp(1.0, e)[:, :, None]
    scaled = np.abs(blk) * np.ldexp(1.0, -e)[:, :, None]
    _, ex = np.frexp(scaled)
    half_ulp = np.ldexp(1.0, np.maximum(ex - 4, -9)) / 2 * np.ldexp(1.0, e)[:, :, None]
    assert np.all(np.abs(dec - blk) <= half_ulp)


# ----------------------------------------------------------------------------
# Coeffs
# ----------------------------------------------------------------------------

def test_coeffs_zero_projection_closed_form():
    rng = np.random.default_rng(4)
    T, C = 3, 1024
    x = _bf16_values((T, 4, C), rng)
    cf = O.coeffs(x, np.zeros((4 * C, 24)), np.zeros(24), **_kw())
    assert np.all(cf[:, 0:4] == 0.5)
    assert np.all(cf[:, 4:8] == S / 2)
    m = 1.0                              # all logits 0: every entry follows m -> m/(4m+eps)
    for _ in range(40):
        m = m / (4.0 * m + EPS)
    np.testing.assert_allclose(cf[:, 8:], m, rtol=1e-14, atol=0)


def test_coeffs_rms_scale_closed_form():
    # x constant a: r = 1/sqrt(a^2 + eps); a one-hot phi column gives l = r*a + b
    C = 1024
    for a in (0.75, -3.0, 1e-3):
        x = np.full((1, 4, C), a)
        phi = np.zeros((4 * C, 24))
        phi[5, 0] = 1.0
        phi[2 * C + 7, 1] = -2.0
        bias = np.zeros(24)
        bias[0], bias[1] = 0.25, -0.5
        cf = O.coeffs(x, phi, bias, **_kw())
        r = 1.0 / math.sqrt(a * a + EPS)
        assert math.isclose(_logit(cf[0, 0]), r * a + 0.25, rel_tol=1e-12, abs_tol=1e-12)
        assert math.isclose(_logit(cf[0, 1]), -2.0 * r * a - 0.5, rel_tol=1e-12, abs_tol=1e-12)


def test_coeffs_flatten_order_is_route_major():
    # a one-hot phi row k = i*C + c must pick x[t, i, c]
    rng = np.random.default_rng(5)
    T, C = 4, 1024
    x = _bf16_values((T, 4, C), rng)
    picks = [(0, 3), (1, 1000), (2, 17), (3, 512), (3, 0), (0, 1023), (2, 600), (1, 5)]
    phi = np.zeros((4 * C, 24))
    for m, (i, c) in enumerate(picks):
        phi[i * C + c, m] = 0.01
    cf = O.coeffs(x, phi, np.zeros(24), **_kw())
    r = 1.0 / np.sqrt((x ** 2).sum(axis=(1, 2)) / (4 * C) + EPS)
    for m, (i, c) in enumerate(picks):
        p = cf[:, m] if m < 4 else cf[:, m] / S
        lg = np.log(p / (1 - p))
        np.testing.assert_allclose(lg, 0.01 * r * x[:, i, c], rtol=1e-9, atol=1e-12)


def test_coeffs_projection_against_torch_rms_norm():
    # library special case: logits = rms_norm(x_flat) @ phi + bias (torch, fp64)
    rng = np.random.default_rng(6)
    T, C = 8, 2048
    x = _bf16_values((T, 4, C), rng)
    phi = rng.standard_normal((4 * C, 24)) * 0.02
    bias = rng.standard_normal(24) * 0.1
    cf = O.coeffs(x, phi, bias, **_kw())
    xt = torch.from_numpy(x.reshape(T, 4 * C))
    lg = torch.nn.functional.rms_norm(xt, (4 * C,), eps=EPS) @ torch.from_numpy(phi) + torch.from_numpy(bias)
    lg = lg.numpy()
    np.testing.assert_allclose(cf[:, 0:4], torch.sigmoid(torch.from_numpy(lg[:, 0:4])).numpy(), rtol=1e-12)
    np.testing.assert_allclose(cf[:, 4:8], S * torch.sigmoid(torch.from_numpy(lg[:, 4:8])).numpy(), rtol=1e-12)
    # res entries are a positive rescaling of exp(logit): D1 exp(l) D2, so the
    # cross ratios res_ab res_cd / (res_ad res_cb) equal those of exp(l)
    res = cf[:, 8:].reshape(T, 4, 4)
    ex = np.exp(lg[:, 8:]).reshape(T, 4, 4)
    for (a, b, c, d) in [(0, 0, 1, 1), (0, 2, 3, 1), (2, 3, 1, 0)]:
        lhs = res[:, a, b] * res[:, c, d] / (res[:, a, d] * res[:, c, b])
        rhs = ex[:, a, b] * ex[:, c, d] / (ex[:, a, d] * ex[:, c, b])
        np.testing.assert_allclose(lhs, rhs, rtol=1e-10)


def test_coeffs_power_of_two_scale_invariance():
    rng = np.random.default_rng(7)
    T, C = 5, 1024
    x = _bf16_values((T, 4, C), rng)
    phi = rng.standard_normal((4 * C, 24)) * 0.02
    bias = rng.standard_normal(24) * 0.1
    base = O.coeffs(x, phi, bias, **_kw(hc_norm_eps=0.0))
    for k in (-5, 3, 11):
        assert np.array_equal(O.coeffs(x * 2.0 ** k, phi, bias, **_kw(hc_norm_eps=0.0)), base)


def test_coeffs_ranges_and_column_sums():
    rng = np.random.default_rng(8)
    T, C = 64, 1024
    x = _bf16_values((T, 4, C), rng)
    phi = rng.standard_normal((4 * C, 24)) * 0.02
    bias = rng.standard_normal(24) * 0.1
    cf = O.coeffs(x, phi, bias, **_kw())
    pre, post, res = O.split_coeffs(cf)
    assert np.all((pre > 0) & (pre < 1))
    assert np.all((post > 0) & (post < S))
    assert np.all(res > 0)
    # the last pass normalises columns: each column sums to S/(S+eps) ~ 1 - eps
    col = res.sum(axis=1)
    assert np.all(np.abs(col - 1.0) <= 2e-6)


def test_sinkhorn_order_rows_then_columns():
    # after one iteration the columns are normalised and the rows are not
    rng = np.random.default_rng(9)
    m = np.exp(rng.standard_normal((32, 4, 4)) * 2.0)
    r = O.sinkhorn(m, 1, 0.0)
    np.testing.assert_allclose(r.sum(axis=1), 1.0, rtol=1e-14)
    assert np.max(np.abs(r.sum(axis=2) - 1.0)) > 1e-2
    # one iteration by hand on a 2-step definition: rows first
    m0 = m[0]
    rows = m0 / m0.sum(axis=1, keepdims=True)
    cols = rows / rows.sum(axis=0, keepdims=True)
    np.testing.assert_allclose(r[0], cols, rtol=1e-14)


def test_sinkhorn_rank_one_gives_quarter():
    rng = np.random.default_rng(10)
    u, v = rng.uniform(-3, 3, size=4), rng.uniform(-3, 3, size=4)
    bias = np.zeros(24)
    bias[8:] = (u[:, None] + v[None, :]).reshape(16)
    cf = O.coeffs(np.ones((1, 4, 1024)), np.zeros((4096, 24)), bias, **_kw(sinkhorn_eps=0.0, sinkhorn_iters=1))
    np.testing.assert_allclose(cf[0, 8:], 0.25, rtol=1e-14)


def test_sinkhorn_limit_recovers_doubly_stochastic_core():
    # Sinkhorn scaling is unique: D1 K D2 with K doubly stochastic converges
    # to K (and a transposed layout would give K^T, which differs here)
    rng = np.random.default_rng(11)
    perms = [np.eye(4)[list(p)] for p in ([1, 2, 3, 0], [0, 1, 2, 3], [2, 0, 3, 1], [3, 2, 0, 1])]
    w = np.array([0.4, 0.3, 0.2, 0.1])
    K = 0.9 * sum(wi * P for wi, P in zip(w, perms)) + 0.1 / 4.0   # positive, doubly stochastic
    assert not np.allclose(K, K.T)
    d1, d2 = rng.uniform(0.2, 5, 4), rng.uniform(0.2, 5, 4)
    bias = np.zeros(24)
    bias[8:] = np.log(d1[:, None] * K * d2[None, :]).reshape(16)
    cf = O.coeffs(np.ones((1, 4, 1024)), np.zeros((4096, 24)), bias, **_kw(sinkhorn_eps=0.0, sinkhorn_iters=2000))
    np.testing.assert_allclose(cf[0, 8:].reshape(4, 4), K, atol=1e-12)


def test_sinkhorn_diagonal_bias_gives_identity():
    bias = np.full(24, -30.0)
    for j in range(4):
        bias[8 + 4 * j + j] = 30.0
    cf = O.coeffs(np.ones((1, 4, 1024)), np.zeros((4096, 24)), bias, **_kw())
    np.testing.assert_allclose(cf[0, 8:].reshape(4, 4), np.eye(4), atol=1e-20 + 2e-6)
    off = cf[0, 8:].reshape(4, 4)[~np.eye(4, dtype=bool)]
    assert np.all(off < 1e-25)


def test_sinkhorn_rows_converge_on_small_logits():
    # with small logits 20 iterations bring the rows within 1e-4 of 1 as well
    rng = np.random.default_rng(12)
    T, C = 64, 1024
    x = _bf16_values((T, 4, C), rng)
    phi = rng.standard_normal((4 * C, 24)) * 0.004
    bias = rng.standard_normal(24) * 0.05
    res = O.split_coeffs(O.coeffs(x, phi, bias, **_kw()))[2]
    assert np.max(np.abs(res.sum(axis=2) - 1.0)) < 1e-4
    assert np.max(np.abs(res.sum(axis=1) - 1.0)) < 1e-4


def test_coeffs_route_permutation_equivariance():
    # permuting the routes of x together with phi's row blocks and the
    # pre/post/res indices permutes the outputs the same way
    rng = np.random.default_rng(13)
    T, C = 6, 1024
    x = _bf16_values((T, 4, C), rng)
    phi = rng.standard_normal((4 * C, 24)) * 0.02
    bias = rng.standard_normal(24) * 0.1
    p = np.array([2, 0, 3, 1])
    xp = x[:, p, :]
    blocks = phi.reshape(4, C, 24)[p].reshape(4 * C, 24)
    col = np.concatenate([p, 4 + p, 8 + (4 * p[:, None] + p[None, :]).reshape(16)])
    cf = O.coeffs(x, phi, bias, **_kw())
    cfp = O.coeffs(xp, blocks[:, col], bias[col], **_kw())
    np.testing.assert_allclose(cfp, cf[:, col], rtol=1e-12)


# ----------------------------------------------------------------------------
# Pre and Post
# ----------------------------------------------------------------------------

def test_pre_one_hot_is_rms_norm_of_a_route():
    rng = np.random.default_rng(14)
    T, C = 4, 2048
    x = _bf16_values((T, 4, C), rng)
    gamma = 1.0 + rng.standard_normal(C) * 0.05
    for k in range(4):
        w = np.zeros((T, 4))
        w[:, k] = 1.0
        h = O.pre(x, w, gamma, rmsnorm_eps=EPS)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x[:, k, :]), (C,), weight=torch.from_numpy(gamma), eps=EPS).numpy()
        assert np.all(np.abs(h - ref) <= np.abs(ref) * 2.0 ** -8 * (1 + 1e-9))
        assert np.mean(h == O.bf16_round(ref)) > 0.9999


def test_pre_matches_torch_for_general_weights():
    rng = np.random.default_rng(15)
    T, C = 8, 1024
    x = _bf16_values((T, 4, C), rng)
    w = rng.uniform(0.05, 0.95, size=(T, 4))
    gamma = 1.0 + rng.standard_normal(C) * 0.05
    h = O.pre(x, w, gamma, rmsnorm_eps=EPS)
    g = torch.einsum("ti,tic->tc", torch.from_numpy(w), torch.from_numpy(x))
    ref = torch.nn.functional.rms_norm(g, (C,), weight=torch.from_numpy(gamma), eps=EPS).numpy()
    assert h.shape == ref.shape and np.mean(h == O.bf16_round(ref)) > 0.9999
    assert np.all(np.abs(h - ref) <= np.abs(ref) * 2.0 ** -8 * (1 + 1e-9))


def test_pre_scale_invariance_with_zero_eps():
    rng = np.random.default_rng(16)
    x = _bf16_values((3, 4, 1024), rng)
    w = rng.uniform(0.05, 0.95, size=(3, 4))
    gamma = 1.0 + rng.standard_normal(1024) * 0.05
    h = O.pre(x, w, gamma, rmsnorm_eps=0.0)
    for k in (-7, 4):
        assert np.array_equal(O.pre(x * 2.0 ** k, w, gamma, rmsnorm_eps=0.0), h)


def test_post_identity_and_pure_y():
    rng = np.random.default_rng(17)
    T, C = 5, 1024
    x = _bf16_values((T, 4, C), rng)
    y = _bf16_values((T, C), rng)
    eye = np.broadcast_to(np.eye(4), (T, 4, 4))
    assert np.array_equal(O.post(x, y, np.zeros((T, 4)), eye), x)
    for j in range(4):
        pw = np.zeros((T, 4))
        pw[:, j] = 1.0
        out = O.post(x, y, pw, np.zeros((T, 4, 4)))
        assert np.array_equal(out[:, j], y)
        assert np.all(np.delete(out, j, axis=1) == 0)


def test_post_matches_torch_bmm():
    rng = np.random.default_rng(18)
    T, C = 6, 1024
    x = _bf16_values((T, 4, C), rng)
    y = _bf16_values((T, C), rng)
    res = O.f32_round(rng.uniform(0, 0.5, size=(T, 4, 4)))   # not symmetric: catches a transposed res
    pw = O.f32_round(rng.uniform(0, 2, size=(T, 4)))
    out = O.post(x, y, pw, res)
    ref = torch.bmm(torch.from_numpy(res), torch.from_numpy(x)) + torch.from_numpy(pw)[:, :, None] * torch.from_numpy(y)[:, None, :]
    ref = ref.numpy()
    # bf16 rounding plus the binary32 chain's error, bounded by the absolute terms
    absum = np.abs(pw)[:, :, None] * np.abs(y)[:, None, :] + np.einsum("tji,tic->tjc", np.abs(res), np.abs(x))
    assert np.all(np.abs(out - ref) <= np.abs(ref) * 2.0 ** -8 + absum * 2.0 ** -21)
    # and it is the plain definition except near bf16 midpoints
    assert np.mean(out == O.post_exact(x, y, pw, res)) > 0.9995
    assert np.mean(O.post_exact(x, y, pw, res) == O.bf16_round(ref)) > 0.99999


def _fma_exact(a, b, c):
    """Correctly rounded binary32 a*b+c from exact rationals."""
    from fractions import Fraction
    v = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    r = np.float32(float(v))
    best = None
    for cand in (np.nextafter(r, np.float32(-np.inf)), r, np.nextafter(r, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - v)
        key = (d, int(np.array(cand).view(np.uint32)) & 1)   # ties to even mantissa
        if best is None or key < best[0]:
            best = (key, cand)
    return float(best[1])


def test_fma_f32_against_exact_rationals():
    rng = np.random.default_rng(21)
    n = 3000
    a = O.f32_round(rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3, n))
    b = O.bf16_round(rng.standard_normal(n))
    c = O.f32_round(-a * b * (1 + rng.standard_normal(n) * 1e-3))    # heavy cancellation too
    ours = O.fma_f32(a, b, c)
    ref = np.array([_fma_exact(*t) for t in zip(a, b, c)])
    assert np.array_equal(ours, ref)


def test_fma_f32_midpoint_ties():
    mid = 1.0 + 2.0 ** -24            # halfway between 1 and the next binary32
    tiny = 2.0 ** -40
    assert O.fma_f32(np.array([tiny]), np.array([tiny]), np.array([mid]))[0] == 1.0 + 2.0 ** -23
    assert O.fma_f32(np.array([-tiny]), np.array([tiny]), np.array([mid]))[0] == 1.0
    assert O.fma_f32(np.array([0.0]), np.array([1.0]), np.array([mid]))[0] == 1.0       # tie to even
    mid2 = 1.0 + 3 * 2.0 ** -24       # halfway between 1+2^-23 and 1+2^-22: even is up
    assert O.fma_f32(np.array([0.0]), np.array([1.0]), np.array([mid2]))[0] == 1.0 + 2.0 ** -22
    assert O.fma_f32(np.array([-tiny]), np.array([tiny]), np.array([mid2]))[0] == 1.0 + 2.0 ** -23
    # the product is the midpoint and the addend is absorbed
    a = 1.0 + 2.0 ** -12              # a*a = 1 + 2^-11 + 2^-24: a binary32 midpoint
    below = 2.0 ** -80                # below binary64 resolution of a*a
    assert O.fma_f32(np.array([a]), np.array([a]), np.array([below]))[0] == 1.0 + 2.0 ** -11 + 2.0 ** -23
    assert O.fma_f32(np.array([a]), np.array([a]), np.array([-below]))[0] == 1.0 + 2.0 ** -11


def _midpoint_token(C=1024):
    """One token whose route-0 output sits just above a bf16 midpoint.

    post_0 * y = 1 + 2^-8 (a bf16 midpoint, exact in binary32) and
    res[0, 0] * x_0 = 2^-30: the exact sum rounds up to 1 + 2^-7, but the
    binary32 chain absorbs 2^-30 and the tie goes to the even value 1.
    """
    x = np.zeros((1, 4, C))
    x[0, 0, :] = 1.0
    y = np.ones((1, C))
    pw = np.array([[1.0 + 2.0 ** -8, 0.5, 0.25, 1.0]])
    res = np.zeros((1, 4, 4))
    res[0, 0, 0] = 2.0 ** -30
    res[0, 1, 0] = res[0, 2, 0] = res[0, 3, 0] = 0.5
    return x, y, pw, res


def test_post_rounding_decision_is_binary32():
    x, y, pw, res = _midpoint_token()
    assert np.all(O.post_exact(x, y, pw, res)[0, 0] == 1.0 + 2.0 ** -7)
    assert np.all(O.post(x, y, pw, res)[0, 0] == 1.0)
    assert np.array_equal(O.post(x, y, pw, res)[0, 1:], O.post_exact(x, y, pw, res)[0, 1:])


def test_fused_takes_the_binary32_post():
    x, y, pw, res = _midpoint_token()
    cf_in = np.concatenate([np.full((1, 4), 0.5), pw, res.reshape(1, 16)], axis=1)
    rng = np.random.default_rng(22)
    phi = rng.standard_normal((4096, 24)) * 0.02
    out = O.post_pre_fused(x, y, cf_in, phi, np.zeros(24), np.ones(1024), hc_norm_eps=EPS, rmsnorm_eps=EPS,
                           hc_post_scale=S, sinkhorn_eps=EPS, sinkhorn_iters=20)
    assert np.all(out["x_out"][0, 0] == 1.0)


# ----------------------------------------------------------------------------
# The fused pass: hand expansion of one token
# ----------------------------------------------------------------------------

def _sk_lists(m, iters, eps):
    m = [row[:] for row in m]
    for _ in range(iters):
        for j in range(4):
            s = sum(m[j]) + eps
            m[j] = [v / s for v in m[j]]
        for i in range(4):
            s = sum(m[j][i] for j in range(4)) + eps
            for j in range(4):
                m[j][i] /= s
    return m


def _bf(v):
    return float(O.bf16_round(np.array([v]))[0])


def test_fused_hand_expansion_one_token():
    # T=1, C=1024, x_i = a_i constant, y = b constant, phi[iC+c, m] = w[i,m]/C,
    # gamma = gamma0 constant: every quantity reduces to a few scalars
    C = 1024
    a = [0.5, -1.25, 2.0, 0.375]
    b = -0.75
    rng = np.random.default_rng(19)
    w = np.round(rng.standard_normal((4, 24)) * 64) / 64          # exact /1024 below
    bias = np.round(rng.standard_normal(24) * 64) / 64
    gamma0 = 1.125
    pre_in = [0.3, 0.6, 0.2, 0.9]
    post_in = [0.5, 1.5, 0.25, 1.0]
    res_in = [[0.4, 0.1, 0.2, 0.3], [0.25, 0.25, 0.25, 0.25], [0.1, 0.6, 0.1, 0.2], [0.7, 0.05, 0.15, 0.1]]
    cf_in = O.f32_round(np.array([pre_in + post_in + sum(res_in, [])]))   # stored as binary32
    pre_in, post_in = list(cf_in[0, 0:4]), list(cf_in[0, 4:8])
    res_in = [list(cf_in[0, 8 + 4 * j:12 + 4 * j]) for j in range(4)]
    x = np.array([[[ai] * C for ai in a]], dtype=np.float64)
    y = np.full((1, C), b)
    phi = np.repeat(w, C, axis=0) / C                                  # row k = i*C + c
    out = O.post_pre_fused(x, y, cf_in, phi, bias, np.full(C, gamma0), hc_norm_eps=EPS,
                           rmsnorm_eps=EPS, hc_post_scale=S, sinkhorn_eps=EPS, sinkhorn_iters=20)
    # by hand
    xp = [_bf(sum(res_in[j][i] * a[i] for i in range(4)) + post_in[j] * b) for j in range(4)]
    r = 1.0 / math.sqrt(sum(v * v for v in xp) / 4.0 + EPS)
    d = [sum(xp[i] * w[i, m] for i in range(4)) for m in range(24)]
    lg = [r * d[m] + bias[m] for m in range(24)]
    sig = [1.0 / (1.0 + math.exp(-v)) for v in lg]
    pre_n = sig[0:4]
    post_n = [S * v for v in sig[4:8]]
    res_n = _sk_lists([[math.exp(lg[8 + 4 * j + i]) for i in range(4)] for j in range(4)], 20, EPS)
    g = sum(pre_n[i] * xp[i] for i in range(4))
    h = _bf(g * (1.0 / math.sqrt(g * g + EPS)) * gamma0)
    assert np.array_equal(out["x_out"][0], np.array([[v] * C for v in xp]))
    np.testing.assert_allclose(out["coeffs_next"][0, 0:4], pre_n, rtol=1e-12)
    np.testing.assert_allclose(out["coeffs_next"][0, 4:8], post_n, rtol=1e-12)
    np.testing.assert_allclose(out["coeffs_next"][0, 8:].reshape(4, 4), res_n, rtol=1e-12)
    assert np.all(out["h"][0] == h)


def test_fused_mxfp8_consistent_with_h():
    rng = np.random.default_rng(20)
    T, C = 8, 1024
    x = _bf16_values((T, 4, C), rng)
    y = _bf16_values((T, C), rng)
    phi = rng.standard_normal((4 * C, 24)) * 0.02
    bias = rng.standard_normal(24) * 0.1
    cf_in = O.f32_round(O.coeffs(x, phi, bias, **_kw()))
    out = O.post_pre_fused(x, y, cf_in, phi, bias, np.ones(C), hc_norm_eps=EPS, rmsnorm_eps=EPS,
                           hc_post_scale=S, sinkhorn_eps=EPS, sinkhorn_iters=20, with_mxfp8=True)
    # q decodes to h within half an e4m3 step of the block scale
    e = out["h_scale"].astype(np.int64) - 127
    dec = O.e4m3_decode(out["h_fp8"]).reshape(T, C // 32, 32) * np.ldexp(1.0, e)[:, :, None]
    blk = out["h"].reshape(T, C // 32, 32)
    assert np.all(np.abs(dec - blk) <= np.ldexp(1.0, e)[:, :, None] * 16.0 + 0.0)
    ref = torch.from_numpy((blk * np.ldexp(1.0, -e)[:, :, None]).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(ref.view(torch.uint8).numpy().reshape(T, C), out["h_fp8"])


# ----------------------------------------------------------------------------
# broadcast (first-layer) pre
# ----------------------------------------------------------------------------
def test_pre_broadcast_closed_forms():
    # A stream whose 4 routes are one row x0: the projection is x0 against the
    # route-summed phi (a [C, 24] matrix), the sum of squares is 4 * sum x0^2,
    # and since the pre weights are positive, h = x0 / sqrt(mean x0^2 +
    # eps / (sum pre)^2) * gamma (the norm does not see the common factor).
    rng = np.random.default_rng(23)
    T, C = 5, 1024
    x0 = _bf16_values((T, C), rng)
    phi = rng.standard_normal((4 * C, 24)) * 0.02
    bias = rng.standard_normal(24) * 0.1
    gamma = 1.0 + rng.standard_normal(C) * 0.05
    cf, h = O.pre_broadcast(x0, phi, bias, gamma, rmsnorm_eps=EPS, **_kw())
    phi_c = phi.reshape(4, C, 24).sum(axis=0)
    r = 1.0 / np.sqrt(4.0 * np.sum(x0 * x0, axis=1) / (4 * C) + EPS)
    logit = r[:, None] * (x0 @ phi_c) + bias[None, :]
    np.testing.assert_allclose(cf[:, 0:4], 1.0 / (1.0 + np.exp(-logit[:, 0:4])), rtol=1e-12)
    np.testing.assert_allclose(cf[:, 4:8], S / (1.0 + np.exp(-logit[:, 4:8])), rtol=1e-12)
    ps = cf[:, 0:4].sum(axis=1)
    hh = x0 / np.sqrt(np.mean(x0 * x0, axis=1) + EPS / ps ** 2)[:, None] * gamma[None, :]
    ref = torch.from_numpy(hh).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(h, ref)
    # res: the Sinkhorn of the broadcast logits (columns sum to 1)
    res = cf[:, 8:].reshape(T, 4, 4)
    np.testing.assert_allclose(res.sum(axis=1), 1.0, atol=1e-5)


# ----------------------------------------------------------------------------
# post of an int8 sublayer output with per-token scales
# ----------------------------------------------------------------------------

def _mul_exact_f32(q, s):
    """Correctly rounded binary32 product q * s from exact rationals."""
    from fractions import Fraction
    v = Fraction(int(q)) * Fraction(float(s))
    r = np.float32(float(v))
    best = None
    for cand in (np.nextafter(r, np.float32(-np.inf)), r, np.nextafter(r, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - v)
        key = (d, int(np.array(cand).view(np.uint32)) & 1)   # ties to even mantissa
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def test_post_int8_dequantises_per_token_in_binary32():
    # post_j = 1 on one route and res = 0 leave x'_j = bf16(y) with y the
    # binary32 product of the code and its token's scale; brute force on a
    # sample of elements
    rng = np.random.default_rng(41)
    T, C = 6, 1024
    q = rng.integers(-128, 128, (T, C))
    s = O.f32_round(10.0 ** rng.uniform(-4, 1, T) / 127.0)
    x = _bf16_values((T, 4, C), rng)
    j = 2
    pw = np.zeros((T, 4))
    pw[:, j] = 1.0
    out = O.post_int8(x, q, s, pw, np.zeros((T, 4, 4)))
    assert np.all(np.delete(out, j, axis=1) == 0)
    for t, c in zip(rng.integers(0, T, 400), rng.integers(0, C, 400)):
        y = _mul_exact_f32(q[t, c], s[t])
        want = torch.tensor([float(y)], dtype=torch.float32).to(torch.bfloat16).double().item()
        assert out[t, j, c] == want, (t, c)


def test_post_int8_power_of_two_scales_equal_bf16_post():
    # with a power-of-two scale per token the products are exact and bf16
    # values, so the int8 post is the bf16 post of y = q * 2**k[t]
    rng = np.random.default_rng(43)
    T, C = 7, 2048
    q = rng.integers(-128, 128, (T, C))
    k = rng.integers(-24, 6, T)
    y = np.ldexp(q.astype(np.float64), k[:, None])
    assert np.array_equal(O.bf16_round(y), y)
    x = _bf16_values((T, 4, C), rng)
    pw = O.f32_round(rng.uniform(0.0, 2.0, (T, 4)))
    res = O.f32_round(rng.dirichlet(np.ones(4), (T, 4)))
    got = O.post_int8(x, q, np.ldexp(1.0, k), pw, res)
    assert np.array_equal(got, O.post(x, y, pw, res))
    # a scale taken per channel instead of per token would differ
    assert not np.array_equal(got, O.post(x, q * np.ldexp(1.0, k[0]), pw, res))


def test_post_int8_rejects_bad_inputs():
    T, C = 2, 1024
    x = np.zeros((T, 4, C))
    pw, res = np.zeros((T, 4)), np.zeros((T, 4, 4))
    with pytest.raises(ValueError):
        O.post_int8(x, np.full((T, C), 200), np.ones(T), pw, res)
    with pytest.raises(ValueError):
        O.post_int8(x, np.zeros((T, C), dtype=np.int64), np.full(T, 0.1), pw, res)


def test_post_int8_rounds_the_product_to_binary32_first():
    # y32 = 65/64 times post = 1.25 is exactly the bf16 midpoint M = 325/256,
    # which bf16 rounds to even (324/256).  Codes and scales whose exact
    # product is y32 + e, with 0.4 < e / 2**-23 < 0.5, dequantise to y32 in
    # binary32 and give x' = 324/256; a product kept exact would put
    # post * y past M by more than half a binary32 step and round up to
    # 326/256
    from fractions import Fraction
    y32, u = Fraction(65, 64), Fraction(1, 2 ** 23)
    pairs = []
    for q in range(3, 128, 2):
        s0 = np.float32(float(y32 / q))
        for d in range(-4, 5):
            s = np.float32(s0)
            for _ in range(abs(d)):
                s = np.nextafter(s, np.float32(np.inf if d > 0 else -np.inf))
            e = Fraction(q) * Fraction(float(s)) - y32
            if Fraction(2, 5) * u < e < u / 2:
                pairs.append((q, float(s)))
    assert len(pairs) >= 3
    T, C = len(pairs), 1024
    q = np.array([[p[0]] * C for p in pairs])
    sc = np.array([p[1] for p in pairs])
    pw = np.zeros((T, 4))
    pw[:, 1] = 1.25
    zero_x, zero_r = np.zeros((T, 4, C)), np.zeros((T, 4, 4))
    assert np.all(O.post_int8(zero_x, q, sc, pw, zero_r)[:, 1] == 324 / 256)
    assert np.all(O.post_int8(zero_x, -q, sc, pw, zero_r)[:, 1] == -324 / 256)


def test_post_int8_pre_fused_is_the_fused_pass_on_the_int8_post():
    # power-of-two scales make y = q * 2**k exact bf16 values: the int8 fused
    # pass is then the bf16 fused pass, and its x_out is post_int8's
    rng = np.random.default_rng(47)
    T, C = 5, 1024
    q = rng.integers(-128, 128, (T, C))
    k = rng.integers(-12, 2, T)
    x = _bf16_values((T, 4, C), rng)
    cf = O.f32_round(O.coeffs(x, rng.standard_normal((4 * C, 24)) * 0.02, rng.standard_normal(24) * 0.1, **_kw()))
    phi, bias = rng.standard_normal((4 * C, 24)) * 0.02, rng.standard_normal(24) * 0.1
    gamma = 1.0 + rng.standard_normal(C) * 0.05
    fkw = dict(hc_norm_eps=EPS, rmsnorm_eps=EPS, hc_post_scale=S, sinkhorn_eps=EPS, with_mxfp8=True)
    got = O.post_int8_pre_fused(x, q, np.ldexp(1.0, k), cf, phi, bias, gamma, **fkw)
    want = O.post_pre_fused(x, np.ldexp(q.astype(np.float64), k[:, None]), cf, phi, bias, gamma, **fkw)
    for key in want:
        assert np.array_equal(got[key], want[key]), key
    _, pw, res = O.split_coeffs(cf)
    assert np.array_equal(got["x_out"], O.post_int8(x, q, np.ldexp(1.0, k), pw, res))
