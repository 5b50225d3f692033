"""Plain fp64 CPU oracle for the mHC hyper-connection hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or constant with the HIP library; the two meet only at the seeded
input generator, which holds none of the method's arithmetic.

Sources.  The pages are three public pull-request threads:

* P1 "[SM80] Backport mHC fused post + int8 all-reduce; fixes #28, #29"
  (vllm-backport PR 30), section "What this fixes": the mHC post kernel can
  carry a fused sum of squares ("sqrsum") that feeds the prenorm GEMM.
* P2 "[DSv4.1] Integrate Mega-mHC from DeepGEMM" (vLLM PR 56255), review
  "Correctness findings" / "Verified OK": the residual stream has
  hc_mult = 4 routes, hidden % 1024 == 0, and the scalar vocabulary
  hc_norm_eps, rmsnorm_eps, hc_post_scale, sinkhorn_eps; the SM12x comment
  states that the prenorm GEMM takes the flattened row of width
  hc_mult * hidden.  Its "Purpose" and review name the post kernel, the
  delayed pre kernel and the fused post->pre kernel.
* P3 "[DSV4.1] Four BS=1 critical-path fixes for DSpark decode" (SGLang PR
  39301), "What changed" item 3 and "Correctness": the combine+RMSNorm
  output is written in BF16 and can be quantised to MXFP8 (UE8M0 scales)
  as an epilogue, bitwise equal to the unfused pair; "Measured and
  deliberately left out": per-token mHC statistics and Sinkhorn.

The pages print no formula and no worked example.  The formulas below are
the method this library specifies, in the pages' vocabulary; every point the
pages leave open is a numbered reading (R1..R16) stated where it is used.

Definition (all arithmetic in IEEE binary64; inputs are widened exactly from
their bf16 / fp32 values):

  x[t, i, c]  residual stream, 4 routes i, C channels (bf16 values)
  y[t, c]     sublayer output (bf16 values)
  phi[k, m]   projection, k = i*C + c (R1: route-major flatten), m = 0..23
  bias[m], gamma[c]  fp32 values

  Coeffs(x_t):
    ss    = sum_{i,c} x^2 ;  r = 1 / sqrt(ss / (4C) + hc_norm_eps)      (R2)
    d_m   = sum_k x_flat[k] * phi[k, m]
    l_m   = r * d_m + bias_m                                            (R2)
    pre_i = sigmoid(l_i),  post_j = hc_post_scale * sigmoid(l_{4+j})    (R4)
    M_ji  = exp(l_{8+4j+i})  (row j = output route, no max shift: R6)
    repeat sinkhorn_iters times: divide each row j by (row sum + eps_sk),
      then each column i by (column sum + eps_sk)                        (R5)
    coeffs = [pre_0..3, post_0..3, M row-major]  (24 values per token)
  Pre(x_t, pre, gamma):
    g_c = sum_i pre_i x[i, c];  h_c = g_c / sqrt(mean_c g^2 + rmsnorm_eps)
    * gamma_c, rounded once to bf16 with round-to-nearest-even          (R9)
  Post(x_t, y_t, post, res):
    x'[j, c] = sum_i res[j, i] x[i, c] + post_j y[c], rounded to bf16; the
    value that is rounded is the binary32 chain of ``post`` (R20), pinned
    against the exact sum (``post_exact``)
  Fused:
    x' = Post(x, y, coeffs_l);  coeffs' = Coeffs(x'; phi', bias');
    h = Pre(x', pre', gamma')   (x' enters as its bf16 values: R10)
  MXFP8(h_bf16): per 32-channel block, amax = max |h|; the scale exponent e
    is the smallest integer with amax <= 448 * 2^e, clamped to [-127, 127]
    (amax = 0 gives -127) (R12, R16); scale byte = e + 127 (UE8M0);
    q = OCP e4m3fn round-to-nearest-even of h * 2^-e (R13); the scale
    bytes are stored in a linear [T, C/32] layout (R14).

Parity of every function here is pinned in ``tests/test_oracle_pins.py``
against closed forms, invariants, library routines and brute force.
"""

from __future__ import annotations

import numpy as np

N_ROUTES = 4
N_LOGITS = 24
MX_BLOCK = 32
E4M3_MAX = 448.0


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_round(a) -> np.ndarray:
    """Round binary64 values to the nearest bfloat16 value, ties to even.

    bfloat16 has 8 significant bits and the binary32 exponent range, so the
    rounding quantum of a normal value a = m * 2**e (0.5 <= m < 1) is
    2**(e - 8); below 2**-126 it is the subnormal quantum 2**-133.  Dividing
    by a power of two is exact, and ``np.round`` rounds half to even.
    Results beyond the bfloat16 range become +-inf (R11: not exercised).
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(a / q) * q
    big = np.abs(r) >= 2.0 ** 128
    if np.any(big):
        r = np.where(big, np.copysign(np.inf, r), r)
    return r


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen raw bfloat16 bit patterns (uint16) to binary64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a) -> np.ndarray:
    """Bit patterns of values that are already exact bfloat16 values."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(a, np.float64), equal_nan=True):
        raise ValueError("value is not exactly representable")
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value is not a bfloat16 value")
    return (bits >> 16).astype(np.uint16)


def e4m3_encode(v) -> np.ndarray:
    """OCP e4m3fn code of each value, round-to-nearest-even (R13).

    e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
    infinity, code 0x7F/0xFF is NaN, largest finite value 448 = 1.75 * 2**8.
    A value a = m * 2**e (0.5 <= m < 1) has 4 significant bits, so its
    quantum is 2**(e - 4); below the smallest normal 2**-6 the quantum is the
    subnormal step 2**-9.  Inputs must satisfy |v| <= 448 (the scale rule
    guarantees it); larger inputs raise instead of saturating.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3 input out of range")
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e - 4, -9))
    val = np.round(a / step) * step            # rounded magnitude
    if np.any(val > E4M3_MAX):
        raise ValueError("e4m3 rounding overflow")
    # encode the rounded magnitude
    sub = val < 2.0 ** -6
    m2, e2 = np.frexp(np.where(sub, 1.0, val))  # val = m2 * 2**e2
    E = e2 - 1                                   # val = (2*m2) * 2**E, 1 <= 2*m2 < 2
    frac = np.round((2.0 * m2 - 1.0) * 8.0)      # exact: 3 mantissa bits
    normal_code = (E + 7) * 8 + frac
    sub_code = val / 2.0 ** -9                   # 0..7 (8 would be the smallest normal)
    code = np.where(sub, sub_code, normal_code).astype(np.int64)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Value of OCP e4m3fn codes (NaN codes decode to NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    fr = c & 0x7
    mag = np.where(ex == 0, fr * 2.0 ** -9, (1.0 + fr / 8.0) * np.ldexp(1.0, ex - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


# ----------------------------------------------------------------------------
# The method
# ----------------------------------------------------------------------------

def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def sinkhorn(m, iters: int, eps: float) -> np.ndarray:
    """Sinkhorn-Knopp on positive [..., 4, 4] matrices (R5).

    One iteration divides every row by (its sum + eps) and then every column
    by (its sum + eps); the result is taken after the last column pass.
    Rows are the first matrix axis (j, the output route).
    """
    m = np.array(m, dtype=np.float64, copy=True)
    for _ in range(iters):
        m = m / (m.sum(axis=-1, keepdims=True) + eps)   # row j: sum over i
        m = m / (m.sum(axis=-2, keepdims=True) + eps)   # column i: sum over j
    return m


def coeffs(x, phi, bias, *, hc_norm_eps, hc_post_scale, sinkhorn_eps,
           sinkhorn_iters=20) -> np.ndarray:
    """Per-token coefficients [T, 24] = [pre(4), post(4), res(4x4 row-major)].

    x [T, 4, C] (bf16 values), phi [4C, 24], bias [24].  The RMS scale of the
    flattened 4C row multiplies the projection before the bias (R2); the
    flattening is route-major, k = i*C + c (R1).  See the module docstring.
    """
    x = np.asarray(x, dtype=np.float64)
    T, n, C = x.shape
    assert n == N_ROUTES
    phi = np.asarray(phi, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    assert phi.shape == (n * C, N_LOGITS) and bias.shape == (N_LOGITS,)
    xf = x.reshape(T, n * C)                       # k = i*C + c
    ss = np.sum(xf * xf, axis=1)
    r = 1.0 / np.sqrt(ss / (n * C) + hc_norm_eps)
    d = xf @ phi                                   # 24 dot products of length 4C
    logit = r[:, None] * d + bias[None, :]
    pre = _sigmoid(logit[:, 0:4])
    post = hc_post_scale * _sigmoid(logit[:, 4:8])
    m = np.exp(logit[:, 8:24]).reshape(T, 4, 4)    # m[t, j, i]
    res = sinkhorn(m, sinkhorn_iters, sinkhorn_eps)
    return np.concatenate([pre, post, res.reshape(T, 16)], axis=1)


def pre(x, pre_w, gamma, *, rmsnorm_eps) -> np.ndarray:
    """Combine the routes with pre, RMSNorm with gamma, one bf16 rounding (R9).

    x [T, 4, C], pre_w [T, 4], gamma [C]; returns bf16 values [T, C].
    """
    x = np.asarray(x, dtype=np.float64)
    pre_w = np.asarray(pre_w, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    T, n, C = x.shape
    g = np.zeros((T, C))
    for i in range(n):
        g = g + pre_w[:, i, None] * x[:, i, :]
    rh = 1.0 / np.sqrt(np.mean(g * g, axis=1) + rmsnorm_eps)
    return bf16_round(g * rh[:, None] * gamma[None, :])


def f32_round(a) -> np.ndarray:
    """Round binary64 values to binary32, ties to even (numpy's cast)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def fma_f32(a, b, c) -> np.ndarray:
    """Single-rounding binary32 fused multiply-add round(a*b + c), emulated exactly.

    a, b, c are binary32 values held in binary64.  a*b has at most 48
    significant bits, so it is exact in binary64.  TwoSum then gives the exact
    sum p + c = s + err.  Rounding s to binary32 equals rounding the exact sum
    except when s lies exactly halfway between two binary32 values (binary32
    midpoints are binary64 values, and |err| is below half a binary64 ulp of
    s); in that case the sign of err decides, and a zero err keeps the tie to
    even.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    p = a * b
    s = p + c
    bp = s - c
    err = (p - bp) + (c - (s - bp))
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    # neighbours of s in binary32 and the tie test
    other = np.where(r64 > s, np.nextafter(r, np.float32(-np.inf)),
                     np.nextafter(r, np.float32(np.inf))).astype(np.float64)
    tie = (r64 != s) & (np.abs(r64 - s) == np.abs(other - s))
    up_needed = tie & (err > 0) & (other > r64) | tie & (err < 0) & (other < r64)
    return np.where(up_needed, other, r64)


def post_exact(x, y, post_w, res) -> np.ndarray:
    """The plain definition of Post: the exact sum rounded once to bf16.

    x'[t, j, c] = sum_i res[t, j, i] x[t, i, c] + post_w[t, j] y[t, c] in
    binary64, then bf16.  Used to pin ``post``.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    post_w = np.asarray(post_w, dtype=np.float64)
    res = np.asarray(res, dtype=np.float64)
    T, n, C = x.shape
    out = np.empty_like(x)
    for j in range(n):
        acc = post_w[:, j, None] * y
        for i in range(n):
            acc = acc + res[:, j, i, None] * x[:, i, :]
        out[:, j, :] = acc
    return bf16_round(out)


def post(x, y, post_w, res) -> np.ndarray:
    """Post with its bf16 rounding decided in binary32 (R20).

    x' is stored in bf16 and is the input of the next layer's coefficients,
    so the value that is rounded is fixed to the binary32 sequence
        acc = f32(post_j * y);  acc = fma_f32(res[j, i], x_i, acc) for i = 0..3
    and x' = bf16(acc).  It differs from ``post_exact`` by at most one bf16
    step, and only where the exact sum lies within binary32 rounding of a
    bf16 midpoint.  post_w and res must hold binary32 values.
    x [T, 4, C], y [T, C], post_w [T, 4], res [T, 4, 4] (row j = output
    route); returns bf16 values [T, 4, C].
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    post_w = np.asarray(post_w, dtype=np.float64)
    res = np.asarray(res, dtype=np.float64)
    if not (np.array_equal(f32_round(post_w), post_w) and np.array_equal(f32_round(res), res)):
        raise ValueError("post weights must be binary32 values")
    T, n, C = x.shape
    out = np.empty_like(x)
    for j in range(n):
        acc = f32_round(post_w[:, j, None] * y)
        for i in range(n):
            acc = fma_f32(np.broadcast_to(res[:, j, i, None], x[:, i, :].shape), x[:, i, :], acc)
        out[:, j, :] = acc
    return bf16_round(out)


def post_int8(x, y_q, y_scale, post_w, res) -> np.ndarray:
    """Post of a sublayer output that arrives as int8 codes with one binary32
    scale per token ([P1] "What this fixes": the int8 all-reduce hands the
    post kernel int8 values and per-token scales, and the post consumes them
    directly).  Reading R22: the dequantised value is the binary32 product
    y[t, c] = f32(y_q[t, c] * y_scale[t]), which then enters ``post``'s
    binary32 chain in place of the bf16 y.
    x [T, 4, C] bf16 values, y_q [T, C] integers in [-128, 127], y_scale [T]
    binary32 values; returns bf16 values [T, 4, C].
    """
    return post(x, dequant_int8(y_q, y_scale), post_w, res)


def dequant_int8(y_q, y_scale) -> np.ndarray:
    """R22: y[t, c] = f32(y_q[t, c] * y_scale[t]) for int8 codes and binary32
    per-token scales."""
    q = np.asarray(y_q)
    if not np.issubdtype(q.dtype, np.integer) or (q.size and (q.min() < -128 or q.max() > 127)):
        raise ValueError("y_q must hold int8 values")
    sc = np.asarray(y_scale, dtype=np.float64)
    if not np.array_equal(f32_round(sc), sc):
        raise ValueError("y_scale must hold binary32 values")
    # an int8 times a binary32 value is exact in binary64 (8 + 24 bits), so
    # one rounding to binary32 gives the IEEE binary32 product
    return f32_round(q.astype(np.float64) * sc[:, None])


def split_coeffs(cf):
    """Views of a packed [T, 24] coefficient array: pre [T,4], post [T,4], res [T,4,4]."""
    cf = np.asarray(cf, dtype=np.float64)
    return cf[:, 0:4], cf[:, 4:8], cf[:, 8:24].reshape(-1, 4, 4)


def mxfp8_scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2**e, clamped to [-127, 127] (R12, R16)."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    guess = np.ceil(np.log2(np.where(nz, amax, 1.0) / E4M3_MAX)).astype(np.int64)
    # exact correction of the floating-point guess: both tests are exact in binary64
    for _ in range(2):
        up = nz & (amax > E4M3_MAX * np.ldexp(1.0, guess))
        guess = np.where(up, guess + 1, guess)
        down = nz & (amax <= E4M3_MAX * np.ldexp(1.0, guess - 1))
        guess = np.where(down, guess - 1, guess)
    e = np.where(nz, guess, e)
    return np.clip(e, -127, 127)


def mxfp8(h_bf16):
    """MXFP8 encoding of bf16 values h [T, C] (C % 32 == 0).

    Returns (q [T, C] uint8 e4m3fn codes, scale [T, C/32] uint8 UE8M0 bytes).
    """
    h = np.asarray(h_bf16, dtype=np.float64)
    T, C = h.shape
    assert C % MX_BLOCK == 0
    blk = h.reshape(T, C // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blk), axis=2)
    e = mxfp8_scale_exponent(amax)
    scaled = blk * np.ldexp(1.0, -e)[:, :, None]     # exact: power-of-two scaling
    q = e4m3_encode(scaled).reshape(T, C)
    scale = (e + 127).astype(np.uint8)
    return q, scale


def mxfp8_scales_mfma(scale) -> np.ndarray:
    """UE8M0 scale bytes [T, C/32] in the operand order of the gfx950
    MX-scaled matrix instruction that a consumer GEMM with h as its A matrix
    reads them in (reading R23 of the pages' "swizzled UE8M0 scale block",
    [P3] "Correctness": the layout belongs to the consumer's matrix
    instruction; here v_mfma_scale_f32_16x16x128_f8f6f4, whose lane l holds
    row l % 16 and the 32-channel K-block l / 16 of a 128-channel K-tile and
    reads its scale from one byte of a 32-bit register).

    Layout [ceil(T/16)][C/512][64][4]: byte ((rb * C/512 + kg) * 64 + l) * 4
    + b is the scale of token 16 rb + l % 16 and block 16 kg + 4 b + l / 16;
    rows past T are the bytes of all-zero blocks (0).  A pure permutation of
    the linear bytes plus that padding.
    """
    s = np.asarray(scale, dtype=np.uint8)
    T, nb = s.shape
    assert nb % 16 == 0, "C must be a multiple of 512"
    tp = (T + 15) // 16 * 16
    pad = np.zeros((tp, nb), dtype=np.uint8)
    pad[:T] = s
    # [rb][r][kg][b][lb]  ->  [rb][kg][lb][r][b]   (lane l = 16 lb + r)
    return pad.reshape(tp // 16, 16, nb // 16, 4, 4).transpose(0, 2, 4, 1, 3).reshape(-1).copy()


def post_pre_fused(x, y, coeffs_in, phi_next, bias_next, gamma_next, *,
                   hc_norm_eps, rmsnorm_eps, hc_post_scale, sinkhorn_eps,
                   sinkhorn_iters=20, with_mxfp8=False):
    """The fused pass: post with this layer's coefficients, then the next pre.

    Returns a dict with x_out [T,4,C] (bf16 values), coeffs_next [T,24],
    h [T,C] (bf16 values) and, with ``with_mxfp8``, h_fp8 / h_scale.
    """
    _, post_w, res = split_coeffs(coeffs_in)
    x_out = post(x, y, post_w, res)          # R20: binary32 rounding decision
    cn = coeffs(x_out, phi_next, bias_next, hc_norm_eps=hc_norm_eps,
                hc_post_scale=hc_post_scale, sinkhorn_eps=sinkhorn_eps,
                sinkhorn_iters=sinkhorn_iters)
    h = pre(x_out, cn[:, 0:4], gamma_next, rmsnorm_eps=rmsnorm_eps)
    out = {"x_out": x_out, "coeffs_next": cn, "h": h}
    if with_mxfp8:
        out["h_fp8"], out["h_scale"] = mxfp8(h)
    return out


def post_int8_pre_fused(x, y_q, y_scale, coeffs_in, phi_next, bias_next, gamma_next, **kw):
    """post_pre_fused of an int8 sublayer output with per-token scales ([P1]
    "What this fixes"): the same pass with y = dequant_int8(y_q, y_scale)."""
    return post_pre_fused(x, dequant_int8(y_q, y_scale), coeffs_in, phi_next, bias_next, gamma_next, **kw)


def pre_broadcast(x0, phi, bias, gamma, *, hc_norm_eps, rmsnorm_eps, hc_post_scale, sinkhorn_eps,
                  sinkhorn_iters=20):
    """Coefficients and pre of a first-layer input: x0 [T, C] (bf16 values)
    stands for every route ([P2] review, SM12x comment: the broadcast pre
    takes a (T, H) input), i.e. the stream x[t, i, c] = x0[t, c].  Returns
    (coeffs [T, 24], h [T, C] bf16 values): Coeffs and Pre of that stream.
    """
    x0 = np.asarray(x0, dtype=np.float64)
    T, C = x0.shape
    x = np.broadcast_to(x0[:, None, :], (T, N_ROUTES, C))
    cf = coeffs(x, phi, bias, hc_norm_eps=hc_norm_eps, hc_post_scale=hc_post_scale,
                sinkhorn_eps=sinkhorn_eps, sinkhorn_iters=sinkhorn_iters)
    h = pre(x, cf[:, 0:4], gamma, rmsnorm_eps=rmsnorm_eps)
    return cf, h


def rms(a, axis=-1):
    """Root mean square along an axis (used by the comparison metric)."""
    a = np.asarray(a, dtype=np.float64)
    return np.sqrt(np.mean(a * a, axis=axis))


__all__ = [
    "N_ROUTES", "N_LOGITS", "MX_BLOCK", "E4M3_MAX",
    "bf16_round", "bf16_bits_to_f64", "f64_to_bf16_bits", "f32_round", "fma_f32",
    "post_exact", "post_int8", "dequant_int8", "post_int8_pre_fused",
    "e4m3_encode", "e4m3_decode", "sinkhorn", "coeffs", "pre", "post",
    "split_coeffs", "mxfp8_scale_exponent", "mxfp8", "mxfp8_scales_mfma", "post_pre_fused", "pre_broadcast", "rms",
]
