"""The INT8 append's fast-path decision rule, modelled on the CPU.

The append kernel estimates the biased code x / scale + 128 as
fma(x, rcp(scale), 128) with the hardware reciprocal and lets the byte
conversion round it; it falls back to IEEE division where the estimate lies
within 2^-14 of a half-integer, and for every element of a row whose scale is
subnormal (absmax below 127 * 2^-126). This file models that arithmetic in
exact rational arithmetic rounded to fp32 (the reciprocal correctly rounded and
one ulp to either side, covering the hardware's 1-ulp error) and checks the
rule against the oracle's codes across the subnormal-scale boundary, where
the reciprocal alone fails. It is a model of the kernel's steps, kept in the
tests; the oracle knows nothing of it.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle

HEAD_DIM = 128
MARGIN = np.float32(0.5) - np.float32(2.0 ** -14)


def _f32(fr):
    """Round a Fraction to the nearest fp32 value (ties to even, subnormals kept)."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    fr = abs(fr)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1                                    # now 2^e <= fr < 2^(e+1)
    q = max(e - 23, -149)
    n = round(fr / Fraction(2) ** q)              # round half to even on a Fraction
    return np.float32(sign * float(n * Fraction(2) ** q))


def _fma_plus_128(x, r):
    """fp32 fma(x, r, 128): the exact x * r + 128, rounded once."""
    if not np.isfinite(r):
        if x == 0:
            return np.float32(np.nan)
        return np.float32(np.inf if (x > 0) == (r > 0) else -np.inf)
    return _f32(Fraction(float(x)) * Fraction(float(r)) + 128)


def _cvt_u8(v):
    """The byte conversion: round half to even, saturate to [0, 255], NaN -> 0."""
    if np.isnan(v):
        return 0
    return int(np.clip(np.rint(v), 0, 255))


def kernel_model(x_row, rcp_ulps=0, tiny_switch=True):
    """Codes and scale of one 128-value row as the kernel forms them."""
    x = np.asarray(x_row, dtype=np.float32)
    a = np.max(np.abs(x))
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        scale = np.float32(a) / np.float32(127.0)            # IEEE fp32 division
        tiny = tiny_switch and scale != 0 and scale < np.float32(2.0 ** -126)
        if scale == 0 or tiny:
            rcp = np.float32(0.0)
        else:
            rcp = np.float32(1.0) / scale                      # correctly rounded, may overflow
            for _ in range(abs(rcp_ulps)):
                rcp = np.nextafter(rcp, np.float32(np.inf if rcp_ulps > 0 else 0.0), dtype=np.float32)
        v = [_fma_plus_128(xi, rcp) for xi in x]
        near = [tiny or (np.isfinite(vi) and abs(vi - np.rint(vi)) >= MARGIN) for vi in v]
        if any(near):
            for i, xi in enumerate(x):
                if near[i]:
                    q = np.float32(xi) / scale                 # IEEE fp32 division
                    v[i] = np.float32(min(max(np.rint(q), -127.0), 127.0) + 128.0)
    codes = np.array([(_cvt_u8(vi) ^ 0x80) for vi in v], dtype=np.uint8).view(np.int8)
    return codes, scale


def _rows_at_exponents(exps, seed):
    """One row per exponent e: absmax exactly 2^e, with halves, quarters,
    zeros, negatives and random values on the bf16 grid below it."""
    rng = np.random.default_rng(seed)
    rows = []
    for e in exps:
        a = 2.0 ** e
        r = rng.standard_normal(HEAD_DIM) * a / 4
        r[:6] = [a, a / 2, -a / 4, 0.0, -a, a * 0.75]
        rows.append(r)
    return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array(rows)))


def _boundary_rows():
    """Rows whose absmax puts the scale on either side of 2^-126: 127 * 2^-126
    gives scale exactly 2^-126 (normal); the bf16 values just below it give a
    subnormal scale."""
    a_norm = 127.0 * 2.0 ** -126                  # on the bf16 grid (7 significant bits)
    below = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array([a_norm])) - 1)[0]
    rows = []
    for a in (a_norm, below):
        r = np.linspace(-a, a, HEAD_DIM)
        r[0] = a
        rows.append(r)
    return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array(rows)))


def _oracle_codes(rows):
    return oracle.quantise_int8(rows)


@pytest.mark.parametrize("rcp_ulps", [-1, 0, 1])
def test_rule_matches_oracle_across_the_subnormal_scale_boundary(rcp_ulps):
    rows = np.concatenate([_rows_at_exponents(range(-133, -99), 3), _boundary_rows()])
    want_c, want_s = _oracle_codes(rows)
    for i, r in enumerate(rows):
        c, s = kernel_model(r, rcp_ulps)
        assert np.float32(s) == want_s[i], i
        assert np.array_equal(c, want_c[i]), (i, c[:6], want_c[i][:6])
        assert c.min() >= -127


def test_scale_subnormal_exactly_below_the_boundary():
    rows = _boundary_rows()
    _, s = _oracle_codes(rows)
    assert s[0] == np.float32(2.0 ** -126)
    assert 0 < s[1] < np.float32(2.0 ** -126)


def test_reciprocal_alone_fails_where_it_overflows():
    # without the subnormal-scale switch, absmax 2^-122 and below give a
    # reciprocal of infinity: positive values saturate to 127, negative ones
    # and zeros come out as -128 (outside the +-127 range)
    rows = _rows_at_exponents([-122, -126, -130], 5)
    want_c, _ = _oracle_codes(rows)
    for i, r in enumerate(rows):
        c, _ = kernel_model(r, 0, tiny_switch=False)
        assert not np.array_equal(c, want_c[i])
        assert c.min() == -128
        assert list(want_c[i][:4]) in ([127, 64, -32, 0], [127, 63, -32, 0])


@pytest.mark.parametrize("rcp_ulps", [-1, 0, 1])
def test_rule_matches_oracle_on_unit_scale_rows_with_near_ties(rcp_ulps):
    # quotients next to half-integers: the 2^-14 margin sends them to the
    # division; everything else is decided by the estimate alone
    rng = np.random.default_rng(77)
    x = rng.standard_normal((12, HEAD_DIM))
    a = np.abs(x).max(axis=1)
    scale = (a / 127.0).astype(np.float32).astype(np.float64)
    k = rng.integers(-126, 126, size=x.shape) + 0.5
    near = k * scale[:, None] * (1.0 + rng.choice([-1, 1], size=k.shape) * 2.0 ** -20)
    x = np.where(rng.random(x.shape) < 0.5, near, x)
    x[np.arange(len(x)), np.argmax(np.abs(x), axis=1)] = a
    rows = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(x))
    want_c, want_s = _oracle_codes(rows)
    for i, r in enumerate(rows):
        c, s = kernel_model(r, rcp_ulps)
        assert np.float32(s) == want_s[i]
        assert np.array_equal(c, want_c[i]), i
