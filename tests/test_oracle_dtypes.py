"""Pins of the oracle's reductions over the README's other element types
(float16, bfloat16, float64, int8, uint8, int32, int64), CPU only.

Pinned against torch's CPU half and bfloat16 arithmetic (each add and divide
correctly rounded to the type), exact rational rounding, Python's correctly
rounded Fraction-to-float conversion, and numpy's wrapping integer adds.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import exactfp as X

TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}


def as_torch16(codes, dt):
    return torch.from_numpy(codes.view(np.int16).copy()).view(TORCH16[dt])


def codes_of(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def random_codes(rng, n, dt):
    u = rng.integers(0, 1 << 16, n).astype(np.uint16)
    return u


def same16(got, want, dt):
    """Compare 16-bit codes; NaN codes compare as NaN."""
    g = as_torch16(got, dt).float().numpy()
    w = as_torch16(want, dt).float().numpy()
    gn, wn = np.isnan(g), np.isnan(w)
    assert (gn == wn).all()
    assert (got[~gn] == want[~wn]).all()


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_half_sum_matches_torch_on_every_first_operand(dt):
    rng = np.random.default_rng(70)
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for _ in range(8):
        b = random_codes(rng, a.size, dt)
        got = O.reduce_typed([a, b], dt, O.OP_SUM)
        want = codes_of(as_torch16(a, dt) + as_torch16(b, dt))
        same16(got, want, dt)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_half_fold_and_average_match_torch(dt):
    rng = np.random.default_rng(71)
    k, n = 4, 50000
    xs = [random_codes(rng, n, dt) for _ in range(k)]
    acc = as_torch16(xs[0], dt)
    for x in xs[1:]:
        acc = acc + as_torch16(x, dt)
    same16(O.reduce_typed(xs, dt, O.OP_SUM), codes_of(acc), dt)
    same16(O.reduce_typed(xs, dt, O.OP_AVG, 12), codes_of(acc / 12), dt)


def test_f16_exact_rational_rounding():
    rng = np.random.default_rng(72)
    a = random_codes(rng, 3000, "f16")
    b = random_codes(rng, 3000, "f16")
    got = O.reduce_typed([a, b], "f16", O.OP_SUM)
    va = as_torch16(a, "f16").double().numpy()
    vb = as_torch16(b, "f16").double().numpy()
    vg = as_torch16(got, "f16").double().numpy()
    for i in range(a.size):
        if not (np.isfinite(va[i]) and np.isfinite(vb[i])):
            continue
        want = X.round_to_format(Fraction(float(va[i])) + Fraction(float(vb[i])), 11, -14, 15)
        want = float(want)
        assert vg[i] == want or (want == 0 and vg[i] == 0), (va[i], vb[i], vg[i], want)


def test_f64_sum_and_average_are_correctly_rounded_folds():
    rng = np.random.default_rng(73)
    xs = [rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000) for _ in range(3)]
    s = O.reduce_typed(xs, "f64", O.OP_SUM)
    a = O.reduce_typed(xs, "f64", O.OP_AVG, 7)
    for i in range(2000):
        acc = float(xs[0][i])
        for x in xs[1:]:
            acc = float(Fraction(acc) + Fraction(float(x[i])))  # Fraction -> float rounds correctly
        assert s[i] == acc
        assert a[i] == float(Fraction(acc) / 7)


@pytest.mark.parametrize("dt", ["i8", "u8", "i32", "i64"])
def test_integer_sums_wrap_like_numpy(dt):
    rng = np.random.default_rng(74)
    nt = O.NP_DTYPES[dt]
    info = np.iinfo(nt)
    xs = [rng.integers(info.min, info.max, 5000, dtype=nt, endpoint=True) for _ in range(5)]
    got = O.reduce_typed(xs, dt, O.OP_SUM)
    want = xs[0].copy()
    for x in xs[1:]:
        want = want + x  # numpy wraps on overflow for fixed-width arrays
    assert (got == want).all()
    assert (O.reduce_typed(xs, dt, O.OP_MAX) == np.max(xs, axis=0)).all()
    assert (O.reduce_typed(xs, dt, O.OP_MIN) == np.min(xs, axis=0)).all()


@pytest.mark.parametrize("dt", ["f16", "bf16", "f64"])
def test_float_max_min_with_zeros_and_nan(dt):
    rng = np.random.default_rng(75)
    pool = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 2.5, -2.5])
    k, n = 3, 2000
    vals = [pool[rng.integers(0, pool.size, n)] for _ in range(k)]
    if dt == "f64":
        xs = vals
        dec = lambda a: a
    else:
        xs = [codes_of(torch.from_numpy(v).to(TORCH16[dt])) for v in vals]
        dec = lambda a: as_torch16(a, dt).double().numpy()
    for op in (O.OP_MAX, O.OP_MIN):
        got = dec(O.reduce_typed(xs, dt, op))
        for i in range(n):
            col = [v[i] for v in vals]
            if any(np.isnan(c) for c in col):
                assert np.isnan(got[i])
                continue
            best = col[0]
            for c in col[1:]:
                better = c > best if op == O.OP_MAX else c < best
                tie_zero = c == best == 0 and (np.signbit(c) == (op == O.OP_MIN)) and np.signbit(best) != np.signbit(c)
                if better or tie_zero:
                    best = c
            assert got[i] == best and np.signbit(got[i]) == np.signbit(best), (i, col, got[i])
