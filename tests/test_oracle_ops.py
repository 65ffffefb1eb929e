"""Pins of the oracle's AVG, MAX and MIN (CPU only).

Source: gpubridge README "API" (all_reduce with SUM, AVG, MAX or MIN; AVG is
a SUM divided by the world size, identically on every rank).  MAX/MIN follow
the IEEE 754-2019 maximum/minimum (a reading: the README leaves NaN to the
backends).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests import exactfp as X


def test_avg_of_k_copies_over_k_is_the_value():
    rng = np.random.default_rng(60)
    for k in (1, 2, 4, 8):
        x = rng.integers(-2 ** 20, 2 ** 20, 1000).astype(np.float32)  # k*x stays exact
        out = O.reduce([x] * k, O.OP_AVG, k)
        assert (out.view(np.uint32) == x.view(np.uint32)).all()


def test_avg_is_the_rounded_quotient_of_the_exact_sum():
    rng = np.random.default_rng(61)
    for k, d in [(2, 2), (3, 7), (4, 12), (5, 1000)]:
        ints = rng.integers(-10 ** 6, 10 ** 6, size=(k, 500))
        xs = [a.astype(np.float32) for a in ints]
        out = O.reduce(xs, O.OP_AVG, d)
        for i in range(500):
            want = X.round_f32(Fraction(int(ints[:, i].sum()), d))
            assert float(out[i]) == want


def _max_exact(vals):
    if any(np.isnan(v) for v in vals):
        return None
    best = vals[0]
    for v in vals[1:]:
        if v > best or (v == best and v == 0 and not np.signbit(v)):
            best = v
    return best


def _min_exact(vals):
    if any(np.isnan(v) for v in vals):
        return None
    best = vals[0]
    for v in vals[1:]:
        if v < best or (v == best and v == 0 and np.signbit(v)):
            best = v
    return best


@pytest.mark.parametrize("op", [O.OP_MAX, O.OP_MIN])
def test_max_min_brute_force_with_zeros_and_nan(op):
    rng = np.random.default_rng(62)
    k, n = 4, 3000
    pool = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 3.5],
                    dtype=np.float32)
    xs = [pool[rng.integers(0, pool.size, n)] for _ in range(k)]
    out = O.reduce(xs, op)
    ref = _max_exact if op == O.OP_MAX else _min_exact
    for i in range(n):
        want = ref([x[i] for x in xs])
        if want is None:
            assert np.isnan(out[i])
        else:
            assert out[i].view(np.uint32) == np.float32(want).view(np.uint32), (i, [x[i] for x in xs])


@pytest.mark.parametrize("op", [O.OP_MAX, O.OP_MIN])
def test_max_min_do_not_depend_on_rank_order(op):
    rng = np.random.default_rng(63)
    xs = [(rng.standard_normal(2000) * 10.0 ** rng.integers(-3, 3, 2000)).astype(np.float32) for _ in range(4)]
    xs[1][:100] = 0.0
    xs[2][:100] = -0.0
    base = O.reduce(xs, op)
    for perm in itertools.permutations(range(4)):
        assert (O.reduce([xs[i] for i in perm], op).view(np.uint32) == base.view(np.uint32)).all()
    want = np.max(xs, axis=0) if op == O.OP_MAX else np.min(xs, axis=0)
    assert (base[100:] == want[100:]).all()
    zero_sign = np.signbit(base[:100])
    assert (zero_sign == (op == O.OP_MIN)).all()


def test_sum_through_reduce_is_the_plain_sum():
    rng = np.random.default_rng(64)
    xs = [rng.standard_normal(1000).astype(np.float32) for _ in range(3)]
    assert (O.reduce(xs, O.OP_SUM).view(np.uint32) == O.reduce_sum(xs).view(np.uint32)).all()
