"""Pins of the oracle's fixed-order sum (CPU only).

Source: gpubridge README "How it works" (the leaders' sum of the island sums)
and "API" (all_reduce with SUM).  The order is a reading: a left fold over
ranks 0..k-1 from rank 0's value.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests import exactfp as X


@pytest.mark.parametrize("k", range(1, 9))
def test_k_copies_of_one_sum_to_k(k):
    xs = [np.ones(1000, dtype=np.float32) for _ in range(k)]
    out = O.reduce_sum(xs)
    assert (out == np.float32(k)).all()


def test_integer_sums_are_exact_and_order_free():
    rng = np.random.default_rng(11)
    for k in range(1, 9):
        ints = rng.integers(-1024, 1025, size=(k, 777))
        xs = [a.astype(np.float32) for a in ints]
        exact = ints.sum(axis=0)
        out = O.reduce_sum(xs)
        assert (out.astype(np.int64) == exact).all()
        # every rank permutation gives the same bits on exact data
        for perm in itertools.islice(itertools.permutations(range(k)), 24):
            out_p = O.reduce_sum([xs[i] for i in perm])
            assert (out_p.view(np.uint32) == out.view(np.uint32)).all()


def test_fold_order_is_rank_order():
    # 2^24 + 1 rounds back to 2^24 (a tie, to even), so the left fold from
    # rank 0 loses both ones; adding the ones first keeps them.
    big = np.float32(2.0 ** 24)
    one = np.float32(1.0)
    a = O.reduce_sum([np.array([big]), np.array([one]), np.array([one])])
    b = O.reduce_sum([np.array([one]), np.array([one]), np.array([big])])
    assert a[0] == big
    assert b[0] == big + 2


def test_two_ranks_commute():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000).astype(np.float32) * np.float32(1e3)
    y = rng.standard_normal(10000).astype(np.float32)
    a = O.reduce_sum([x, y])
    b = O.reduce_sum([y, x])
    assert (a.view(np.uint32) == b.view(np.uint32)).all()


def test_negative_zero_survives():
    z = np.full(5, -0.0, dtype=np.float32)
    out = O.reduce_sum([z, z, z])
    assert (out.view(np.uint32) == 0x80000000).all()


def _rand_floats(rng, n):
    """Floats spanning many binades, with subnormals and exact ties."""
    mant = rng.integers(1 << 23, 1 << 24, size=n)
    exp = rng.integers(-150, 40, size=n)
    sign = rng.choice([-1, 1], size=n)
    vals = [float(np.float32(s * float(Fraction(int(m)) * Fraction(2) ** int(e - 23))))
            for s, m, e in zip(sign, mant, exp)]
    return np.array(vals, dtype=np.float32)


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_brute_force_exact_left_fold(k):
    rng = np.random.default_rng(100 + k)
    n = 300
    xs = [_rand_floats(rng, n) for _ in range(k)]
    # plant cancellations and near-ties
    xs[0][:10] = np.float32(2.0 ** 24)
    if k > 1:
        xs[1][:10] = np.float32(1.0)
        xs[1][10:20] = -xs[0][10:20]
    out = O.reduce_sum(xs)
    for i in range(n):
        acc = float(xs[0][i])
        for r in range(1, k):
            acc = X.add_f32(acc, float(xs[r][i]))
        assert X.f32_bits(acc) == int(out.view(np.uint32)[i]), (i, acc, out[i])
