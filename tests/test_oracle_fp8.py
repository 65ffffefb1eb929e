"""Pins of the oracle's fp8 codec: OCP E4M3 codes with one fp32 scale per 256
values (CPU only).

Source: gpubridge README "Bridge compression" (OCP E4M3; one scale per 256
values; about 3.9x fewer bytes than fp32; one significant digit relative to
the block's largest value).  Pinned against torch's float8_e4m3fn decode and
saturating cast, exact rational brute force and the format's closed forms.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import exactfp as X

LOW_PATTERNS = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)


def _torch_e4m3_sat(x):
    t = torch.clamp(torch.from_numpy(x), -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _check_chunk(u):
    x = u.view(np.float32)
    keep = ~np.isnan(x)
    return int((O.e4m3_encode(x)[keep] != _torch_e4m3_sat(x)[keep]).sum())


def test_all_256_codes_decode_like_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (ours[~nan].view(np.uint32) == ref[~nan].view(np.uint32)).all()
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    for c in range(256):
        v = X.e4m3_value(c)
        if v is not None:
            assert Fraction(float(ours[c])) == v


def test_every_upper_half_with_every_rounding_class():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    rng = np.random.default_rng(6)
    lows = np.concatenate([LOW_PATTERNS, rng.integers(0, 1 << 16, 10).astype(np.uint32)])
    u = (hi[:, None] | lows[None, :]).ravel()
    assert _check_chunk(u) == 0


@pytest.mark.exhaustive
def test_all_2_32_patterns_match_torch():
    chunk = 1 << 25

    def run(i):
        u = np.arange(i * chunk, (i + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        return _check_chunk(u)

    with ThreadPoolExecutor(max_workers=os.cpu_count() or 4) as ex:
        bad = sum(ex.map(run, range((1 << 32) // chunk)))
    assert bad == 0


def test_midpoints_go_to_even_code():
    vals = [X.e4m3_value(c) for c in range(0x7F)]
    mids, want_even, below, above = [], [], [], []
    for c in range(0x7E):
        m = (vals[c] + vals[c + 1]) / 2
        mf = np.float32(float(m))
        assert Fraction(float(mf)) == m
        mids.append(mf)
        want_even.append(c if c % 2 == 0 else c + 1)
        below.append(c)
        above.append(c + 1)
    mids = np.array(mids, dtype=np.float32)
    assert O.e4m3_encode(mids).tolist() == want_even
    assert O.e4m3_encode(np.nextafter(mids, np.float32(0))).tolist() == below
    assert O.e4m3_encode(np.nextafter(mids, np.float32(np.inf))).tolist() == above
    assert O.e4m3_encode(-mids).tolist() == [c | 0x80 for c in want_even]


def test_saturation_zero_and_nan():
    x = np.array([448, 449, 463.99, 464, 480, 1e30, np.inf, -np.inf, -464,
                  0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -149], dtype=np.float32)
    assert O.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE,
                                         0x00, 0x80, 0x00, 0x02, 0x00]
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    nan[1] = -abs(nan[1])
    assert O.e4m3_encode(nan).tolist() == [0x7F, 0xFF]


def test_brute_force_nearest_code():
    rng = np.random.default_rng(7)
    mags = 2.0 ** rng.uniform(-14, 9.2, 4000)
    x = (mags * rng.choice([-1, 1], 4000)).astype(np.float32)
    ours = O.e4m3_encode(x)
    for xi, ci in zip(x, ours):
        assert ci == X.e4m3_nearest(float(xi), xi < 0 or (xi == 0 and np.signbit(xi)))


def test_absmax_ignores_nan_and_order():
    rng = np.random.default_rng(8)
    for _ in range(50):
        blk = (rng.standard_normal(256) * 10.0 ** rng.integers(-5, 5)).astype(np.float32)
        blk[rng.integers(0, 256, 3)] = np.nan
        a = O.block_absmax(blk)
        finite = blk[~np.isnan(blk)]
        assert a == np.abs(finite).max()
        for _ in range(5):
            assert O.block_absmax(rng.permutation(blk)).view(np.uint32) == a.view(np.uint32)
    assert O.block_absmax(np.full(7, -0.0, np.float32)).view(np.uint32) == 0
    assert O.block_absmax(np.full(7, np.nan, np.float32)) == 0
    assert O.block_absmax(np.array([1.0, -np.inf], np.float32)) == np.inf


def test_absmax_scale_puts_block_max_on_448():
    rng = np.random.default_rng(12)
    for _ in range(2000):
        e = int(rng.integers(-118, 120))
        blk = (rng.standard_normal(256) * 2.0 ** e).astype(np.float32)
        a = O.block_absmax(blk)
        if not np.isfinite(a) or a < 448 * 2.0 ** -126:
            continue
        s = O.block_scale(a, O.SCALE_ABSMAX_DIV_448)
        assert s == X.div_f32(float(a), 448.0)
        i = int(np.argmax(np.abs(blk)))
        assert O.fp8_quantize_one(blk[i], s) & 0x7F == 0x7E
    assert O.block_scale(0.0, O.SCALE_ABSMAX_DIV_448) == 0.0
    assert O.block_scale(np.inf, O.SCALE_ABSMAX_DIV_448) == np.inf


def test_pow2_scale_is_the_smallest_power_that_fits():
    rng = np.random.default_rng(13)
    u = rng.integers(1, 0x7F800000, 5000, dtype=np.uint64).astype(np.uint32)
    for a in u.view(np.float32):
        s = O.block_scale(a, O.SCALE_POW2)
        fa, fs = Fraction(float(a)), Fraction(float(s))
        e = math.frexp(float(s))[1] - 1
        assert fs == Fraction(2) ** e  # a power of two
        assert fa <= 448 * fs
        assert e == -149 or fa > 448 * fs / 2  # the smallest such power
    assert O.block_scale(0.0, O.SCALE_POW2) == 1.0
    assert O.block_scale(448.0, O.SCALE_POW2) == 1.0
    assert O.block_scale(np.float32(448.00003), O.SCALE_POW2) == 2.0
    assert O.block_scale(2.0 ** -149, O.SCALE_POW2) == np.float32(2.0 ** -149)
    assert O.block_scale(np.inf, O.SCALE_POW2) == np.inf


def test_quantize_matches_exact_division_then_nearest_code():
    rng = np.random.default_rng(14)
    for _ in range(3000):
        s = np.float32(2.0 ** rng.uniform(-140, 100))
        if rng.random() < 0.3:
            s = np.float32(2.0 ** int(rng.integers(-149, 120)))
        x = np.float32(float(s) * rng.uniform(-448, 448) * 2.0 ** -rng.integers(0, 14))
        if not np.isfinite(x):
            continue
        v = X.div_f32(float(x), float(s))
        want = X.e4m3_nearest(v, bool(np.signbit(x)))
        assert O.fp8_quantize_one(x, s) == want, (x, s)
    # zero block with absmax scale: quotient step skipped, codes keep the sign
    assert O.fp8_quantize_one(np.float32(0.0), np.float32(0.0)) == 0x00
    assert O.fp8_quantize_one(np.float32(-0.0), np.float32(0.0)) == 0x80
    # an Inf in a block gives an Inf scale: Inf / Inf is NaN, finite / Inf is 0
    assert O.fp8_quantize_one(np.float32(-np.inf), np.float32(np.inf)) == 0xFF
    assert O.fp8_quantize_one(np.float32(3.0), np.float32(np.inf)) == 0x00


def test_block_layout_partial_tail_and_payload_ratio():
    rng = np.random.default_rng(15)
    n = 256 * 3 + 17
    x = rng.standard_normal(n).astype(np.float32)
    x[256:512] *= 1000
    codes, scales = O.encode_fp8(x, O.SCALE_ABSMAX_DIV_448)
    assert scales.size == 4
    for b in range(4):
        blk = x[b * 256:(b + 1) * 256]
        assert scales[b] == X.div_f32(float(np.abs(blk).max()), 448.0)
        for j in range(blk.size):
            assert codes[b * 256 + j] == O.fp8_quantize_one(blk[j], scales[b])
    # one 4-byte scale per 256 one-byte codes: 1024/260 = 3.94x fewer bytes
    n = 1 << 20
    ratio = 4 * n / (n + 4 * O.nblocks(n))
    assert round(ratio, 1) == 3.9


def test_pow2_round_trip_within_half_ulp():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(256 * 64) * 10.0 ** rng.integers(-6, 6)).astype(np.float32)
    codes, scales = O.encode_fp8(x, O.SCALE_POW2)
    dec = O.decode_accumulate([codes], [scales], O.CODEC_FP8)
    for b in range(64):
        s = float(scales[b])
        v = x[b * 256:(b + 1) * 256].astype(np.float64) / s  # exact: s is 2^e
        e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
        half_ulp = 2.0 ** (e - 4) * s  # E4M3 has 3 fraction bits
        err = np.abs(dec[b * 256:(b + 1) * 256].astype(np.float64) - x[b * 256:(b + 1) * 256])
        assert (err <= half_ulp).all()
