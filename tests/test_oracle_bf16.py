"""Pins of the oracle's bf16 codec (CPU only).

Source: gpubridge README "Bridge compression" (bf16 payloads).  The codec is
round-to-nearest-even to bf16, pinned here against torch's float32->bfloat16
cast (a library routine with the same definition), the format's midpoints
and exact rational rounding.  The NaN rule is a convention of this library.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import exactfp as X

# Low halves that cover every rounding class below bit 16: exact, below,
# at and above the midpoint, with and without sticky bits.
LOW_PATTERNS = np.array([0x0000, 0x0001, 0x3FFF, 0x4000, 0x7FFE, 0x7FFF, 0x8000,
                         0x8001, 0x8002, 0xBFFF, 0xC000, 0xFFFE, 0xFFFF],
                        dtype=np.uint32)


def _torch_bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _check_chunk(u):
    x = u.view(np.float32)
    keep = ~np.isnan(x)
    ours = O.encode_bf16(x)
    ref = _torch_bf16(x)
    return int((ours[keep] != ref[keep]).sum())


def test_every_upper_half_with_every_rounding_class():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    rng = np.random.default_rng(5)
    lows = np.concatenate([LOW_PATTERNS, rng.integers(0, 1 << 16, 19).astype(np.uint32)])
    u = (hi[:, None] | lows[None, :]).ravel()
    assert _check_chunk(u) == 0


@pytest.mark.exhaustive
def test_all_2_32_patterns_match_torch():
    chunk = 1 << 26

    def run(i):
        u = np.arange(i * chunk, (i + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        return _check_chunk(u)

    with ThreadPoolExecutor(max_workers=os.cpu_count() or 4) as ex:
        bad = sum(ex.map(run, range((1 << 32) // chunk)))
    assert bad == 0


def test_every_code_round_trips():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = O.decode_bf16(codes)
    assert (vals.view(np.uint32) == codes.astype(np.uint32) << 16).all()
    back = O.encode_bf16(vals)
    nan = np.isnan(vals)
    assert (back[~nan] == codes[~nan]).all()
    # NaN convention: sign and top payload kept, quiet bit forced
    assert (back[nan] == (codes[nan] | 0x0040)).all()


def test_midpoints_go_to_even_code_and_neighbours_to_nearer():
    c = np.arange(0, 0x7F7F, dtype=np.uint32)  # pairs (c, c+1), finite
    lo = (c << 16).view(np.float32).astype(np.float64)
    hi = ((c + 1) << 16).view(np.float32).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: 9 significant bits
    assert ((mid.astype(np.float64)) == (lo + hi) / 2).all()
    even = np.where(c % 2 == 0, c, c + 1)
    assert (O.encode_bf16(mid) == even).all()
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert (O.encode_bf16(below) == c).all()
    assert (O.encode_bf16(above) == c + 1).all()
    assert (O.encode_bf16(-mid) == (even | 0x8000)).all()


def test_overflow_to_inf_at_the_ieee_boundary():
    maxb = np.float64(np.array([0x7F7F0000], np.uint32).view(np.float32)[0])
    half_ulp = 2.0 ** (127 - 8)
    tie = np.float32(maxb + half_ulp)  # 2^128 - 2^119... exact in float32
    assert float(tie) == maxb + half_ulp
    assert O.encode_bf16(np.array([tie]))[0] == 0x7F80  # tie, odd -> Inf
    assert O.encode_bf16(np.array([np.nextafter(tie, np.float32(0))]))[0] == 0x7F7F
    assert O.encode_bf16(np.array([np.float32(np.inf), -np.float32(np.inf)])).tolist() == [0x7F80, 0xFF80]


def test_exact_rational_rounding_on_random_values():
    rng = np.random.default_rng(9)
    u = rng.integers(0, 1 << 32, 3000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ours = O.encode_bf16(x)
    for xi, ci in zip(x, ours):
        want = X.bf16_round(float(xi))
        got = float(np.array([int(ci) << 16], np.uint32).view(np.float32)[0])
        assert got == want or (got == want == 0), (xi, got, want)
        if want == 0:
            assert (int(ci) >> 15) == (X.f32_bits(float(xi)) >> 31)


def test_half_ulp_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    d = O.decode_bf16(O.encode_bf16(x)).astype(np.float64)
    e = np.floor(np.log2(np.abs(x.astype(np.float64))))
    half_ulp = 2.0 ** (np.maximum(e, -126) - 8)
    assert (np.abs(d - x.astype(np.float64)) <= half_ulp).all()
