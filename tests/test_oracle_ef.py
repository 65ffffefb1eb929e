"""Pins of the oracle's error-feedback encoders (CPU only).

Source: gpubridge README "Bridge compression" (each bridge member keeps an
error-feedback residual per buffer, so rounding error carries into the next
step).  Reading: y = x + residual is encoded, and the residual becomes y minus
what the payload decodes to.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests import exactfp as X


def test_zero_residual_gives_the_plain_payload():
    rng = np.random.default_rng(50)
    x = (rng.standard_normal(3000) * 1e-3).astype(np.float32)
    c, res = O.encode_bf16_ef(x, np.zeros_like(x))
    assert (c == O.encode_bf16(x)).all()
    for mode in (0, 1):
        c8, s8, _ = O.encode_fp8_ef(x, np.zeros_like(x), mode)
        wc, ws = O.encode_fp8(x, mode)
        assert (c8 == wc).all() and (s8.view(np.uint32) == ws.view(np.uint32)).all()


def test_bf16_residual_is_exact_and_within_half_an_ulp():
    rng = np.random.default_rng(51)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    r0 = (rng.standard_normal(20000) * 1e-3 * np.abs(x)).astype(np.float32)
    c, res = O.encode_bf16_ef(x, r0)
    y = (x + r0)  # float32 add, the same rounding as the oracle's
    dec = (c.astype(np.uint32) << 16).view(np.float32)
    # the residual is y - dec exactly (binary64 holds both and their difference)
    assert (res.astype(np.float64) == y.astype(np.float64) - dec.astype(np.float64)).all()
    e = np.floor(np.log2(np.abs(y.astype(np.float64))))
    assert (np.abs(res.astype(np.float64)) <= 2.0 ** (np.maximum(e, -126) - 8)).all()


@pytest.mark.parametrize("codec,mode", [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)])
def test_running_mean_of_decoded_values_converges_to_the_input(codec, mode):
    """With the same input every step, the residual stays bounded, so the mean
    of the decoded values over T steps is within max|residual| / T of x.  A
    wrong sign or a dropped feedback term makes the error stay at the size of
    one rounding (or grow)."""
    rng = np.random.default_rng(52)
    x = (rng.standard_normal(256 * 8) * 1e-3).astype(np.float32)
    res = np.zeros_like(x)
    total = np.zeros(x.size)
    T = 200
    worst_res = 0.0
    for _ in range(T):
        if codec == O.CODEC_BF16:
            c, res = O.encode_bf16_ef(x, res)
            dec = O.decode_accumulate([c], None, O.CODEC_BF16)
        else:
            c, s, res = O.encode_fp8_ef(x, res, mode)
            dec = O.decode_accumulate([c], [s], O.CODEC_FP8)
        total += dec.astype(np.float64)
        worst_res = max(worst_res, float(np.abs(res).max()))
    err = np.abs(total / T - x.astype(np.float64))
    # bound: max residual / T, plus binary32 roundings of y = x + res
    assert (err <= worst_res / T + T * 2.0 ** -23 * np.abs(x) / T + 1e-12).all()
    # and the plain (no feedback) encoder does much worse on the same data
    if codec == O.CODEC_FP8:
        c, s = O.encode_fp8(x, mode)
        plain = np.abs(O.decode_accumulate([c], [s], O.CODEC_FP8).astype(np.float64) - x)
        assert plain.max() > 20 * err.max()


def _exact_step_bf16(x, r):
    y = X.add_f32(x, r)
    code_val = X.bf16_round(y)
    return code_val, X.round_f32(Fraction(y) - Fraction(code_val))


def test_bf16_exact_rational_steps():
    rng = np.random.default_rng(53)
    x = (rng.standard_normal(400) * 10.0 ** rng.integers(-8, 8, 400)).astype(np.float32)
    res = np.zeros_like(x)
    want_res = [0.0] * x.size
    for step in range(3):
        c, res = O.encode_bf16_ef(x, res)
        for i in range(x.size):
            val, want_res[i] = _exact_step_bf16(float(x[i]), want_res[i])
            got_val = float(np.array([int(c[i]) << 16], np.uint32).view(np.float32)[0])
            assert got_val == val, (step, i)
            assert float(res[i]) == want_res[i], (step, i)


def test_fp8_exact_rational_steps():
    """One block per step, every rounding done with exact rationals and the
    E4M3 code found by brute force over the format's values."""
    rng = np.random.default_rng(54)
    x = (rng.standard_normal(256) * 1e-2).astype(np.float32)
    res = np.zeros_like(x)
    want_res = [0.0] * 256
    for step in range(3):
        c, s, res = O.encode_fp8_ef(x, res, O.SCALE_ABSMAX_DIV_448)
        y = [X.add_f32(float(x[i]), want_res[i]) for i in range(256)]
        a = max(abs(v) for v in y)
        scale = X.div_f32(a, 448.0)
        assert float(s[0]) == scale
        for i in range(256):
            q = X.div_f32(y[i], scale)
            code = X.e4m3_nearest(q, y[i] < 0 or (y[i] == 0 and np.signbit(np.float32(y[i]))))
            assert int(c[i]) == code, (step, i)
            dec = X.mul_f32(float(X.e4m3_value(code)), scale)
            want_res[i] = X.round_f32(Fraction(y[i]) - Fraction(dec))
            assert float(res[i]) == want_res[i], (step, i)


@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
def test_bucket_stream_with_feedback_equals_per_rank_encodes(codec):
    rng = np.random.default_rng(55)
    k, n, bucket = 3, 256 * 9 + 100, 256 * 4
    xs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(k)]
    rs = [(rng.standard_normal(n) * 1e-6).astype(np.float32) for _ in range(k)]
    out, codes, scales, new_res = O.bucket_allreduce_ef(xs, rs, bucket, codec, 0)
    enc = []
    for r in range(k):
        if codec == O.CODEC_BF16:
            c, nr = O.encode_bf16_ef(xs[r], rs[r])
            enc.append((c, None))
        else:
            c, s, nr = O.encode_fp8_ef(xs[r], rs[r], 0)
            enc.append((c, s))
            assert (scales[r].view(np.uint32) == s.view(np.uint32)).all()
        assert (codes[r] == c).all()
        assert (new_res[r].view(np.uint32) == nr.view(np.uint32)).all()
    want = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc] if codec == O.CODEC_FP8 else None, codec)
    assert (out.view(np.uint32) == want.view(np.uint32)).all()
