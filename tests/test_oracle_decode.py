"""Pins of the oracle's decode-and-accumulate and bucket stream (CPU only).

Source: gpubridge README "Bridge compression" (payloads are decoded and added
in float32 after the bridge step; every rank ends with the same bits) and
"DistributedDataParallel" (one all_reduce per gradient bucket).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests import exactfp as X


def test_k1_bf16_is_the_plain_decode():
    rng = np.random.default_rng(20)
    codes = rng.integers(0, 1 << 16, 5000).astype(np.uint16)
    out = O.decode_accumulate([codes], None, O.CODEC_BF16)
    want = (codes.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(want)
    assert (out[~nan].view(np.uint32) == want[~nan].view(np.uint32)).all()
    assert np.isnan(out[nan]).all()


def test_bf16_exact_data_equals_uncompressed_sum_in_any_order():
    rng = np.random.default_rng(21)
    k, n = 4, 3000
    ints = rng.integers(-255, 256, size=(k, n))  # 8 significant bits: bf16-exact
    xs = [a.astype(np.float32) for a in ints]
    codes = [O.encode_bf16(x) for x in xs]
    out = O.decode_accumulate(codes, None, O.CODEC_BF16)
    assert (out.astype(np.int64) == ints.sum(axis=0)).all()
    for perm in itertools.permutations(range(k)):
        o2 = O.decode_accumulate([codes[i] for i in perm], None, O.CODEC_BF16)
        assert (o2.view(np.uint32) == out.view(np.uint32)).all()


def test_fp8_pow2_exact_data_equals_uncompressed_sum():
    rng = np.random.default_rng(22)
    k, n = 4, 256 * 8
    # every value a (E4M3 value) * 2^e with the block max making s = 2^e
    xs = []
    for r in range(k):
        c = rng.integers(0, 0x7F, n)
        vals = np.array([float(X.e4m3_value(int(ci))) for ci in c])
        vals[::256] = 448.0
        e = rng.integers(-20, 20, n // 256).repeat(256)
        xs.append((vals * rng.choice([-1, 1], n) * 2.0 ** e).astype(np.float32))
    enc = [O.encode_fp8(x, O.SCALE_POW2) for x in xs]
    for x, (codes, scales) in zip(xs, enc):
        assert (O.decode_accumulate([codes], [scales], O.CODEC_FP8).view(np.uint32)
                == x.view(np.uint32)).all()
    out = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8)
    assert (out.view(np.uint32) == O.reduce_sum(xs).view(np.uint32)).all()


def test_fp8_decode_is_code_value_times_scale_then_add():
    rng = np.random.default_rng(23)
    k, n = 3, 256 * 2 + 5
    xs = [rng.standard_normal(n).astype(np.float32) * np.float32(1e-3) for _ in range(k)]
    enc = [O.encode_fp8(x, O.SCALE_ABSMAX_DIV_448) for x in xs]
    out = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8)
    for i in range(0, n, 7):
        acc = None
        for codes, scales in enc:
            v = X.mul_f32(float(X.e4m3_value(int(codes[i]))), float(scales[i // 256]))
            acc = v if acc is None else X.add_f32(acc, v)
        assert X.f32_bits(acc) == int(out.view(np.uint32)[i])


def test_accumulate_starts_from_the_buffer():
    rng = np.random.default_rng(24)
    n = 1000
    acc0 = rng.integers(-100, 100, n).astype(np.float32)
    ints = rng.integers(-100, 100, size=(3, n))
    codes = [O.encode_bf16(a.astype(np.float32)) for a in ints]
    out = O.decode_accumulate(codes, None, O.CODEC_BF16, acc=acc0)
    assert (out.astype(np.int64) == acc0.astype(np.int64) + ints.sum(axis=0)).all()
    # the fp32 'codec' is the plain fold
    xs = [a.astype(np.float32) for a in ints]
    out2 = O.decode_accumulate(xs, None, O.CODEC_NONE)
    assert (out2.view(np.uint32) == O.reduce_sum(xs).view(np.uint32)).all()


@pytest.mark.parametrize("mode", [O.SCALE_ABSMAX_DIV_448, O.SCALE_POW2])
def test_error_bound_against_exact_sum(mode):
    rng = np.random.default_rng(25 + mode)
    k, n = 4, 256 * 16
    xs = []
    for _ in range(k):
        x = rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)
        idx = rng.choice(n, n // 100, replace=False)
        x[idx] *= np.float32(100)
        xs.append(x)
    enc = [O.encode_fp8(x, mode) for x in xs]
    out = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8).astype(np.float64)
    exact = np.sum([x.astype(np.float64) for x in xs], axis=0)
    bound = np.zeros(n)
    for x, (_, s) in zip(xs, enc):
        sv = np.repeat(s.astype(np.float64), 256)[:n]
        v = np.abs(x.astype(np.float64)) / sv
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
        # half an E4M3 ulp of the quotient, plus the binary32 divide and
        # multiply roundings
        bound += 2.0 ** (e - 4) * sv + 2 * 2.0 ** -24 * np.abs(x.astype(np.float64)) + 2.0 ** -24 * 448 * sv
    bound += (k - 1) * 2.0 ** -24 * (np.abs(exact) + bound)
    assert (np.abs(out - exact) <= bound).all()


@pytest.mark.parametrize("codec", [O.CODEC_NONE, O.CODEC_BF16, O.CODEC_FP8])
def test_bucket_stream_equals_whole_buffer_when_buckets_are_block_multiples(codec):
    rng = np.random.default_rng(30 + codec)
    k, n, bucket = 3, 256 * 10 + 33, 256 * 3
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(k)]
    out, codes, scales = O.bucket_allreduce(xs, bucket, codec, O.SCALE_ABSMAX_DIV_448)
    if codec == O.CODEC_NONE:
        want = O.reduce_sum(xs)
    elif codec == O.CODEC_BF16:
        whole = [O.encode_bf16(x) for x in xs]
        for a, b in zip(codes, whole):
            assert (a == b).all()
        want = O.decode_accumulate(whole, None, O.CODEC_BF16)
    else:
        whole = [O.encode_fp8(x, O.SCALE_ABSMAX_DIV_448) for x in xs]
        for a, b, (wc, ws) in zip(codes, scales, whole):
            assert (a == wc).all() and (b.view(np.uint32) == ws.view(np.uint32)).all()
        want = O.decode_accumulate([c for c, _ in whole], [s for _, s in whole], O.CODEC_FP8)
    assert (out.view(np.uint32) == want.view(np.uint32)).all()


def test_bucket_blocks_restart_at_each_bucket():
    rng = np.random.default_rng(40)
    n, bucket = 1000, 300  # not a block multiple: blocks restart at 300, 600, 900
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(2)]
    xs[0][250:260] *= 1e4  # a large run straddling a bucket edge
    out, codes, scales = O.bucket_allreduce(xs, bucket, O.CODEC_FP8, O.SCALE_ABSMAX_DIV_448)
    starts = list(range(0, n, bucket))
    nb = [O.nblocks(min(bucket, n - s)) for s in starts]
    assert scales[0].size == sum(nb)
    si = 0
    for s, b in zip(starts, nb):
        c, sc = O.encode_fp8(xs[0][s:s + bucket], O.SCALE_ABSMAX_DIV_448)
        assert (codes[0][s:s + bucket] == c).all()
        assert (scales[0][si:si + b] == sc).all()
        si += b
