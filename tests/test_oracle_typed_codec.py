"""Pins of the oracle's bridge codecs over float16, bfloat16 and float64
arrays (README "Bridge compression": leaders quantize their island's sum, and
the payloads are dequantized and added in float32), CPU only.

Each typed function is pinned to the already-pinned binary32 path fed by an
independent conversion: torch's CPU half / bfloat16 casts and numpy's float64
to float32 cast for the inputs, torch's float32 to half / bfloat16 casts for
the total.  bfloat16 input through the bf16 codec must come out unchanged.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O

TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}


def as_f32(x, dt):
    """Values of a typed array as float32, by torch / numpy."""
    if dt in TORCH16:
        return torch.from_numpy(x.view(np.int16).copy()).view(TORCH16[dt]).float().numpy()
    return x.astype(np.float32)


def from_f32(v, dt):
    """float32 values rounded to the type, by torch / numpy."""
    if dt in TORCH16:
        return torch.from_numpy(v).to(TORCH16[dt]).view(torch.int16).numpy().view(np.uint16)
    return v.astype(np.float64)


def same_typed(got, want, dt):
    if dt in TORCH16:
        g = torch.from_numpy(got.view(np.int16).copy()).view(TORCH16[dt]).float().numpy()
        w = torch.from_numpy(want.view(np.int16).copy()).view(TORCH16[dt]).float().numpy()
    else:
        g, w = got, want
    gn, wn = np.isnan(g), np.isnan(w)
    assert (gn == wn).all()
    assert (got[~gn] == want[~wn]).all()


def inputs(dt, k, n, seed):
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(k):
        v = (rng.standard_normal(n) * 1e-2).astype(np.float64)
        v[rng.choice(n, max(1, n // 50), replace=False)] *= 300.0
        if dt == "f64":
            xs.append(v)
        else:
            xs.append(from_f32(v.astype(np.float32), dt))
    return xs


def test_bf16_through_the_bf16_codec_is_unchanged():
    rng = np.random.default_rng(80)
    x = rng.integers(0, 1 << 16, 100000).astype(np.uint16)
    codes, scales = O.encode_typed(x, "bf16", O.CODEC_BF16)
    assert scales is None
    v = as_f32(x, "bf16")
    fin = ~np.isnan(v)
    assert (codes[fin] == x[fin]).all()
    assert np.isnan(as_f32(codes[~fin], "bf16")).all()


@pytest.mark.parametrize("dt", ["f16", "bf16", "f64"])
@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
@pytest.mark.parametrize("mode", [0, 1])
def test_encode_is_the_binary32_encode_of_the_converted_values(dt, codec, mode):
    if codec == O.CODEC_BF16 and mode == 1:
        pytest.skip("the scale mode applies to fp8 only")
    x = inputs(dt, 1, 5000 + 37, 81)[0]
    codes, scales = O.encode_typed(x, dt, codec, mode)
    if codec == O.CODEC_BF16:
        assert (codes == O.encode_bf16(as_f32(x, dt))).all()
    else:
        wc, ws = O.encode_fp8(as_f32(x, dt), mode)
        assert (codes == wc).all() and (scales.view(np.uint32) == ws.view(np.uint32)).all()


def test_f64_input_rounds_once_to_binary32():
    # 1 + 2^-24 + 2^-40 is above the binary32 midpoint 1 + 2^-24: it must
    # round up to 1 + 2^-23 (bf16 code of that: 0x3F80); 1 + 2^-24 exactly is
    # a tie and goes to the even 1.0.  Through the fp8 codec with 448 planted,
    # values near 448 differ by whole codes only through that rounding.
    x = np.array([448.0, 1 + 2.0 ** -24 + 2.0 ** -40, 1 + 2.0 ** -24, 416.0 + 16.0 - 2.0 ** -30,
                  416.0 + 16.0 + 2.0 ** -30], dtype=np.float64)
    codes, _ = O.encode_typed(x, "f64", O.CODEC_FP8, 0)
    want, _ = O.encode_fp8(x.astype(np.float32), 0)
    assert (codes == want).all()
    # 432 = 416 + 16 is the midpoint of the E4M3 codes 416 (mantissa 101) and
    # 448 (mantissa 110).  binary32 holds 432 - 2^-30 as 432 itself, a tie that
    # goes to the even 448; quantizing the float64 value directly would give
    # 416, so this separates the two readings.
    assert O.e4m3_decode(codes[3:4])[0] == 448.0 and O.e4m3_decode(codes[4:5])[0] == 448.0


@pytest.mark.parametrize("dt", ["f16", "bf16", "f64"])
@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
def test_decode_sum_rounds_the_binary32_total_once(dt, codec):
    k, n = 4, 3000 + 11
    xs = inputs(dt, k, n, 82)
    enc = [O.encode_typed(x, dt, codec) for x in xs]
    codes = [c for c, _ in enc]
    scales = [s for _, s in enc] if codec == O.CODEC_FP8 else None
    got = O.decode_sum_typed(codes, scales, codec, dt)
    total = O.decode_accumulate(codes, scales, codec)
    same_typed(got, from_f32(total, dt), dt)


def test_f16_total_overflows_to_inf():
    # two ranks of the largest half, 65504, through bf16 (65504 -> 65536): the
    # binary32 total 131072 is beyond the half range and rounds to +Inf
    x = np.full(256, 0x7BFF, dtype=np.uint16)
    enc = [O.encode_typed(x, "f16", O.CODEC_BF16) for _ in range(2)]
    got = O.decode_sum_typed([c for c, _ in enc], None, O.CODEC_BF16, "f16")
    assert (got == 0x7C00).all()


@pytest.mark.parametrize("dt", ["f16", "bf16", "f64"])
@pytest.mark.parametrize("codec", [O.CODEC_NONE, O.CODEC_BF16, O.CODEC_FP8])
def test_bucket_stream(dt, codec):
    k, bucket, n = 3, 1024, 5 * 1024 + 300
    xs = inputs(dt, k, n, 83)
    out, codes, scales = O.bucket_allreduce_typed(xs, dt, bucket, codec)
    if codec == O.CODEC_NONE:
        same_typed(out, O.reduce_typed(xs, dt, O.OP_SUM), dt)
        return
    want, wc, ws = O.bucket_allreduce([as_f32(x, dt) for x in xs], bucket, codec)
    same_typed(out, from_f32(want, dt), dt)
    for r in range(k):
        assert (codes[r] == wc[r]).all()
        if codec == O.CODEC_FP8:
            assert (scales[r].view(np.uint32) == ws[r].view(np.uint32)).all()


@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
def test_every_f16_code_including_nan_payloads(codec):
    """All 2^16 half codes: the encode equals the binary32 encode of torch's
    own half -> float cast, which keeps a NaN's sign and payload (so the bf16
    code of a NaN carries the top payload bits and the fp8 code its sign)."""
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    codes, scales = O.encode_typed(x, "f16", codec, 0)
    if codec == O.CODEC_BF16:
        assert (codes == O.encode_bf16(as_f32(x, "f16"))).all()
    else:
        wc, ws = O.encode_fp8(as_f32(x, "f16"), 0)
        assert (codes == wc).all() and (scales.view(np.uint32) == ws.view(np.uint32)).all()


def test_f64_nan_payload_and_sign():
    """float64 NaNs with payloads and both signs: numpy's float64 -> float32
    cast keeps the sign and the top payload bits, quiet."""
    u = np.array([0x7FF8000000000000, 0xFFF8000000000000, 0x7FF0000000000001, 0x7FF4000000000000,
                  0xFFFABCDEF0123456, 0x7FF0000020000000, 0x7FFFFFFFFFFFFFFF], dtype=np.uint64)
    x = np.concatenate([u.view(np.float64), np.ones(256 - u.size)])
    codes, _ = O.encode_typed(x, "f64", O.CODEC_BF16)
    with np.errstate(invalid="ignore"):  # signalling NaNs raise "invalid" as they are quieted
        want = O.encode_bf16(x.astype(np.float32))
    assert (codes == want).all()
    assert codes[4] & 0x8000 and codes[4] != 0xFFC0  # sign and payload survive
