"""The oracle against a second, independent implementation of the whole path
on tiny shapes (CPU only).

The second implementation is written here in torch's float32 arithmetic and
casts, nothing shared with the C oracle: the rank-order sum is a left fold of
float32 adds; bf16 is torch's round-to-nearest-even cast; an fp8 block takes
its largest magnitude, its scale (float32 absmax / 448, or the smallest power
of two 2^e, e >= -149, with absmax <= 448 * 2^e, found by exact double
comparisons), the float32 quotient, and torch's E4M3 cast after clamping to
+-448 (the clamp is what makes torch's cast saturating); decoding is the
E4M3 value times the scale in float32, added in rank order.  Buckets restart
blocks.  Inputs are finite (torch's casts are not a pin for NaN).  Shapes:
k in {1, 2, 3, 5}, n in {0, 1, 3, 4, 255, 256, 257, 511, 1000}, buckets of
256 and 512 values.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O

KS = [1, 2, 3, 5]
NS = [0, 1, 3, 4, 255, 256, 257, 511, 1000]


def data(k, n, seed):
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(k):
        v = rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 2)
        if n:
            v[rng.random(n) < 0.05] *= 1e3
            v[rng.random(n) < 0.02] = 0.0
            v[rng.random(n) < 0.02] = -0.0
            if n > 300:
                v[256:300] *= 1e-38  # a block of float32 subnormals and tiny values
        xs.append(v.astype(np.float32))
    return xs


def fold(vals):
    acc = vals[0].clone()
    for v in vals[1:]:
        acc = acc + v
    return acc


def pow2_scale(a):
    if a == 0.0:
        return 1.0
    e = math.frexp(a)[1] - 9
    while a > 448.0 * 2.0 ** e:
        e += 1
    while e > -149 and a <= 448.0 * 2.0 ** (e - 1):
        e -= 1
    return 2.0 ** max(e, -149)


def fp8_block(x, mode):
    """(codes, scale, decoded values) of one block, torch float32 throughout."""
    a = float(x.abs().max()) if x.numel() else 0.0
    if mode == O.SCALE_ABSMAX_DIV_448:
        s = (torch.tensor(a, dtype=torch.float32) / torch.tensor(448.0, dtype=torch.float32)).item()
    else:
        s = pow2_scale(a)
    st = torch.tensor(s, dtype=torch.float32)
    v = x if s == 0.0 else x / st
    q = v.clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s, q.float() * st


def second_encode_fp8(x, mode):
    codes, scales, dec = [], [], []
    for b in range(0, x.numel(), 256):
        c, s, d = fp8_block(x[b:b + 256], mode)
        codes.append(c)
        scales.append(s)
        dec.append(d)
    if not codes:
        return torch.empty(0, dtype=torch.uint8), np.empty(0, np.float32), torch.empty(0)
    return torch.cat(codes), np.array(scales, dtype=np.float32), torch.cat(dec)


def second_bucket_stream(xs, bucket, codec, mode):
    n = xs[0].numel()
    out = torch.empty(n, dtype=torch.float32)
    for s0 in range(0, n, bucket):
        parts = [x[s0:s0 + bucket] for x in xs]
        if codec == O.CODEC_BF16:
            dec = [p.to(torch.bfloat16).float() for p in parts]
        else:
            dec = [second_encode_fp8(p, mode)[2] for p in parts]
        out[s0:s0 + bucket] = fold(dec)
    return out


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("k", KS)
@pytest.mark.parametrize("n", NS)
def test_sum(k, n):
    xs = data(k, n, 100 * k + n)
    want = fold([torch.from_numpy(x) for x in xs]).numpy() if n else np.empty(0, np.float32)
    assert (bits(O.reduce_sum(xs)) == bits(want)).all()


@pytest.mark.parametrize("n", NS)
@pytest.mark.parametrize("mode", [O.SCALE_ABSMAX_DIV_448, O.SCALE_POW2])
def test_fp8_encode(n, mode):
    x = data(1, n, 7 + n)[0]
    codes, scales = O.encode_fp8(x, mode)
    wc, ws, _ = second_encode_fp8(torch.from_numpy(x), mode)
    assert (codes == wc.numpy()).all()
    assert (bits(scales) == bits(ws)).all()


@pytest.mark.parametrize("n", NS)
def test_bf16_encode(n):
    x = data(1, n, 11 + n)[0]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (O.encode_bf16(x) == want).all()


@pytest.mark.parametrize("k", KS)
@pytest.mark.parametrize("n", NS)
@pytest.mark.parametrize("codec,mode", [(O.CODEC_BF16, 0), (O.CODEC_FP8, O.SCALE_ABSMAX_DIV_448),
                                        (O.CODEC_FP8, O.SCALE_POW2)])
@pytest.mark.parametrize("bucket", [256, 512])
def test_bucket_stream(k, n, codec, mode, bucket):
    xs = data(k, n, 1000 * k + n + bucket)
    out, _, _ = O.bucket_allreduce(xs, bucket, codec, mode)
    want = second_bucket_stream([torch.from_numpy(x) for x in xs], bucket, codec, mode)
    assert (bits(out) == bits(want.numpy())).all()


@pytest.mark.parametrize("k", KS)
@pytest.mark.parametrize("n", [1, 257, 1000])
def test_decode_accumulate_fp8(k, n):
    """The decode of k oracle payloads, added in rank order, against the second
    implementation's decode of its own payloads."""
    xs = data(k, n, 77 + k + n)
    enc = [O.encode_fp8(x, O.SCALE_ABSMAX_DIV_448) for x in xs]
    got = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8)
    want = fold([second_encode_fp8(torch.from_numpy(x), O.SCALE_ABSMAX_DIV_448)[2] for x in xs])
    assert (bits(got) == bits(want.numpy())).all()
