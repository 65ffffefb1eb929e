"""Pins of the oracle's error feedback over float16, bfloat16 and float64
gradients (README "Bridge compression": a residual per buffer carries each
step's rounding error into the next), CPU only.

Reading: the error-feedback step runs in binary32 whatever the gradient's
type, with a binary32 residual, exactly as for float32 gradients; the type
only changes how the gradient is converted on the way in (as the typed
codecs convert it) and how the decoded total is rounded on the way out.
Each typed function is pinned to the already-pinned binary32 error-feedback
path fed by independent conversions (torch's half / bfloat16 casts, numpy's
float64 casts), and by the convergence the feedback exists for.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_typed_codec import as_f32, from_f32, inputs, same_typed

TYPES = ["f16", "bf16", "f64"]
CODECS = [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)]


def residuals(k, n, seed, scale=1e-4):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(n) * scale).astype(np.float32) for _ in range(k)]


@pytest.mark.parametrize("dt", TYPES)
@pytest.mark.parametrize("codec,mode", CODECS)
def test_encode_is_the_binary32_step_on_the_converted_values(dt, codec, mode):
    n = 256 * 9 + 77
    x = inputs(dt, 1, n, 300)[0]
    r0 = residuals(1, n, 301)[0]
    codes, scales, res = O.encode_ef_typed(x, r0, dt, codec, mode)
    xf = as_f32(x, dt)
    if codec == O.CODEC_BF16:
        wc, wres = O.encode_bf16_ef(xf, r0)
    else:
        wc, ws, wres = O.encode_fp8_ef(xf, r0, mode)
        assert (scales.view(np.uint32) == ws.view(np.uint32)).all()
    assert (codes == wc).all()
    assert (res.view(np.uint32) == wres.view(np.uint32)).all()


def test_f64_rounding_to_binary32_is_not_fed_back():
    """A float64 gradient is rounded to binary32 before the step, as the
    codecs round it: its sub-binary32 part is not carried in the residual."""
    x = np.array([1.0 + 2.0 ** -30] * 256, dtype=np.float64)  # rounds to 1.0 in binary32
    codes, _, res = O.encode_ef_typed(x, np.zeros(256, np.float32), "f64", O.CODEC_BF16)
    assert (res == 0).all()  # 1.0 is a bf16 value: nothing left over
    assert (codes == 0x3F80).all()


@pytest.mark.parametrize("dt", TYPES + ["f32"])
@pytest.mark.parametrize("codec,mode", CODECS)
def test_bucket_stream_over_steps(dt, codec, mode):
    """Three steps with the residuals carried: the typed stream is the binary32
    stream on the converted gradients, its total rounded once to the type."""
    k, bucket, n = 3, 1024, 4 * 1024 + 300
    res = residuals(k, n, 310, 0.0)
    wres = [r.copy() for r in res]
    for step in range(3):
        xs = inputs(dt, k, n, 320 + step) if dt != "f32" else [
            (np.random.default_rng(320 + step + r).standard_normal(n) * 1e-2).astype(np.float32) for r in range(k)]
        out, codes, scales, res = O.bucket_allreduce_ef_typed(xs, res, dt, bucket, codec, mode)
        xf = [as_f32(x, dt) for x in xs] if dt != "f32" else xs
        want, wc, ws, wres = O.bucket_allreduce_ef(xf, wres, bucket, codec, mode)
        if dt == "f32":
            assert (out.view(np.uint32) == want.view(np.uint32)).all()
        else:
            same_typed(out, from_f32(want, dt), dt)
        for r in range(k):
            assert (codes[r] == wc[r]).all()
            assert (res[r].view(np.uint32) == wres[r].view(np.uint32)).all()
            if codec == O.CODEC_FP8:
                assert (scales[r].view(np.uint32) == ws[r].view(np.uint32)).all()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("codec,mode", CODECS)
def test_running_mean_converges_for_half_gradients(dt, codec, mode):
    """The same half-precision gradient every step: the mean of the decoded
    payloads approaches its value, within the largest residual over T, which a
    dropped or mis-signed feedback term would not give."""
    n, T = 256 * 4, 150
    x = inputs(dt, 1, n, 330)[0]
    xf = as_f32(x, dt).astype(np.float64)
    res = np.zeros(n, np.float32)
    total = np.zeros(n)
    worst = 0.0
    for _ in range(T):
        codes, scales, res = O.encode_ef_typed(x, res, dt, codec, mode)
        dec = O.decode_accumulate([codes], [scales] if codec == O.CODEC_FP8 else None, codec)
        total += dec.astype(np.float64)
        worst = max(worst, float(np.abs(res).max()))
    err = np.abs(total / T - xf).max()
    assert err <= worst / T * 1.01 + 1e-12
    # without feedback the error is that of one rounding, far larger here;
    # bfloat16 gradients through the bf16 codec are exact either way
    pc, ps = O.encode_typed(x, dt, codec, mode)
    plain = O.decode_accumulate([pc], [ps] if codec == O.CODEC_FP8 else None, codec)
    plain_err = np.abs(plain.astype(np.float64) - xf).max()
    if dt == "bf16" and codec == O.CODEC_BF16:
        assert plain_err == 0 and err == 0 and worst == 0
    else:
        assert plain_err > 20 * err
