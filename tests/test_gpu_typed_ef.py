"""GPU parity of error feedback over float16, bfloat16 and float64 gradients
(gb_encode_ef, gb_bucket_allreduce_local_ef_typed) against the oracle, bit
for bit: codes, scales, the updated binary32 residuals and the total rounded
to the gradient's type, over several steps with the residuals carried."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}
CODECS = [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)]


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def to_dev(a, dt):
    a = np.ascontiguousarray(a)
    if dt in ("f16", "bf16"):
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(TORCH[dt])
    return torch.from_numpy(a).to(DEV)


def to_host(t):
    if t.element_size() == 2 and t.is_floating_point():
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def same(got, want, dt, what, nan_as_nan=False):
    """Every byte, NaN included; nan_as_nan only for exact reductions of the
    other element types (NaN payloads of format conversions are a reading)."""
    if not nan_as_nan:
        assert got.tobytes() == want.tobytes(), what
        return
    if dt == "f16":
        gn, wn = np.isnan(got.view(np.float16)), np.isnan(want.view(np.float16))
    elif dt == "bf16":
        gn = np.isnan((got.astype(np.uint32) << 16).view(np.float32))
        wn = np.isnan((want.astype(np.uint32) << 16).view(np.float32))
    else:
        gn, wn = np.isnan(got), np.isnan(want)
    assert (gn == wn).all(), what + ": NaN positions differ"
    assert got[~gn].tobytes() == want[~wn].tobytes(), what


def f32_bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f64", "f32"])
@pytest.mark.parametrize("codec,mode", CODECS)
@pytest.mark.parametrize("n", [1, 255, 256 * 7 + 13, 4096 * 5 + 77])
def test_encode_ef(gb, dt, codec, mode, n):
    x = W.typed(n, dt, 400 + n)
    r0 = (np.random.default_rng(401 + n).standard_normal(n) * 1e-4).astype(np.float32)
    codes = torch.empty(n, dtype=torch.uint16 if codec == O.CODEC_BF16 else torch.uint8, device=DEV)
    scales = torch.empty(O.nblocks(n), device=DEV) if codec == O.CODEC_FP8 else None
    res = torch.from_numpy(r0.copy()).to(DEV)
    gb.gb_encode_ef(codec, codes, scales, res, to_dev(x, dt), mode)
    torch.cuda.synchronize()
    wc, ws, wr = O.encode_ef_typed(x, r0, dt, codec, mode)
    got = codes.view(torch.int16).cpu().numpy().view(np.uint16) if codec == O.CODEC_BF16 else codes.cpu().numpy()
    assert (got == wc).all()
    if codec == O.CODEC_FP8:
        assert (f32_bits(scales.cpu().numpy()) == f32_bits(ws)).all()
    assert (f32_bits(res.cpu().numpy()) == f32_bits(wr)).all()


@pytest.mark.parametrize("dt", ["f16", "bf16", "f64"])
@pytest.mark.parametrize("codec,mode", CODECS)
@pytest.mark.parametrize("k", [1, 3, 4, 8])
def test_bucket_stream_over_steps(gb, dt, codec, mode, k):
    bucket, n = 4096 * 2, 4096 * 7 + 300
    lay = gb.gb_bucket_workspace_layout(codec, k, n, bucket)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    res0 = [(np.random.default_rng(410 + r).standard_normal(n) * 1e-4).astype(np.float32) for r in range(k)]
    dres = [torch.from_numpy(r.copy()).to(DEV) for r in res0]
    wres = [r.copy() for r in res0]
    for step in range(3):
        xs = [W.typed(n, dt, 420 + 10 * step + r) for r in range(k)]
        dx = [to_dev(x, dt) for x in xs]
        out = torch.empty(n, dtype=TORCH[dt], device=DEV)
        gb.gb_bucket_allreduce_local_ef_typed(out, dx, dres, bucket, codec, mode, ws)
        torch.cuda.synchronize()
        want, wc, wsc, wres = O.bucket_allreduce_ef_typed(xs, wres, dt, bucket, codec, mode)
        what = f"dt={dt} codec={codec} mode={mode} k={k} step={step}"
        same(to_host(out), want, dt, what + " out")
        wsh = ws.cpu().numpy()
        for r in range(k):
            assert (f32_bits(dres[r].cpu().numpy()) == f32_bits(wres[r])).all(), what + f" residual {r}"
            c0 = r * lay["codes_stride"]
            if codec == O.CODEC_BF16:
                assert (wsh[c0:c0 + 2 * n].view(np.uint16) == wc[r]).all(), what + f" codes {r}"
            else:
                assert (wsh[c0:c0 + n] == wc[r]).all(), what + f" codes {r}"
                s0 = lay["scales_offset"] + r * lay["scales_stride"]
                assert (wsh[s0:s0 + 4 * wsc[r].size].view(np.uint32) == f32_bits(wsc[r])).all(), what + f" scales {r}"


@pytest.mark.parametrize("dt", ["bf16", "f64"])
def test_in_place_over_the_first_source(gb, dt):
    k, bucket, n = 4, 4096, 4096 * 3 + 1000
    xs = [W.typed(n, dt, 440 + r) for r in range(k)]
    dx = [to_dev(x, dt) for x in xs]
    res = [torch.zeros(n, device=DEV) for _ in range(k)]
    ws = torch.empty(gb.gb_bucket_workspace_bytes(O.CODEC_FP8, k, n, bucket), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_ef_typed(dx[0], dx, res, bucket, O.CODEC_FP8, 0, ws)
    torch.cuda.synchronize()
    want, _, _, wres = O.bucket_allreduce_ef_typed(xs, [np.zeros(n, np.float32)] * k, dt, bucket, O.CODEC_FP8)
    same(to_host(dx[0]), want, dt, "in place")
    for r in range(k):
        assert (f32_bits(res[r].cpu().numpy()) == f32_bits(wres[r])).all()


@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
def test_float32_through_the_typed_call_is_the_float32_call(gb, codec):
    """Up to 16 ranks: float32 gradients go through the same kernels, and
    beyond 8 ranks through the same folding, as gb_bucket_allreduce_local_ef."""
    for k in (4, 11):
        bucket, n = 4096, 4096 * 3 + 517
        xs = [torch.from_numpy(W.gradients(n, 450 + r)).to(DEV) for r in range(k)]
        r1 = [torch.full((n,), 3e-5, device=DEV) for _ in range(k)]
        r2 = [t.clone() for t in r1]
        o1, o2 = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
        need = gb.gb_bucket_workspace_bytes(codec, k, n, bucket)
        w1 = torch.empty(need, dtype=torch.uint8, device=DEV)
        w2 = torch.empty(need, dtype=torch.uint8, device=DEV)
        gb.gb_bucket_allreduce_local_ef(o1, xs, r1, bucket, codec, 0, w1)
        gb.gb_bucket_allreduce_local_ef_typed(o2, xs, r2, bucket, codec, 0, w2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), k
        for a, b in zip(r1, r2):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), k
