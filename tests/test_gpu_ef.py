"""GPU parity of the error-feedback entry points against the CPU oracle,
over several steps with the residual carried from one step to the next."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"
SIZES = [1, 5, 255, 257, 4096 + 7, 3 * 262144 + 5]


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t):
    torch.cuda.synchronize()
    a = t.cpu().numpy() if t.dtype != torch.uint16 else t.view(torch.int16).cpu().numpy().view(np.uint16)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def same(got, want, what):
    g = got.view(np.float32) if got.dtype == np.uint32 else got
    w = want
    if w.dtype == np.float32:
        bad = np.flatnonzero(g.view(np.uint32) != w.view(np.uint32))
        assert bad.size == 0, f"{what}: {bad.size} mismatches at {bad[:5]}"
    else:
        bad = np.flatnonzero(g != w)
        assert bad.size == 0, f"{what}: {bad.size} mismatches at {bad[:5]}"


@pytest.mark.parametrize("n", SIZES)
def test_encode_bf16_ef_three_steps(gb, n):
    xs = [W.gradients(n, 900 + t) if n >= 100 else W.normal(n, 900 + t) for t in range(3)]
    res_h = np.zeros(n, np.float32)
    res_d = torch.zeros(n, device=DEV)
    codes = torch.empty(n, dtype=torch.uint16, device=DEV)
    for t, x in enumerate(xs):
        gb.gb_encode_bf16_ef(codes, res_d, dev(x))
        wc, res_h = O.encode_bf16_ef(x, res_h)
        same(bits(codes), wc, f"bf16 ef codes n={n} step={t}")
        same(bits(res_d).view(np.float32), res_h, f"bf16 ef residual n={n} step={t}")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("n", SIZES)
def test_encode_fp8_ef_three_steps(gb, n, mode):
    xs = [W.gradients(n, 910 + t) if n >= 100 else W.normal(n, 910 + t) for t in range(3)]
    res_h = np.zeros(n, np.float32)
    res_d = torch.zeros(n, device=DEV)
    codes = torch.empty(n, dtype=torch.uint8, device=DEV)
    scales = torch.empty(O.nblocks(n), device=DEV)
    for t, x in enumerate(xs):
        gb.gb_encode_fp8_e4m3_blockscaled_ef(codes, scales, res_d, dev(x), mode)
        wc, ws, res_h = O.encode_fp8_ef(x, res_h, mode)
        same(bits(scales).view(np.float32), ws, f"fp8 ef scales n={n} step={t}")
        same(bits(codes), wc, f"fp8 ef codes n={n} step={t}")
        same(bits(res_d).view(np.float32), res_h, f"fp8 ef residual n={n} step={t}")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("codec", [1, 2])
@pytest.mark.parametrize("k,n,bucket", [(1, 1000, 256), (3, 100000, 256 * 100), (4, 3 * 262144 + 5, 65536),
                                        (8, 20000 + 1, 2560)])
def test_bucket_allreduce_ef_two_steps(gb, k, n, bucket, codec, mode):
    if codec == 1 and mode == 1:
        pytest.skip("scale mode only applies to fp8")
    res_h = [np.zeros(n, np.float32) for _ in range(k)]
    res_d = [torch.zeros(n, device=DEV) for _ in range(k)]
    out = torch.empty(n, device=DEV)
    lay = gb.gb_bucket_workspace_layout(codec, k, n, bucket)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    for t in range(2):
        xs = W.gradient_ranks(k, n, 920 + 10 * t)
        gb.gb_bucket_allreduce_local_ef(out, [dev(x) for x in xs], res_d, bucket, codec, mode, ws)
        want, codes, scales, res_h = O.bucket_allreduce_ef(xs, res_h, bucket, codec, mode)
        same(bits(out).view(np.float32), want, f"bucket ef out step={t}")
        wsh = ws.cpu().numpy()
        for r in range(k):
            same(bits(res_d[r]).view(np.float32), res_h[r], f"bucket ef residual r={r} step={t}")
            c0 = r * lay["codes_stride"]
            if codec == 1:
                same(wsh[c0:c0 + 2 * n].view(np.uint16), codes[r], f"bucket ef codes r={r}")
            else:
                same(wsh[c0:c0 + n], codes[r], f"bucket ef codes r={r}")
                s0 = lay["scales_offset"] + r * lay["scales_stride"]
                same(wsh[s0:s0 + 4 * O.nblocks(n)].view(np.float32), scales[r], f"bucket ef scales r={r}")


def test_ef_rejects_without_a_lossy_codec(gb):
    x = torch.ones(1024, device=DEV)
    r = torch.zeros(1024, device=DEV)
    with pytest.raises(gb.GbError) as e:
        gb.gb_bucket_allreduce_local_ef(x.clone(), [x], [r], 256, gb.GB_CODEC_NONE)
    assert e.value.status == gb.GB_ERR_UNSUPPORTED
    codes = torch.empty(1024, dtype=torch.uint16, device=DEV)
    with pytest.raises(gb.GbError) as e:
        big = torch.zeros(1028, device=DEV)
        gb.gb_encode_bf16_ef(codes, big[1:1025], x)  # misaligned residual
    assert e.value.status == gb.GB_ERR_MISALIGNED


def same_codes(got, want, codec, what):
    """Codes equal, every byte: a NaN that an invalid operation creates (0 * Inf
    in the decode of an Inf-scaled block, Inf - Inf in a residual) or that two
    NaNs of different sign meet in is the canonical quiet NaN on both sides,
    so the codes that error feedback carries it into agree too."""
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches at {bad[:5]}: {got[bad[:5]]} vs {want[bad[:5]]}"


def planted(n, seed):
    """Gradient-like float32 values with the special values planted: one whole
    block of them (tiled) and 40 more at random places."""
    rng = np.random.default_rng(seed)
    sv = W.special_values()
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    if n >= 512:
        x[256:512] = np.resize(sv, 256)
    idx = rng.choice(n, min(40, n), replace=False)
    x[idx] = rng.choice(sv, idx.size)
    return x


@pytest.mark.parametrize("codec,mode", [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)])
def test_special_values_in_gradients_and_residuals(gb, codec, mode):
    """NaN, Inf, subnormals and the format edges in both the gradient and the
    residual: codes, scales and the new residual as the oracle gives them,
    over two steps, every bit (NaNs included)."""
    n = 256 * 6 + 19
    x = planted(n, 60)
    rng = np.random.default_rng(61)
    r0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    idx = rng.choice(n, 20, replace=False)
    r0[idx] = rng.choice(W.special_values(), idx.size)
    res = dev(r0)
    wres = r0
    for step in range(2):
        if codec == O.CODEC_BF16:
            codes = torch.empty(n, dtype=torch.uint16, device=DEV)
            gb.gb_encode_bf16_ef(codes, res, dev(x))
            wc, wres = O.encode_bf16_ef(x, wres)
        else:
            codes = torch.empty(n, dtype=torch.uint8, device=DEV)
            scales = torch.empty(O.nblocks(n), device=DEV)
            gb.gb_encode_fp8_e4m3_blockscaled_ef(codes, scales, res, dev(x), mode)
            wc, ws, wres = O.encode_fp8_ef(x, wres, mode)
            same(bits(scales), ws, f"scales step {step}")
        same_codes(bits(codes), wc, codec, f"codes step {step}")
        same(bits(res), wres, f"residual step {step}")


@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
def test_special_values_through_the_bucket_stream(gb, codec):
    k, bucket, n = 3, 512, 512 * 5 + 300
    xs = [planted(n, 70 + r) for r in range(k)]
    res = [dev(np.zeros(n, np.float32)) for _ in range(k)]
    out = torch.empty(n, device=DEV)
    ws = torch.empty(gb.gb_bucket_workspace_bytes(codec, k, n, bucket), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_ef(out, [dev(x) for x in xs], res, bucket, codec, 0, ws)
    want, _, _, wres = O.bucket_allreduce_ef(xs, [np.zeros(n, np.float32)] * k, bucket, codec, 0)
    same(bits(out), want, "out")
    for r in range(k):
        same(bits(res[r]), wres[r], f"residual {r}")


@pytest.mark.parametrize("codec,mode", [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)])
def test_every_float16_code_through_error_feedback(gb, codec, mode):
    """All 2^16 float16 codes (NaN payloads, Inf, subnormals) as a gradient with
    a small residual, through the typed error-feedback encoder."""
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    n = x.size
    r0 = (np.random.default_rng(80).standard_normal(n) * 1e-5).astype(np.float32)
    codes = torch.empty(n, dtype=torch.uint16 if codec == O.CODEC_BF16 else torch.uint8, device=DEV)
    scales = torch.empty(O.nblocks(n), device=DEV) if codec == O.CODEC_FP8 else None
    res = dev(r0)
    src = torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(torch.float16)
    gb.gb_encode_ef(codec, codes, scales, res, src, mode)
    wc, ws, wres = O.encode_ef_typed(x, r0, "f16", codec, mode)
    same_codes(bits(codes), wc, codec, "codes")
    if codec == O.CODEC_FP8:
        same(bits(scales), ws, "scales")
    same(bits(res), wres, "residual")
