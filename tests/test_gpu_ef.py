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
        gn, wn = np.isnan(g), np.isnan(w)
        assert (gn == wn).all(), what
        assert (g.view(np.uint32)[~gn] == w.view(np.uint32)[~wn]).all(), what
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
