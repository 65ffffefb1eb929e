"""GPU parity: every libgbreduce entry point against the CPU oracle, through
the C ABI, on seeded inputs that span several workgroups and a ragged tail.

Bar: bit-exact on sums, bf16 codes, E4M3 codes and block scales; the
decode-accumulate sums are compared bit for bit as well (the arithmetic is
the same rounded multiply then rounded add on both sides), which is stricter
than the 1e-6 relative tolerance the method allows for them.  NaN outputs
are compared bit for bit too: every NaN the float32 arithmetic delivers is
the canonical quiet NaN 0x7FC00000 on both sides.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


DEV = "cuda:0"
SIZES = [1, 3, 4, 5, 255, 256, 257, 1000, 4096 + 7, 65536 + 255, 3 * 262144 + 5]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, what
    if got.dtype == np.float32:
        g, w = got.view(np.uint32), want.view(np.uint32)
    else:
        g, w = got, want
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: got {g[bad[:5]]} want {w[bad[:5]]}"


def ranks_with_specials(k, n, seed):
    xs = W.normal_ranks(k, n, seed)
    sp = W.special_values()
    for r, x in enumerate(xs):
        m = min(n, sp.size)
        x[:m] = np.roll(sp, r)[:m] if n >= sp.size else sp[r % sp.size]
    return xs


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k", range(1, 9))
@pytest.mark.parametrize("n", SIZES)
def test_reduce_sum(gb, k, n):
    xs = ranks_with_specials(k, n, 100 * k)
    d = [dev(x) for x in xs]
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    gb.gb_reduce_sum(out, d)
    assert_bits_equal(host(out), O.reduce_sum(xs), f"reduce_sum k={k} n={n}")


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_reduce_sum_in_place(gb, k):
    n = 70000 + 3
    xs = W.normal_ranks(k, n, 7)
    d = [dev(x) for x in xs]
    gb.gb_reduce_sum(d[0], d)
    assert_bits_equal(host(d[0]), O.reduce_sum(xs), "in place")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", SIZES)
def test_encode_bf16(gb, n):
    x = ranks_with_specials(1, n, 31)[0]
    codes = torch.empty(n, dtype=torch.uint16, device=DEV)
    gb.gb_encode_bf16(codes, dev(x))
    assert_bits_equal(host(codes.view(torch.int16)).view(np.uint16), O.encode_bf16(x), f"bf16 n={n}")


@pytest.mark.parametrize("n", [(1 << 23) + 1, (1 << 23) + 1024 + 3, (1 << 23) + 2047, (1 << 23) + 2048,
                               (1 << 23) - 5])
def test_encode_bf16_two_vectors_per_lane(gb, n):
    """From 2^23 values the encoder gives each lane two vectors 1024 values
    apart: tails that end inside the first vector, inside the second, and on
    a workgroup boundary, and the size just below the switch."""
    x = W.gradients(n, 37)
    codes = torch.empty(n, dtype=torch.uint16, device=DEV)
    gb.gb_encode_bf16(codes, dev(x))
    assert_bits_equal(host(codes.view(torch.int16)).view(np.uint16), O.encode_bf16(x), f"bf16 n={n}")
    half = torch.empty(n, dtype=torch.uint16, device=DEV)
    gb.gb_encode(gb.GB_CODEC_BF16, half, None, dev(x).half())
    want = O.encode_typed(dev(x).half().cpu().view(torch.int16).numpy().view(np.uint16), "f16", O.CODEC_BF16)[0]
    assert_bits_equal(host(half.view(torch.int16)).view(np.uint16), want, f"f16 -> bf16 n={n}")


def test_encode_bf16_every_rounding_class(gb):
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x4000, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF,
                     0x1234, 0x9ABC, 0x7FFE, 0x8002, 0x0F0F, 0xF0F0, 0x5555], dtype=np.uint32)
    x = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    codes = torch.empty(x.size, dtype=torch.uint16, device=DEV)
    gb.gb_encode_bf16(codes, dev(x))
    assert_bits_equal(host(codes.view(torch.int16)).view(np.uint16), O.encode_bf16(x), "bf16 classes")


# ---------------------------------------------------------------------------
def gpu_encode_fp8(gb, x, mode):
    n = x.size
    codes = torch.empty(n, dtype=torch.uint8, device=DEV)
    scales = torch.empty(O.nblocks(n), dtype=torch.float32, device=DEV)
    gb.gb_encode_fp8_e4m3_blockscaled(codes, scales, dev(x), mode)
    return host(codes), host(scales)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("n", SIZES)
def test_encode_fp8(gb, n, mode):
    x = W.gradients(n, 41) if n >= 100 else W.normal(n, 41)
    c, s = gpu_encode_fp8(gb, x, mode)
    wc, ws = O.encode_fp8(x, mode)
    assert_bits_equal(s, ws, f"fp8 scales n={n} mode={mode}")
    assert_bits_equal(c, wc, f"fp8 codes n={n} mode={mode}")


def special_blocks():
    """Blocks whose scale or codes sit on an edge of the format."""
    rng = np.random.default_rng(77)
    blocks = []
    blocks.append(np.zeros(256, np.float32))
    blocks.append(np.full(256, -0.0, np.float32))
    blocks.append((rng.standard_normal(256) * 2.0 ** -140).astype(np.float32))  # subnormal block
    blocks.append((rng.standard_normal(256) * 2.0 ** -128).astype(np.float32))  # subnormal scale
    for e in range(-152, -115):  # every binade where a / 448 is subnormal or nearly so
        blocks.append((rng.standard_normal(256) * 2.0 ** e).astype(np.float32))
    b = rng.standard_normal(256).astype(np.float32)
    b[17] = 448.0
    blocks.append(b)  # scale 1 in both modes
    b = (rng.standard_normal(256) * 1e30).astype(np.float32)
    blocks.append(b)  # near the top of the range
    b = rng.standard_normal(256).astype(np.float32)
    b[3] = np.inf
    blocks.append(b)  # Inf scale
    b = rng.standard_normal(256).astype(np.float32)
    b[5] = np.nan
    b[9] = -np.inf
    blocks.append(b)
    b = np.full(256, np.nan, np.float32)
    b[0] = 0.0
    blocks.append(b)  # zero scale with NaNs
    # E4M3 ties of the quotient: values on the midpoints, block max 448
    mids = []
    for c in range(0x7E):
        lo = O.e4m3_decode(np.array([c], np.uint8))[0]
        hi = O.e4m3_decode(np.array([c + 1], np.uint8))[0]
        mids.append((np.float64(lo) + np.float64(hi)) / 2)
    mids = np.array(mids, np.float32)
    for part in (mids[:126], -mids[:126]):
        b = np.zeros(256, np.float32)
        b[0] = 448.0
        b[1:127] = part
        b[127:253] = np.nextafter(part, np.float32(0))
        blocks.append(b)
    b = np.zeros(256, np.float32)
    b[0] = 448.0
    b[1:] = (rng.uniform(-448, 448, 255)).astype(np.float32)
    blocks.append(b)
    return np.concatenate(blocks)


@pytest.mark.parametrize("mode", [0, 1])
def test_encode_fp8_special_blocks(gb, mode):
    x = special_blocks()
    c, s = gpu_encode_fp8(gb, x, mode)
    wc, ws = O.encode_fp8(x, mode)
    assert_bits_equal(s, ws, f"fp8 special scales mode={mode}")
    assert_bits_equal(c, wc, f"fp8 special codes mode={mode}")


def test_encode_fp8_every_rounding_class(gb):
    # one 448 per block gives scale 1 in both modes, so each other value is
    # encoded on its own: every upper half with every sticky pattern of the
    # low half, magnitudes above 448 excluded (they would change the scale)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    x = u.view(np.float32)
    x = x[np.abs(x) <= 448]  # also drops NaN
    nb = -(-x.size // 255)
    blk = np.zeros((nb, 256), np.float32)
    blk[:, 0] = 448.0
    flat = np.zeros(nb * 255, np.float32)
    flat[:x.size] = x
    blk[:, 1:] = flat.reshape(nb, 255)
    buf = blk.ravel()
    for mode in (0, 1):
        c, s = gpu_encode_fp8(gb, buf, mode)
        wc, ws = O.encode_fp8(buf, mode)
        assert (ws == 1.0).all()
        assert_bits_equal(s, ws, f"fp8 classes scales mode={mode}")
        assert_bits_equal(c, wc, f"fp8 classes codes mode={mode}")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n", [5, 257, 4096 + 7, 3 * 262144 + 5])
def test_decode_accumulate_bf16(gb, n, k, accumulate):
    xs = W.gradient_ranks(k, n, 500) if n >= 100 else W.normal_ranks(k, n, 500)
    codes = [O.encode_bf16(x) for x in xs]
    acc0 = W.normal(n, 9)
    acc = dev(acc0)
    gb.gb_decode_accumulate(acc, [dev(c.view(np.int16)).view(torch.uint16) for c in codes], None,
                            gb.GB_CODEC_BF16, accumulate)
    want = O.decode_accumulate(codes, None, O.CODEC_BF16, acc=acc0 if accumulate else None)
    assert_bits_equal(host(acc), want, f"decode bf16 n={n} k={k} acc={accumulate}")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n", [5, 257, 4096 + 7, 3 * 262144 + 5])
def test_decode_accumulate_fp8(gb, n, k, accumulate, mode):
    xs = W.gradient_ranks(k, n, 600) if n >= 100 else W.normal_ranks(k, n, 600)
    enc = [O.encode_fp8(x, mode) for x in xs]
    acc0 = W.normal(n, 10)
    acc = dev(acc0)
    gb.gb_decode_accumulate(acc, [dev(c) for c, _ in enc], [dev(s) for _, s in enc],
                            gb.GB_CODEC_FP8_E4M3_B256, accumulate)
    want = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8,
                               acc=acc0 if accumulate else None)
    assert_bits_equal(host(acc), want, f"decode fp8 n={n} k={k} acc={accumulate}")


def test_decode_fp8_every_code_and_special_scales(gb):
    codes = np.tile(np.arange(256, dtype=np.uint8), 4)
    scales = np.array([1.0, 2.0 ** -140, 3.4e38, np.inf], np.float32)
    acc = torch.empty(1024, dtype=torch.float32, device=DEV)
    gb.gb_decode_accumulate(acc, [dev(codes)], [dev(scales)], gb.GB_CODEC_FP8_E4M3_B256, False)
    want = O.decode_accumulate([codes], [scales], O.CODEC_FP8)
    assert_bits_equal(host(acc), want, "fp8 decode table")


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("k", [1, 3, 8])
def test_decode_accumulate_fp32_payload(gb, k, accumulate):
    n = 10007
    xs = W.normal_ranks(k, n, 700)
    acc0 = W.normal(n, 11)
    acc = dev(acc0)
    gb.gb_decode_accumulate(acc, [dev(x) for x in xs], None, gb.GB_CODEC_NONE, accumulate)
    want = O.decode_accumulate(xs, None, O.CODEC_NONE, acc=acc0 if accumulate else None)
    assert_bits_equal(host(acc), want, "fp32 payload")


# ---------------------------------------------------------------------------
def run_bucket(gb, xs, bucket, codec, mode, in_place=False):
    k, n = len(xs), xs[0].size
    d = [dev(x) for x in xs]
    out = d[0] if in_place else torch.empty(n, dtype=torch.float32, device=DEV)
    lay = gb.gb_bucket_workspace_layout(codec, k, n, bucket)
    ws = torch.empty(max(lay["total"], 1), dtype=torch.uint8, device=DEV) if codec else None
    gb.gb_bucket_allreduce_local(out, d, bucket, codec, mode, ws)
    return host(out), (host(ws) if ws is not None else None), lay


def workspace_payload(ws, lay, codec, r, n):
    c0 = r * lay["codes_stride"]
    if codec == 1:
        return ws[c0:c0 + 2 * n].view(np.uint16), None
    s0 = lay["scales_offset"] + r * lay["scales_stride"]
    return ws[c0:c0 + n], ws[s0:s0 + 4 * O.nblocks(n)].view(np.float32)


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("codec", [0, 1, 2])
@pytest.mark.parametrize("k,n,bucket", [(1, 1000, 256), (2, 65536 + 3, 4096), (4, 3 * 262144 + 5, 65536),
                                        (3, 100000, 256 * 100), (8, 20000 + 1, 2560)])
def test_bucket_allreduce(gb, k, n, bucket, codec, mode, in_place):
    if codec != 2 and mode == 1:
        pytest.skip("scale mode only applies to fp8")
    xs = W.gradient_ranks(k, n, 800)
    out, ws, lay = run_bucket(gb, xs, bucket, codec, mode, in_place)
    want, wcodes, wscales = O.bucket_allreduce(xs, bucket, codec, mode)
    assert_bits_equal(out, want, f"bucket out k={k} n={n} codec={codec}")
    for r in range(k if codec else 0):
        c, s = workspace_payload(ws, lay, codec, r, n)
        assert_bits_equal(c, wcodes[r], f"bucket codes r={r}")
        if codec == 2:
            assert_bits_equal(s, wscales[r], f"bucket scales r={r}")


# ---------------------------------------------------------------------------
def test_zero_length_is_a_no_op(gb):
    t = torch.full((4,), 7.0, device=DEV)
    gb.gb_reduce_sum(t[:0], [t[:0], t[:0]])
    gb.gb_encode_bf16(torch.empty(0, dtype=torch.uint16, device=DEV), t[:0])
    gb.gb_decode_accumulate(t[:0], [t[:0]], None, gb.GB_CODEC_NONE)
    assert (host(t) == 7.0).all()


def test_errors_enqueue_nothing(gb):
    n = 1024
    out = torch.full((n + 4,), 5.0, device=DEV)
    x = torch.ones(n + 4, device=DEV)
    with pytest.raises(gb.GbError) as e:
        gb.gb_reduce_sum(out[1:n + 1], [x[:n], x[:n]])  # misaligned dst
    assert e.value.status == gb.GB_ERR_MISALIGNED
    with pytest.raises(gb.GbError) as e:
        gb.gb_reduce_sum(out[:n], [x[:n]] * 17)  # k beyond the maximum (16)
    assert e.value.status == gb.GB_ERR_INVALID_ARG
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(gb.GbError) as e:
        gb.gb_bucket_allreduce_local(out[:n], [x[:n]] * 2, 256, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    assert e.value.status == gb.GB_ERR_WORKSPACE
    with pytest.raises(gb.GbError) as e:
        gb.gb_bucket_allreduce_local(out[:n], [x[:n]] * 2, 100, gb.GB_CODEC_NONE, 0, None)
    assert e.value.status == gb.GB_ERR_INVALID_ARG
    assert (host(out) == 5.0).all()
