"""GPU parity of the bridge codecs over float16, bfloat16 and float64 (and
float32) arrays — gb_encode, gb_decode_sum, gb_bucket_allreduce_local_typed —
against the CPU oracle, bit for bit (NaNs included): ragged sizes,
every 16-bit code, float64 values at binary32 rounding boundaries and beyond
its range, every rank count, and the bucket stream at full size on sampled
blocks."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"
TYPES = ["f32", "f16", "bf16", "f64"]
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}
SIZES = [1, 255, 257, 4096 + 3, 3 * 65536 + 77]
CODECS = [O.CODEC_BF16, O.CODEC_FP8]


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


def to_host(t, dt):
    if dt in ("f16", "bf16"):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def codes_host(t):
    if t.dtype == torch.uint16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def values(a, dt):
    if dt == "f16":
        return a.view(np.float16).astype(np.float64)
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def same_typed(got, want, dt, what):
    """Every bit: a NaN total of any type is the canonical NaN's rounding."""
    g, w = got, want
    if dt == "f32":
        g, w = g.view(np.uint32), w.view(np.uint32)
    elif dt == "f64":
        g, w = g.view(np.uint64), w.view(np.uint64)
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first {bad[:4]}"


def inputs(dt, k, n, seed, specials=True):
    """Gradient-like values of type dt with outliers and special values."""
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(k):
        v = rng.standard_normal(n) * 1e-2
        v[rng.random(n) < 0.01] *= 300.0
        if specials:
            pool = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-30, -6e-8, 65504.0, 1e5])
            m = rng.random(n) < 0.002
            v[m] = pool[rng.integers(0, pool.size, int(m.sum()))]
        if dt == "f64":
            xs.append(v)
        elif dt == "f32":
            xs.append(v.astype(np.float32))
        else:
            t = torch.from_numpy(v.astype(np.float32)).to(TORCH[dt])
            xs.append(t.view(torch.int16).numpy().view(np.uint16))
    return xs


def gpu_encode(gb, x, dt, codec, mode):
    n = x.size
    d = to_dev(x, dt)
    codes = torch.empty(n, dtype=torch.uint16 if codec == O.CODEC_BF16 else torch.uint8, device=DEV)
    scales = torch.empty(O.nblocks(n), device=DEV) if codec == O.CODEC_FP8 else None
    gb.gb_encode(codec, codes, scales, d, mode)
    torch.cuda.synchronize()
    return codes_host(codes), (scales.cpu().numpy() if scales is not None else None)


def check_encode(gb, x, dt, codec, mode, what):
    gc, gs = gpu_encode(gb, x, dt, codec, mode)
    wc, ws = O.encode_typed(x, dt, codec, mode)
    bad = np.flatnonzero(gc != wc)
    assert bad.size == 0, f"{what}: {bad.size} code mismatches, first {bad[:4]}"
    if codec == O.CODEC_FP8:
        assert (gs.view(np.uint32) == ws.view(np.uint32)).all(), f"{what}: scales differ"


@pytest.mark.parametrize("dt", TYPES)
@pytest.mark.parametrize("codec,mode", [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)])
@pytest.mark.parametrize("n", SIZES)
def test_encode(gb, dt, codec, mode, n):
    x = inputs(dt, 1, n, 3000 + n % 1000)[0]
    check_encode(gb, x, dt, codec, mode, f"{dt} codec={codec} mode={mode} n={n}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("codec,mode", [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)])
def test_encode_every_16_bit_code(gb, dt, codec, mode):
    """All 2^16 codes, in their natural order (so each 256-block holds a run of
    neighbouring codes, from tiny to huge, NaN and Inf), then shuffled."""
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    check_encode(gb, x, dt, codec, mode, f"{dt} ordered")
    check_encode(gb, np.random.default_rng(3100).permutation(x), dt, codec, mode, f"{dt} shuffled")


def test_encode_f64_rounding_boundaries(gb):
    """float64 values at and beside binary32 midpoints, beyond its range, and
    below its subnormals: the encoders see the binary32 rounding of each."""
    rng = np.random.default_rng(3200)
    base = rng.standard_normal(4096).astype(np.float32).astype(np.float64)
    ulp = np.spacing(base.astype(np.float32)).astype(np.float64)
    mids = base + ulp / 2
    vals = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                           [3.4028235677973366e38, 3.4028235677973366e38 * (1 + 2 ** -30), 1e39, -1e300,
                            2.0 ** -150, 2.0 ** -150 * (1 + 2 ** -40), 1e-300, -1e-46, np.nan, np.inf]])
    for codec, mode in [(O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)]:
        check_encode(gb, vals, "f64", codec, mode, f"f64 boundaries codec={codec}")


@pytest.mark.parametrize("dt", TYPES)
@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("k", range(1, 9))
def test_decode_sum(gb, dt, codec, k):
    n = 2 * 4096 + 300
    xs = inputs(dt, k, n, 3300 + k)
    enc = [O.encode_typed(x, dt, codec) for x in xs]
    codes = [c for c, _ in enc]
    scales = [s for _, s in enc] if codec == O.CODEC_FP8 else None
    dcodes = [torch.from_numpy(c.view(np.int16) if c.dtype == np.uint16 else c).to(DEV) for c in codes]
    if codec == O.CODEC_BF16:
        dcodes = [c.view(torch.uint16) for c in dcodes]
    dscales = [torch.from_numpy(s).to(DEV) for s in scales] if scales is not None else None
    out = torch.empty(n, dtype=TORCH[dt], device=DEV)
    gb.gb_decode_sum(out, dcodes, dscales, codec)
    torch.cuda.synchronize()
    same_typed(to_host(out, dt), O.decode_sum_typed(codes, scales, codec, dt), dt, f"{dt} codec={codec} k={k}")


def test_decode_sum_f16_overflow_and_f32_equals_decode_accumulate(gb):
    # two ranks of 65504 through bf16 give 131072 in float32: +Inf in float16
    x = np.full(4096, 0x7BFF, dtype=np.uint16)
    c = torch.empty(4096, dtype=torch.uint16, device=DEV)
    gb.gb_encode(O.CODEC_BF16, c, None, to_dev(x, "f16"))
    out = torch.empty(4096, dtype=torch.float16, device=DEV)
    gb.gb_decode_sum(out, [c, c], None, O.CODEC_BF16)
    torch.cuda.synchronize()
    assert (to_host(out, "f16") == 0x7C00).all()
    a = torch.empty(4096, device=DEV)
    b = torch.empty(4096, device=DEV)
    gb.gb_decode_sum(a, [c, c], None, O.CODEC_BF16)
    gb.gb_decode_accumulate(b, [c, c], None, O.CODEC_BF16)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def run_bucket(gb, xs, dt, bucket, codec, mode=0):
    k, n = len(xs), xs[0].size
    d = [to_dev(x, dt) for x in xs]
    out = torch.empty(n, dtype=TORCH[dt], device=DEV)
    need = gb.gb_bucket_workspace_bytes(codec, k, n, bucket)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV) if codec != O.CODEC_NONE else None
    gb.gb_bucket_allreduce_local_typed(out, d, bucket, codec, mode, ws)
    torch.cuda.synchronize()
    return to_host(out, dt), ws


@pytest.mark.parametrize("dt", TYPES)
@pytest.mark.parametrize("codec,mode", [(O.CODEC_NONE, 0), (O.CODEC_BF16, 0), (O.CODEC_FP8, 0), (O.CODEC_FP8, 1)])
@pytest.mark.parametrize("k", [1, 3, 4, 8])
def test_bucket_stream(gb, dt, codec, mode, k):
    bucket, n = 4096, 5 * 4096 + 256 * 3 + 17
    xs = inputs(dt, k, n, 3400 + k + 10 * codec)
    got, ws = run_bucket(gb, xs, dt, bucket, codec, mode)
    want, codes, scales = O.bucket_allreduce_typed(xs, dt, bucket, codec, mode)
    same_typed(got, want, dt, f"{dt} codec={codec} k={k}")
    if codec == O.CODEC_NONE:
        return
    lay = gb.gb_bucket_workspace_layout(codec, k, n, bucket)
    for r in range(k):
        raw = ws[r * lay["codes_stride"]:][:n * (2 if codec == O.CODEC_BF16 else 1)]
        c = raw.view(torch.int16).cpu().numpy().view(np.uint16) if codec == O.CODEC_BF16 else raw.cpu().numpy()
        assert (c == codes[r]).all(), r
        if codec == O.CODEC_FP8:
            s = ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * O.nblocks(n)].view(torch.float32)
            assert (s.cpu().numpy().view(np.uint32) == scales[r].view(np.uint32)).all(), r


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_bucket_stream_in_place(gb, dt):
    xs = inputs(dt, 4, 3 * 4096 + 5, 3500)
    d = [to_dev(x, dt) for x in xs]
    need = gb.gb_bucket_workspace_bytes(O.CODEC_FP8, 4, d[0].numel(), 4096)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_typed(d[0], d, 4096, O.CODEC_FP8, 0, ws)
    torch.cuda.synchronize()
    want, _, _ = O.bucket_allreduce_typed(xs, dt, 4096, O.CODEC_FP8)
    same_typed(to_host(d[0], dt), want, dt, f"{dt} in place")


def gather_blocks(t, blocks):
    idx = (torch.as_tensor(blocks, device=t.device, dtype=torch.int64)[:, None] * 256
           + torch.arange(256, device=t.device)[None, :]).reshape(-1)
    return t[idx]


def test_ddp_1b_buckets_bf16_gradients_sampled(gb):
    """The DDP bucket stream over bfloat16 gradients at full size (4 x 1e9,
    25 MiB fp32-sized buckets), fp8 codec, one call, as the benchmark's
    --dtype bf16 run makes it; checked on random blocks and on the first and
    last block of every bucket."""
    k, n, bucket = 4, W.DDP_N, W.DDP_BUCKET
    x = [W.device_gradients_typed(n, W.BASE_SEED + r, DEV, "bf16") for r in range(k)]
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    lay = gb.gb_bucket_workspace_layout(O.CODEC_FP8, k, n, bucket)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_typed(out, x, bucket, O.CODEC_FP8, 0, ws)
    torch.cuda.synchronize()
    nb = n // 256
    edges = [e for s, l in W.ddp_buckets() for e in (s // 256, (s + l) // 256 - 1)]
    rng = np.random.default_rng(3600)
    blocks = np.array(sorted(set(rng.choice(nb, 3000, replace=False).tolist()) | set(edges)), dtype=np.int64)
    xs = [to_host(gather_blocks(t, blocks), "bf16") for t in x]
    want, codes, scales = O.bucket_allreduce_typed(xs, "bf16", 256, O.CODEC_FP8)
    same_typed(to_host(gather_blocks(out, blocks), "bf16"), want, "bf16", "ddp bf16")
    bt = torch.as_tensor(blocks, device=DEV)
    for r in range(k):
        c = ws[r * lay["codes_stride"]:r * lay["codes_stride"] + n]
        s = ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32)
        assert (gather_blocks(c, blocks).cpu().numpy() == codes[r]).all(), r
        assert (s[bt].cpu().numpy().view(np.uint32) == scales[r].view(np.uint32)).all(), r
    assert bool(torch.isfinite(out).all())


def double_rounding_payload(seed):
    """fp8 codes and block scales whose decoded products v * s round to
    float16 differently through binary32 (the definition: the float32 total is
    rounded once to the type) than directly: the exact product is a hair off
    an f16 midpoint that its binary32 rounding lands on.  Found by search with
    numpy's correctly rounded casts; -0 codes are mixed in."""
    rng = np.random.default_rng(seed)
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    codes, scales = [], []
    while len(scales) < 24:
        s = np.float32(rng.uniform(1e-4, 30.0))
        p = vals * np.float64(s)
        with np.errstate(invalid="ignore"):
            two = p.astype(np.float32).astype(np.float16).view(np.uint16)
            one = p.astype(np.float16).view(np.uint16)
        hit = np.flatnonzero((two != one) & np.isfinite(vals))
        if hit.size == 0:
            continue
        block = rng.integers(0, 256, 256).astype(np.uint8)
        block[rng.integers(0, 256, 64)] = 0x80  # -0
        block[rng.integers(0, 256, 128)] = hit[rng.integers(0, hit.size, 128)].astype(np.uint8)
        codes.append(block)
        scales.append(s)
    return np.concatenate(codes), np.array(scales, dtype=np.float32)


def test_decode_sum_f16_rounds_through_binary32(gb):
    """24 blocks over two workgroups of the decode (16 blocks each), the second
    one ragged (the last block is cut short)."""
    codes, scales = double_rounding_payload(3700)
    n = codes.size - 100
    codes = codes[:n]
    out = torch.empty(n, dtype=torch.float16, device=DEV)
    gb.gb_decode_sum(out, [torch.from_numpy(codes).to(DEV)], [torch.from_numpy(scales).to(DEV)], O.CODEC_FP8)
    torch.cuda.synchronize()
    want = O.decode_sum_typed([codes], [scales], O.CODEC_FP8, "f16")
    same_typed(to_host(out, "f16"), want, "f16", "f16 through binary32")
