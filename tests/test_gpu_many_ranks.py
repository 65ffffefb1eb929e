"""More ranks than one kernel launch reads (9..GB_MAX_K = 16): every call that
takes k folds the ranks beyond the eighth in further launches.  Each result
must still equal the oracle's single left fold over all k ranks, bit for bit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"
KS = [9, 12, 15, 16]


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.uint16)
    return torch.from_numpy(a).to(DEV)


def bits(t):
    return t.view(torch.int32).cpu().numpy()


def u32(a):
    return np.ascontiguousarray(a).view(np.int32)


def same_nan(got, want):
    """Every bit, NaN included (the canonical NaN on both sides)."""
    assert (got.view(np.uint32) == want.view(np.uint32)).all()


def test_max_k_constant(gb):
    assert gb.GB_MAX_K == 16


@pytest.mark.parametrize("k", KS)
def test_reduce_sum(gb, k):
    n = 3 * 4096 + 77
    xs = W.normal_ranks(k, n, 4000 + k)
    d = [dev(x) for x in xs]
    out = torch.empty(n, device=DEV)
    gb.gb_reduce_sum(out, d)
    gb.gb_reduce_sum(d[0], d)  # in place on the first source
    torch.cuda.synchronize()
    want = u32(O.reduce_sum(xs))
    assert (bits(out) == want).all()
    assert (bits(d[0]) == want).all()


def test_reduce_sum_order_matters_beyond_eight(gb):
    """2^24 then fifteen 1.0s: rank-order folding keeps 2^24 (each 2^24 + 1
    rounds to even), while summing the 1.0s first would give 2^24 + 16."""
    n = 4096
    xs = [np.full(n, 2.0 ** 24, np.float32)] + [np.ones(n, np.float32) for _ in range(15)]
    out = torch.empty(n, device=DEV)
    gb.gb_reduce_sum(out, [dev(x) for x in xs])
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 2.0 ** 24).all()
    assert (u32(O.reduce_sum(xs)) == bits(out)).all()


@pytest.mark.parametrize("op", [0, 1, 2, 3])
@pytest.mark.parametrize("k", [9, 16])
def test_reduce_ops(gb, k, op):
    n = 2 * 4096 + 5
    xs = W.normal_ranks(k, n, 4100 + k)
    rng = np.random.default_rng(k + op)
    for x in xs:
        idx = rng.choice(n, 40, replace=False)
        x[idx] = np.array([0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)[rng.integers(0, 5, 40)]
    out = torch.empty(n, device=DEV)
    gb.gb_reduce(out, [dev(x) for x in xs], op, 3 * k)
    torch.cuda.synchronize()
    same_nan(out.cpu().numpy(), O.reduce(xs, op, 3 * k))


@pytest.mark.parametrize("dt,op", [("bf16", 0), ("bf16", 1), ("f16", 0), ("f16", 3), ("f64", 1), ("i8", 0),
                                   ("i32", 2), ("i64", 0)])
@pytest.mark.parametrize("k", [9, 16])
def test_reduce_typed(gb, k, dt, op):
    n = 2 * 4096 + 9
    xs = W.typed_ranks(k, n, dt, 4200 + k)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f64": torch.float64, "i8": torch.int8,
           "i32": torch.int32, "i64": torch.int64}[dt]

    def to(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(tdt)
        return torch.from_numpy(a).to(DEV)
    out = torch.empty(n, dtype=tdt, device=DEV)
    gb.gb_reduce_typed(out, [to(x) for x in xs], op, k)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16) if out.element_size() == 2 and \
        out.is_floating_point() else out.cpu().numpy()
    want = O.reduce_typed(xs, dt, op, k)
    assert got.tobytes() == want.tobytes()  # no NaN in these inputs


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("codec", [0, 1, 2])
@pytest.mark.parametrize("k", [10, 16])
def test_decode_accumulate(gb, k, codec, accumulate):
    n = 3 * 4096 + 300
    xs = W.gradient_ranks(k, n, 4300 + k)
    if codec == 0:
        payloads, scales = xs, None
    elif codec == 1:
        payloads, scales = [O.encode_bf16(x) for x in xs], None
    else:
        enc = [O.encode_fp8(x, 0) for x in xs]
        payloads, scales = [c for c, _ in enc], [s for _, s in enc]
    acc0 = W.normal(n, 5)
    acc = dev(acc0)
    gb.gb_decode_accumulate(acc, [dev(p) for p in payloads], [dev(s) for s in scales] if scales else None, codec,
                            accumulate)
    torch.cuda.synchronize()
    want = O.decode_accumulate(payloads, scales, codec, acc=acc0 if accumulate else None)
    assert (bits(acc) == u32(want)).all()


def test_decode_sum_many_payloads(gb):
    k, n = 11, 4096 + 17
    enc = [O.encode_fp8(x, 1) for x in W.gradient_ranks(k, n, 4400)]
    out = torch.empty(n, device=DEV)
    gb.gb_decode_sum(out, [dev(c) for c, _ in enc], [dev(s) for _, s in enc], gb.GB_CODEC_FP8_E4M3_B256)
    torch.cuda.synchronize()
    want = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8)
    assert (bits(out) == u32(want)).all()
    half = torch.empty(n, dtype=torch.float16, device=DEV)
    with pytest.raises(gb.GbError, match="rounded once"):
        gb.gb_decode_sum(half, [dev(c) for c, _ in enc], [dev(s) for _, s in enc], gb.GB_CODEC_FP8_E4M3_B256)


def workspace_payloads(gb, ws, codec, k, n, bucket):
    lay = gb.gb_bucket_workspace_layout(codec, k, n, bucket)
    codes, scales = [], []
    for r in range(k):
        c = ws[r * lay["codes_stride"]:][:n * (2 if codec == 1 else 1)]
        codes.append(c.view(torch.int16).cpu().numpy().view(np.uint16) if codec == 1 else c.cpu().numpy())
        if codec == 2:
            scales.append(ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * O.nblocks(n)]
                          .view(torch.float32).cpu().numpy())
    return codes, scales


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("codec,mode", [(0, 0), (1, 0), (2, 0), (2, 1)])
@pytest.mark.parametrize("k", [9, 16])
def test_bucket_stream(gb, k, codec, mode, in_place):
    bucket, n = 4096, 3 * 4096 + 256 * 2 + 11
    xs = W.gradient_ranks(k, n, 4500 + k)
    d = [dev(x) for x in xs]
    out = d[0] if in_place else torch.empty(n, device=DEV)
    need = gb.gb_bucket_workspace_bytes(codec, k, n, bucket)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV) if codec else None
    gb.gb_bucket_allreduce_local(out, d, bucket, codec, mode, ws)
    torch.cuda.synchronize()
    want, codes, scales = O.bucket_allreduce(xs, bucket, codec, mode)
    assert (bits(out) == u32(want)).all()
    if codec:
        gc, gs = workspace_payloads(gb, ws, codec, k, n, bucket)
        for r in range(k):
            assert (gc[r] == codes[r]).all(), r
            if codec == 2:
                assert (gs[r].view(np.uint32) == scales[r].view(np.uint32)).all(), r


@pytest.mark.parametrize("codec", [1, 2])
@pytest.mark.parametrize("k", [10, 16])
def test_bucket_stream_error_feedback(gb, k, codec):
    bucket, n = 4096, 2 * 4096 + 256 + 3
    xs = W.gradient_ranks(k, n, 4600 + k)
    res0 = [W.gradients(n, 4700 + r) * np.float32(1e-3) for r in range(k)]
    d = [dev(x) for x in xs]
    res = [dev(r) for r in res0]
    out = torch.empty(n, device=DEV)
    ws = torch.empty(gb.gb_bucket_workspace_bytes(codec, k, n, bucket), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_ef(out, d, res, bucket, codec, 0, ws)
    torch.cuda.synchronize()
    want, codes, scales, res1 = O.bucket_allreduce_ef(xs, res0, bucket, codec, 0)
    assert (bits(out) == u32(want)).all()
    for r in range(k):
        assert (bits(res[r]) == u32(res1[r])).all(), r
    gc, _ = workspace_payloads(gb, ws, codec, k, n, bucket)
    for r in range(k):
        assert (gc[r] == codes[r]).all(), r


def test_typed_bucket_stream(gb):
    k, bucket, n = 12, 4096, 2 * 4096 + 100
    xs = W.typed_ranks(k, n, "bf16", 4800)
    d = [torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(torch.bfloat16) for x in xs]
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    gb.gb_bucket_allreduce_local_typed(out, d, bucket, gb.GB_CODEC_NONE)
    torch.cuda.synchronize()
    want, _, _ = O.bucket_allreduce_typed(xs, "bf16", bucket, O.CODEC_NONE)
    assert (out.view(torch.int16).cpu().numpy().view(np.uint16) == want).all()
    ws = torch.empty(gb.gb_bucket_workspace_bytes(2, k, n, bucket), dtype=torch.uint8, device=DEV)
    with pytest.raises(gb.GbError, match="rounded once"):
        gb.gb_bucket_allreduce_local_typed(out, d, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    f32 = [torch.from_numpy(x).to(DEV) for x in W.gradient_ranks(k, n, 4900)]
    o32 = torch.empty(n, device=DEV)
    gb.gb_bucket_allreduce_local_typed(o32, f32, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    torch.cuda.synchronize()
    want, _, _ = O.bucket_allreduce(W.gradient_ranks(k, n, 4900), bucket, O.CODEC_FP8, 0)
    assert (bits(o32) == u32(want)).all()


@pytest.mark.parametrize("codec", [1, 2])
def test_staged_decode_many_ranks(gb, codec):
    k, n, chunk = 13, 65536 + 7, 4096
    xs = W.gradient_ranks(k, n, 5000)
    nb = O.nblocks(n)
    if codec == 1:
        payloads, scales = [O.encode_bf16(x) for x in xs], None
        hosts = [torch.from_numpy(p.view(np.int16)).view(torch.uint16).pin_memory() for p in payloads]
        devs = [torch.empty(n, dtype=torch.uint16, device=DEV) for _ in range(k)]
        sh = sd = None
    else:
        enc = [O.encode_fp8(x, 0) for x in xs]
        payloads, scales = [c for c, _ in enc], [s for _, s in enc]
        hosts = [torch.from_numpy(c).pin_memory() for c in payloads]
        devs = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(k)]
        sh = [torch.from_numpy(s).pin_memory() for s in scales]
        sd = [torch.empty(nb, device=DEV) for _ in range(k)]
    acc = torch.empty(n, device=DEV)
    gb.gb_decode_accumulate_staged(acc, hosts, sh, devs, sd, codec, chunk, False)
    torch.cuda.current_stream().synchronize()
    want = O.decode_accumulate(payloads, scales, codec)
    assert (bits(acc) == u32(want)).all()
