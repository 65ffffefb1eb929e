"""GPU parity of gb_bucket_allreduce_local_batch: buckets in separate
buffers, each with its own sources and output, against the oracle's bucket
stream of that bucket alone (fp8 blocks restart at each bucket), bit for
bit, with every rank's payload checked where the workspace layout puts it.
Up to 16 buckets share a launch; lists of more buckets, empty buckets, ragged
sizes, 9..16 ranks (one bucket at a time), the uncompressed codec, outputs
over the first source, float16, bfloat16 and float64 gradients, and a
replayed HIP graph are covered too."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"
SIZES = [1000, 0, 1, 255, 256, 257, 4096 * 2 + 100, 513, 12_345, 4096, 77, 20_000,
         300, 1024, 5, 700, 4096 * 4, 999, 256 * 3 + 1, 64]  # 20 buckets, 19 of them in two launches
CODECS = [(O.CODEC_BF16, 0), (O.CODEC_FP8, O.SCALE_ABSMAX_DIV_448), (O.CODEC_FP8, O.SCALE_POW2)]


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def host_buckets(sizes, k, seed):
    out = []
    for b, n in enumerate(sizes):
        xs = [W.gradients(n, seed + 100 * b + r) if n else np.empty(0, np.float32) for r in range(k)]
        out.append(xs)
    return out


def to_dev(buckets):
    return [[torch.from_numpy(x.copy()).to(DEV) for x in xs] for xs in buckets]


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def offsets(sizes):
    o, offs = 0, []
    for n in sizes:
        offs.append(o)
        o += (n + 255) // 256 * 256
    return offs, o


def check(gb, sizes, k, codec, mode, seed, in_place=False):
    hb = host_buckets(sizes, k, seed)
    db = to_dev(hb)
    outs = [xs[0] if in_place else torch.full((n,), float("nan"), device=DEV) for xs, n in zip(db, sizes)]
    need = gb.gb_bucket_batch_workspace_bytes(codec, k, sizes)
    ws = torch.full((max(need, 1),), 0xEE, dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch(outs, db, codec, mode, ws if need else None)
    torch.cuda.synchronize()
    offs, total = offsets(sizes)
    lay = gb.gb_bucket_workspace_layout(codec, k, total, 256) if codec != O.CODEC_NONE else None
    wsh = ws.cpu().numpy()
    for b, (xs, n) in enumerate(zip(hb, sizes)):
        if n == 0:
            continue
        bucket = (n + 255) // 256 * 256
        want, wc, wsc = O.bucket_allreduce(xs, bucket, codec, mode)
        what = f"sizes={sizes} k={k} codec={codec} mode={mode} bucket {b} (n={n})"
        assert (bits(outs[b].cpu().numpy()) == bits(want)).all(), what
        if lay is None:
            continue
        for r in range(k):
            if codec == O.CODEC_BF16:
                c0 = r * lay["codes_stride"] + 2 * offs[b]
                assert (wsh[c0:c0 + 2 * n].view(np.uint16) == wc[r]).all(), what + f" codes {r}"
            else:
                c0 = r * lay["codes_stride"] + offs[b]
                assert (wsh[c0:c0 + n] == wc[r]).all(), what + f" codes {r}"
                s0 = lay["scales_offset"] + r * lay["scales_stride"] + 4 * (offs[b] // 256)
                assert (wsh[s0:s0 + 4 * wsc[r].size].view(np.uint32) == bits(wsc[r])).all(), what + f" scales {r}"


@pytest.mark.parametrize("codec,mode", CODECS)
@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_matches_the_oracle_bucket_by_bucket(gb, codec, mode, k):
    check(gb, SIZES, k, codec, mode, 3000 + 10 * k + codec + mode)


@pytest.mark.parametrize("codec,mode", CODECS + [(O.CODEC_NONE, 0)])
def test_more_ranks_than_one_launch_reads(gb, codec, mode):
    check(gb, [300, 0, 4096 + 5, 256], 11, codec, mode, 3100 + codec + mode)


def test_uncompressed_codec_is_the_plain_sum(gb):
    check(gb, SIZES[:5], 3, O.CODEC_NONE, 0, 3200)


@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
def test_outputs_over_the_first_sources(gb, codec):
    check(gb, [1000, 4096 * 3 + 1, 256], 4, codec, 0, 3300, in_place=True)


@pytest.mark.parametrize("codec", [O.CODEC_BF16, O.CODEC_FP8])
def test_equals_one_call_per_bucket_at_bucket_sizes(gb, codec):
    """Buckets of one GPU's 1/8 share of a 25 MiB bucket (819,200 values) and
    a ragged last one, 21 of them (two launches), four ranks: the same bits
    and payloads as gb_bucket_allreduce_local called once per bucket."""
    sizes = [819_200] * 20 + [481_600 + 37]
    k = 4
    x = [[W.device_gradients(n, 3400 + 10 * b + r, DEV) for r in range(k)] for b, n in enumerate(sizes)]
    outs = [torch.empty(n, device=DEV) for n in sizes]
    need = gb.gb_bucket_batch_workspace_bytes(codec, k, sizes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch(outs, x, codec, 0, ws)
    offs, total = offsets(sizes)
    lay = gb.gb_bucket_workspace_layout(codec, k, total, 256)
    csz = 2 if codec == O.CODEC_BF16 else 1
    for b, n in enumerate(sizes):
        ref = torch.empty(n, device=DEV)
        w1 = torch.zeros(gb.gb_bucket_workspace_bytes(codec, k, n, 819_200), dtype=torch.uint8, device=DEV)
        gb.gb_bucket_allreduce_local(ref, x[b], 819_200, codec, 0, w1)
        torch.cuda.synchronize()
        assert torch.equal(outs[b].view(torch.int32), ref.view(torch.int32)), f"bucket {b}"
        l1 = gb.gb_bucket_workspace_layout(codec, k, n, 819_200)
        for r in range(k):
            a = ws[r * lay["codes_stride"] + csz * offs[b]:][:csz * n]
            assert torch.equal(a, w1[r * l1["codes_stride"]:][:csz * n]), f"bucket {b} codes {r}"
            if codec == O.CODEC_FP8:
                nb = (n + 255) // 256
                a = ws[lay["scales_offset"] + r * lay["scales_stride"] + 4 * (offs[b] // 256):][:4 * nb]
                assert torch.equal(a, w1[l1["scales_offset"] + r * l1["scales_stride"]:][:4 * nb]), f"scales {r}"


def test_replayed_graph_matches_eager(gb):
    """The call captured in a HIP graph (kernel launches only) and replayed
    three times with new inputs and eager work in between."""
    sizes, k = [5000, 819_200, 256, 70_000], 4
    x = [[torch.empty(n, device=DEV) for _ in range(k)] for n in sizes]
    outs = [torch.empty(n, device=DEV) for n in sizes]
    ws = torch.empty(gb.gb_bucket_batch_workspace_bytes(O.CODEC_FP8, k, sizes), dtype=torch.uint8, device=DEV)
    for b in range(len(sizes)):
        for r in range(k):
            x[b][r].copy_(W.device_gradients(sizes[b], 3500 + 10 * b + r, DEV))
    gb.gb_bucket_allreduce_local_batch(outs, x, O.CODEC_FP8, 0, ws)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gb.gb_bucket_allreduce_local_batch(outs, x, O.CODEC_FP8, 0, ws)
    for rep in range(3):
        for b in range(len(sizes)):
            for r in range(k):
                x[b][r].copy_(W.device_gradients(sizes[b], 3600 + 100 * rep + 10 * b + r, DEV))
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = [torch.empty_like(o) for o in outs]
        gb.gb_bucket_allreduce_local_batch(ref, x, O.CODEC_FP8, 0, ws)
        torch.cuda.synchronize()
        for b in range(len(sizes)):
            assert torch.equal(got[b].view(torch.int32), ref[b].view(torch.int32)), f"replay {rep} bucket {b}"


TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}


def typed_to_dev(a, dt):
    if dt in ("f16", "bf16"):
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(TORCH[dt])
    return torch.from_numpy(a.copy()).to(DEV)


def typed_to_host(t):
    if t.element_size() == 2:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint64)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f64"])
@pytest.mark.parametrize("codec,mode", CODECS + [(O.CODEC_NONE, 0)])
@pytest.mark.parametrize("k", [1, 4, 8])
def test_typed_gradients_match_the_oracle(gb, dt, codec, mode, k):
    """Buckets of float16, bfloat16 or float64 gradients: each total equals
    the oracle's typed bucket stream of that bucket alone, and each payload
    sits where the workspace layout puts it."""
    sizes = [300, 0, 4096 * 3 + 17, 256, 1, 20_000, 513] + [700] * 12  # 18 buckets: two launches
    hb = [[W.typed(n, dt, 3700 + 50 * b + r) for r in range(k)] for b, n in enumerate(sizes)]
    db = [[typed_to_dev(x, dt) for x in xs] for xs in hb]
    outs = [torch.empty(n, dtype=TORCH[dt], device=DEV) for n in sizes]
    need = gb.gb_bucket_batch_workspace_bytes(codec, k, sizes)
    ws = torch.full((max(need, 1),), 0xEE, dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch(outs, db, codec, mode, ws if need else None)
    torch.cuda.synchronize()
    offs, total = offsets(sizes)
    lay = gb.gb_bucket_workspace_layout(codec, k, total, 256) if codec != O.CODEC_NONE else None
    wsh = ws.cpu().numpy()
    for b, n in enumerate(sizes):
        if n == 0:
            continue
        want, wc, wsc = O.bucket_allreduce_typed(hb[b], dt, (n + 255) // 256 * 256, codec, mode)
        what = f"dt={dt} k={k} codec={codec} mode={mode} bucket {b} (n={n})"
        assert typed_to_host(outs[b]).tobytes() == np.ascontiguousarray(want).tobytes(), what
        if lay is None:
            continue
        for r in range(k):
            if codec == O.CODEC_BF16:
                c0 = r * lay["codes_stride"] + 2 * offs[b]
                assert (wsh[c0:c0 + 2 * n].view(np.uint16) == wc[r]).all(), what + f" codes {r}"
            else:
                c0 = r * lay["codes_stride"] + offs[b]
                assert (wsh[c0:c0 + n] == wc[r]).all(), what + f" codes {r}"
                s0 = lay["scales_offset"] + r * lay["scales_stride"] + 4 * (offs[b] // 256)
                assert (wsh[s0:s0 + 4 * wsc[r].size].view(np.uint32) == bits(wsc[r])).all(), what + f" scales {r}"


def dev_typed(x, dt):
    return torch.from_numpy(x.copy()).to(DEV) if dt == "f32" else typed_to_dev(x, dt)


def host_typed(t, dt):
    return t.cpu().numpy().view(np.uint32) if dt == "f32" else typed_to_host(t)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16", "f64"])
@pytest.mark.parametrize("codec,mode", CODECS)
@pytest.mark.parametrize("k", [1, 4, 8])
def test_error_feedback_matches_the_oracle_over_steps(gb, dt, codec, mode, k):
    """gb_bucket_allreduce_local_batch_ef over three steps, residuals carried:
    each bucket's total, payloads and residuals equal the oracle's typed
    error-feedback stream of that bucket alone.  11 non-empty buckets: two
    launches of at most 8."""
    sizes = [300, 0, 4096 * 3 + 17, 256, 1, 20_000, 513] + [700] * 5
    res = [[(np.random.default_rng(3800 + 50 * b + r).standard_normal(n) * 1e-4).astype(np.float32)
            for r in range(k)] for b, n in enumerate(sizes)]
    dres = [[torch.from_numpy(a.copy()).to(DEV) for a in rb] for rb in res]
    need = gb.gb_bucket_batch_workspace_bytes(codec, k, sizes)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    offs, total = offsets(sizes)
    lay = gb.gb_bucket_workspace_layout(codec, k, total, 256)
    for step in range(3):
        hb = [[W.typed(n, dt, 3900 + 100 * step + 10 * b + r) for r in range(k)] for b, n in enumerate(sizes)]
        db = [[dev_typed(x, dt) for x in xs] for xs in hb]
        outs = [torch.empty(n, dtype=db[b][0].dtype, device=DEV) for b, n in enumerate(sizes)]
        gb.gb_bucket_allreduce_local_batch_ef(outs, db, dres, codec, mode, ws)
        torch.cuda.synchronize()
        wsh = ws.cpu().numpy()
        for b, n in enumerate(sizes):
            if n == 0:
                continue
            want, wc, wsc, res[b] = O.bucket_allreduce_ef_typed(hb[b], res[b], dt, (n + 255) // 256 * 256, codec, mode)
            what = f"dt={dt} k={k} codec={codec} mode={mode} step={step} bucket {b} (n={n})"
            assert host_typed(outs[b], dt).tobytes() == np.ascontiguousarray(want).tobytes(), what
            for r in range(k):
                assert (dres[b][r].cpu().numpy().view(np.uint32) == bits(res[b][r])).all(), what + f" residual {r}"
                if codec == O.CODEC_BF16:
                    c0 = r * lay["codes_stride"] + 2 * offs[b]
                    assert (wsh[c0:c0 + 2 * n].view(np.uint16) == wc[r]).all(), what + f" codes {r}"
                else:
                    c0 = r * lay["codes_stride"] + offs[b]
                    assert (wsh[c0:c0 + n] == wc[r]).all(), what + f" codes {r}"
                    s0 = lay["scales_offset"] + r * lay["scales_stride"] + 4 * (offs[b] // 256)
                    assert (wsh[s0:s0 + 4 * wsc[r].size].view(np.uint32) == bits(wsc[r])).all(), what + f" scales {r}"


@pytest.mark.parametrize("dt,k", [("bf16", 2), ("f16", 3), ("f64", 1)])
def test_error_feedback_batch_takes_its_largest_buckets_shape(gb, dt, k):
    """The bf16 error-feedback batch takes its whole-buffer rule for its
    largest bucket: here a bucket above 2^22 values puts every bucket of the
    launch in 64-lane workgroups, the small and ragged ones included, which
    alone would take 256 lanes.  Each bucket must equal the oracle and the
    same bucket through gb_bucket_allreduce_local_ef_typed alone, bit for
    bit: totals, codes and residuals."""
    codec = O.CODEC_BF16
    sizes = [(1 << 22) + 77, 300, 1, 5000, 513]
    hb = [[W.typed(n, dt, 4100 + 10 * b + r) for r in range(k)] for b, n in enumerate(sizes)]
    res = [[(np.random.default_rng(4200 + 50 * b + r).standard_normal(n) * 1e-4).astype(np.float32)
            for r in range(k)] for b, n in enumerate(sizes)]
    db = [[dev_typed(x, dt) for x in xs] for xs in hb]
    dres = [[torch.from_numpy(a.copy()).to(DEV) for a in rb] for rb in res]
    outs = [torch.empty(n, dtype=db[b][0].dtype, device=DEV) for b, n in enumerate(sizes)]
    ws = torch.empty(gb.gb_bucket_batch_workspace_bytes(codec, k, sizes), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch_ef(outs, db, dres, codec, 0, ws)
    torch.cuda.synchronize()
    for b, n in enumerate(sizes):
        want, _, _, wres = O.bucket_allreduce_ef_typed(hb[b], res[b], dt, (n + 255) // 256 * 256, codec)
        what = f"dt={dt} k={k} bucket {b} (n={n})"
        assert host_typed(outs[b], dt).tobytes() == np.ascontiguousarray(want).tobytes(), what
        one = torch.empty_like(outs[b])
        rone = [torch.from_numpy(a.copy()).to(DEV) for a in res[b]]
        wso = torch.empty(gb.gb_bucket_workspace_bytes(codec, k, n, (n + 255) // 256 * 256), dtype=torch.uint8,
                          device=DEV)
        gb.gb_bucket_allreduce_local_ef_typed(one, db[b], rone, (n + 255) // 256 * 256, codec, 0, wso)
        torch.cuda.synchronize()
        assert host_typed(one, dt).tobytes() == host_typed(outs[b], dt).tobytes(), what + " against the call alone"
        for r in range(k):
            assert (dres[b][r].cpu().numpy().view(np.uint32) == bits(wres[r])).all(), what + f" residual {r}"
            assert torch.equal(rone[r].view(torch.int32), dres[b][r].view(torch.int32)), what + f" residual {r} alone"


def test_error_feedback_with_more_ranks_than_one_launch_reads(gb):
    """11 ranks of float32 gradients: one bucket at a time, as the
    single-buffer error-feedback call, against the oracle."""
    sizes, k = [1000, 4096 + 3, 256], 11
    res = [[np.full(n, 2e-5, np.float32) for _ in range(k)] for n in sizes]
    dres = [[torch.from_numpy(a.copy()).to(DEV) for a in rb] for rb in res]
    hb = [[W.gradients(n, 4000 + 20 * b + r) for r in range(k)] for b, n in enumerate(sizes)]
    db = [[torch.from_numpy(x.copy()).to(DEV) for x in xs] for xs in hb]
    outs = [torch.empty(n, device=DEV) for n in sizes]
    ws = torch.empty(gb.gb_bucket_batch_workspace_bytes(O.CODEC_FP8, k, sizes), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch_ef(outs, db, dres, O.CODEC_FP8, 0, ws)
    torch.cuda.synchronize()
    for b, n in enumerate(sizes):
        want, _, _, wres = O.bucket_allreduce_ef(hb[b], res[b], (n + 255) // 256 * 256, O.CODEC_FP8, 0)
        assert (bits(outs[b].cpu().numpy()) == bits(want)).all(), f"bucket {b}"
        for r in range(k):
            assert (dres[b][r].cpu().numpy().view(np.uint32) == bits(wres[r])).all(), f"bucket {b} residual {r}"


def test_the_largest_batch(gb):
    """GB_MAX_BATCH buckets of 0..700 values (256 launches of 16), two ranks,
    fp8 with power-of-two scales: every bucket equals gb_bucket_allreduce_local
    on that bucket alone."""
    rng = np.random.default_rng(4100)
    sizes = [int(v) for v in rng.integers(0, 701, gb.GB_MAX_BATCH)]
    k = 2
    big = [W.device_gradients(sum(sizes), 4101 + r, DEV) for r in range(k)]
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]]).tolist()
    # each bucket in its own 16-byte-aligned buffer
    x = [[big[r][s:s + n].clone() for r in range(k)] for s, n in zip(starts, sizes)]
    outs = [torch.empty(n, device=DEV) for n in sizes]
    ws = torch.empty(gb.gb_bucket_batch_workspace_bytes(O.CODEC_FP8, k, sizes), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch(outs, x, O.CODEC_FP8, O.SCALE_POW2, ws)
    w1 = torch.empty(gb.gb_bucket_workspace_bytes(O.CODEC_FP8, k, 768, 768), dtype=torch.uint8, device=DEV)
    ref = [torch.empty(n, device=DEV) for n in sizes]
    for r_out, n, xs in zip(ref, sizes, x):
        if n:
            gb.gb_bucket_allreduce_local(r_out, xs, 768, O.CODEC_FP8, O.SCALE_POW2, w1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs).view(torch.int32), torch.cat(ref).view(torch.int32))


def avg_of(total, dt, d):
    """The oracle's AVG of a bucket's total: its SUM divided as the README's
    AVG divides it (float32: O.reduce; other types: O.reduce_typed)."""
    if dt == "f32":
        return O.reduce([total], O.OP_AVG, d)
    return O.reduce_typed([total], dt, O.OP_AVG, d)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16", "f64"])
@pytest.mark.parametrize("codec,mode", CODECS + [(O.CODEC_NONE, 0)])
@pytest.mark.parametrize("d", [2, 3, 8, (1 << 24) - 1, 1 << 24])
def test_avg_matches_the_oracle(gb, dt, codec, mode, d):
    """AVG over world size d: each bucket's compressed SUM from the oracle,
    divided by the oracle's AVG (fused into the pass for float32 totals); with
    codec NONE the oracle's exact AVG of the type."""
    k = 4
    sizes = [1000, 0, 4096 * 3 + 17, 256, 1, 20_000] + [513] * 12  # 17 non-empty: two launches
    hb = [[W.typed(n, dt, 4200 + 50 * b + r) for r in range(k)] for b, n in enumerate(sizes)]
    db = [[dev_typed(x, dt) for x in xs] for xs in hb]
    outs = [torch.empty(n, dtype=db[b][0].dtype, device=DEV) for b, n in enumerate(sizes)]
    need = gb.gb_bucket_batch_workspace_bytes(codec, k, sizes)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV) if need else None
    gb.gb_bucket_allreduce_local_batch(outs, db, codec, mode, ws, divisor=d)
    torch.cuda.synchronize()
    for b, n in enumerate(sizes):
        if n == 0:
            continue
        if codec == O.CODEC_NONE:
            want = O.reduce(hb[b], O.OP_AVG, d) if dt == "f32" else O.reduce_typed(hb[b], dt, O.OP_AVG, d)
        else:
            want = avg_of(O.bucket_allreduce_typed(hb[b], dt, (n + 255) // 256 * 256, codec, mode)[0], dt, d)
        what = f"dt={dt} codec={codec} mode={mode} d={d} bucket {b} (n={n})"
        assert host_typed(outs[b], dt).tobytes() == np.ascontiguousarray(want).tobytes(), what


@pytest.mark.parametrize("dt,codec", [("f32", O.CODEC_FP8), ("f32", O.CODEC_BF16), ("bf16", O.CODEC_FP8),
                                      ("f64", O.CODEC_BF16)])
@pytest.mark.parametrize("d", [4, 6])
def test_avg_with_error_feedback(gb, dt, codec, d):
    """The error-feedback batch with AVG: residuals as for SUM, each total
    divided as above, over two steps."""
    k, sizes = 3, [700, 4096 + 9, 0, 256]
    res = [[np.zeros(n, np.float32) for _ in range(k)] for n in sizes]
    dres = [[torch.zeros(n, device=DEV) for _ in range(k)] for n in sizes]
    ws = torch.empty(gb.gb_bucket_batch_workspace_bytes(codec, k, sizes), dtype=torch.uint8, device=DEV)
    for step in range(2):
        hb = [[W.typed(n, dt, 4300 + 100 * step + 10 * b + r) for r in range(k)] for b, n in enumerate(sizes)]
        db = [[dev_typed(x, dt) for x in xs] for xs in hb]
        outs = [torch.empty(n, dtype=db[b][0].dtype, device=DEV) for b, n in enumerate(sizes)]
        gb.gb_bucket_allreduce_local_batch_ef(outs, db, dres, codec, 0, ws, divisor=d)
        torch.cuda.synchronize()
        for b, n in enumerate(sizes):
            if n == 0:
                continue
            total, _, _, res[b] = O.bucket_allreduce_ef_typed(hb[b], res[b], dt, (n + 255) // 256 * 256, codec, 0)
            what = f"dt={dt} codec={codec} d={d} step={step} bucket {b}"
            assert host_typed(outs[b], dt).tobytes() == np.ascontiguousarray(avg_of(total, dt, d)).tobytes(), what
            for r in range(k):
                assert (dres[b][r].cpu().numpy().view(np.uint32) == bits(res[b][r])).all(), what + f" residual {r}"


def test_avg_with_more_ranks_than_one_launch_reads(gb):
    """11 ranks (one bucket at a time, then the division in a second pass)."""
    k, sizes, d = 11, [1000, 4096 + 3], 11
    hb = [[W.gradients(n, 4400 + 20 * b + r) for r in range(k)] for b, n in enumerate(sizes)]
    db = [[torch.from_numpy(x.copy()).to(DEV) for x in xs] for xs in hb]
    outs = [torch.empty(n, device=DEV) for n in sizes]
    ws = torch.empty(gb.gb_bucket_batch_workspace_bytes(O.CODEC_FP8, k, sizes), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch(outs, db, O.CODEC_FP8, 0, ws, divisor=d)
    torch.cuda.synchronize()
    for b, n in enumerate(sizes):
        total = O.bucket_allreduce(hb[b], (n + 255) // 256 * 256, O.CODEC_FP8, 0)[0]
        assert (bits(outs[b].cpu().numpy()) == bits(avg_of(total, "f32", d))).all(), f"bucket {b}"


@pytest.mark.parametrize("codec,n,ef", [
    (O.CODEC_FP8, 410_000_000 + 4096 * 7 + 99, False),  # above the fp8 passes' permuted-order size
    (O.CODEC_FP8, 410_000_000 + 4096 * 7 + 99, True),
    (O.CODEC_BF16, 72_000_000 + 1234, False),            # above the vector passes' permuted-order size
    (O.CODEC_BF16, 72_000_000 + 1234, True),
])
def test_one_large_bucket_equals_the_single_buffer_call(gb, codec, n, ef):
    """A batch of one bucket large enough to take the permuted workgroup
    order and the large launches' occupancy cap gives the single-buffer
    call's bits: output, payloads and residuals."""
    k = 2
    x = [W.device_gradients(n, 4500 + r, DEV) for r in range(k)]
    need = gb.gb_bucket_batch_workspace_bytes(codec, k, [n])
    assert need == gb.gb_bucket_workspace_bytes(codec, k, n, 256)
    w1 = torch.zeros(need, dtype=torch.uint8, device=DEV)
    w2 = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o1, o2 = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
    if ef:
        r1 = [torch.full((n,), 3e-5, device=DEV) for _ in range(k)]
        r2 = [t.clone() for t in r1]
        gb.gb_bucket_allreduce_local_ef(o1, x, r1, 256 * 25_600, codec, 0, w1)
        gb.gb_bucket_allreduce_local_batch_ef([o2], [x], [r2], codec, 0, w2)
    else:
        gb.gb_bucket_allreduce_local(o1, x, 256 * 25_600, codec, 0, w1)
        gb.gb_bucket_allreduce_local_batch([o2], [x], codec, 0, w2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(w1, w2)
    if ef:
        for a, b in zip(r1, r2):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_half_precision_batch_takes_eight_per_lane(gb, dt):
    """A bf16-codec batch over 4 ranks of float16 or bfloat16 gradients whose
    largest bucket has 2^22 values or more runs 8 values per lane, as the
    single-buffer call does on that bucket: every bucket's total and codes
    must equal the single-buffer call on it, the small buckets included."""
    k, codec = 4, gb.GB_CODEC_BF16
    sizes = [(1 << 22) + 77, 300, 1, 5003, 513]
    xs = [[W.device_gradients_typed(n, 4800 + 10 * b + r, DEV, dt) for r in range(k)] for b, n in enumerate(sizes)]
    outs = [torch.empty(n, dtype=xs[b][0].dtype, device=DEV) for b, n in enumerate(sizes)]
    ws = torch.zeros(gb.gb_bucket_batch_workspace_bytes(codec, k, sizes), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch(outs, xs, codec, workspace=ws)
    torch.cuda.synchronize()
    for b, n in enumerate(sizes):
        ref = torch.empty_like(outs[b])
        bucket = (n + 255) // 256 * 256  # one bucket
        w1 = torch.zeros(gb.gb_bucket_workspace_bytes(codec, k, n, bucket), dtype=torch.uint8, device=DEV)
        gb.gb_bucket_allreduce_local_typed(ref, xs[b], bucket, codec, 0, w1)
        torch.cuda.synchronize()
        assert torch.equal(outs[b].view(torch.int16), ref.view(torch.int16)), f"bucket {b} (n={n})"
