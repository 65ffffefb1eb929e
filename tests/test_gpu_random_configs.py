"""Randomised parity: many drawn configurations of every bucket-stream and
reduction call, the batched bucket calls among them (rank count 1..16, odd
sizes and bucket lengths, each codec and scale mode, every element type, in
place or not, with or without error feedback over every floating type), each
checked bit for bit against the oracle.  The draws are seeded, so a failure
names a reproducible case."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64,
         "i8": torch.int8, "u8": torch.uint8, "i32": torch.int32, "i64": torch.int64}


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def draw_values(rng, dt, n):
    """Gradient-like values with outliers, zeros of both signs and, now and
    then, a whole block of tiny values or special values (Inf, NaN, the
    extremes of the type)."""
    v = rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 1)
    v[rng.random(n) < 0.01] *= 300.0
    v[rng.random(n) < 0.003] = 0.0
    v[rng.random(n) < 0.003] = -0.0
    if n > 600 and rng.random() < 0.3:
        s = int(rng.integers(0, n - 256))
        v[s:s + 256] *= 1e-30
    if rng.random() < 0.15:
        # special values now and then: infinities, NaNs of both signs, the
        # float32 extremes, a float32 subnormal, -0 and float16's edge
        specials = np.array([np.inf, -np.inf, np.nan, -np.nan, 3.4e38, -3.4e38, 1e-45, -0.0, 65504.0, 1e5])
        where = rng.choice(n, max(1, n // 500), replace=False)
        v[where] = rng.choice(specials, where.size)
    if dt == "f64":
        return v
    if dt == "f32":
        return v.astype(np.float32)
    if dt in ("f16", "bf16"):
        return torch.from_numpy(v.astype(np.float32)).to(TORCH[dt]).view(torch.int16).numpy().view(np.uint16)
    info = np.iinfo(O.NP_DTYPES[dt])
    return rng.integers(info.min, info.max, n, endpoint=True, dtype=O.NP_DTYPES[dt])


def to_dev(a, dt):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 and dt in ("f16", "bf16"):
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(TORCH[dt])
    return torch.from_numpy(a).to(DEV)


def to_host(t):
    if t.element_size() == 2 and t.is_floating_point():
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def same(got, want, dt, what, nan_as_nan=False):
    """Every byte equal, NaN included: every NaN the float arithmetic delivers
    is the canonical one on both sides.  The exact reductions of the other
    element types (nan_as_nan) compare NaN as NaN: their payloads are the
    reading on format conversions, not pinned."""
    if not nan_as_nan:
        assert got.tobytes() == want.tobytes(), f"{what}: values differ"
        return
    if dt in ("f32", "f64"):
        gn, wn = np.isnan(got), np.isnan(want)
    elif dt in ("f16", "bf16"):
        f = (lambda a: a.view(np.float16)) if dt == "f16" else (lambda a: (a.astype(np.uint32) << 16).view(np.float32))
        gn, wn = np.isnan(f(got)), np.isnan(f(want))
    else:
        gn = wn = np.zeros(got.size, bool)
    assert (gn == wn).all(), f"{what}: NaN positions differ"
    assert got[~gn].tobytes() == want[~wn].tobytes(), f"{what}: values differ"


@pytest.mark.parametrize("seed", range(400))
def test_bucket_stream(gb, seed):
    rng = np.random.default_rng(7000 + seed)
    k = int(rng.integers(1, 17))
    bucket = 256 * int(rng.integers(1, 40))
    n = int(rng.integers(1, 12 * bucket))
    codec = int(rng.integers(0, 3))
    mode = int(rng.integers(0, 2))
    dt = str(rng.choice(["f32", "f32", "f16", "bf16", "f64"]))
    if codec != 0 and dt != "f32" and k > 8:
        k = int(rng.integers(1, 9))
    ef = codec != 0 and rng.random() < 0.3
    in_place = rng.random() < 0.3
    what = f"seed={seed} k={k} n={n} bucket={bucket} codec={codec} mode={mode} dt={dt} ef={ef} in_place={in_place}"
    xs = [draw_values(rng, dt, n) for _ in range(k)]
    d = [to_dev(x, dt) for x in xs]
    out = d[0] if in_place else torch.empty(n, dtype=TORCH[dt], device=DEV)
    need = gb.gb_bucket_workspace_bytes(codec, k, n, bucket)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV) if codec else None
    if ef:
        res0 = [(rng.standard_normal(n) * 1e-4).astype(np.float32) for _ in range(k)]
        res = [to_dev(r, "f32") for r in res0]
        if dt == "f32":
            gb.gb_bucket_allreduce_local_ef(out, d, res, bucket, codec, mode, ws)
        else:
            gb.gb_bucket_allreduce_local_ef_typed(out, d, res, bucket, codec, mode, ws)
        torch.cuda.synchronize()
        want, _, _, res1 = O.bucket_allreduce_ef_typed(xs, res0, dt, bucket, codec, mode)
        for r in range(k):
            same(res[r].cpu().numpy(), res1[r], "f32", what + f" residual {r}")
    else:
        if dt == "f32":
            gb.gb_bucket_allreduce_local(out, d, bucket, codec, mode, ws)
        else:
            gb.gb_bucket_allreduce_local_typed(out, d, bucket, codec, mode, ws)
        torch.cuda.synchronize()
        want, _, _ = O.bucket_allreduce_typed(xs, dt, bucket, codec, mode)
    same(to_host(out), want, dt, what, nan_as_nan=codec == 0 and dt != "f32")


@pytest.mark.parametrize("seed", range(120))
def test_batched_bucket_stream(gb, seed):
    """gb_bucket_allreduce_local_batch (and _batch_ef): a drawn list of 1..40
    buckets of 0..5000 values, each checked against the oracle's bucket
    stream of that bucket alone."""
    rng = np.random.default_rng(9000 + seed)
    nb = int(rng.integers(1, 41))
    sizes = [int(v) for v in rng.integers(0, 5001, nb)]
    codec = int(rng.integers(0, 3))
    mode = int(rng.integers(0, 2))
    dt = str(rng.choice(["f32", "f32", "f16", "bf16", "f64"]))
    k = int(rng.integers(1, 17)) if dt == "f32" or codec == 0 else int(rng.integers(1, 9))
    ef = codec != 0 and rng.random() < 0.4
    what = f"seed={seed} nb={nb} k={k} codec={codec} mode={mode} dt={dt} ef={ef}"
    empty = np.empty(0, {"f32": np.float32, "f64": np.float64}.get(dt, np.uint16))
    xs = [[draw_values(rng, dt, n) if n else empty for _ in range(k)] for n in sizes]
    d = [[to_dev(x, dt) for x in xb] for xb in xs]
    outs = [torch.empty(n, dtype=TORCH[dt], device=DEV) for n in sizes]
    need = gb.gb_bucket_batch_workspace_bytes(codec, k, sizes)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV) if codec else None
    if ef:
        res0 = [[(rng.standard_normal(n) * 1e-4).astype(np.float32) for _ in range(k)] for n in sizes]
        res = [[to_dev(r, "f32") for r in rb] for rb in res0]
        gb.gb_bucket_allreduce_local_batch_ef(outs, d, res, codec, mode, ws)
    else:
        gb.gb_bucket_allreduce_local_batch(outs, d, codec, mode, ws)
    torch.cuda.synchronize()
    for b, n in enumerate(sizes):
        if n == 0:
            continue
        bucket = (n + 255) // 256 * 256
        if ef:
            want, _, _, res1 = O.bucket_allreduce_ef_typed(xs[b], res0[b], dt, bucket, codec, mode)
            for r in range(k):
                same(res[b][r].cpu().numpy(), res1[r], "f32", what + f" bucket {b} residual {r}")
        else:
            want, _, _ = O.bucket_allreduce_typed(xs[b], dt, bucket, codec, mode)
        same(to_host(outs[b]), want, dt, what + f" bucket {b}", nan_as_nan=codec == 0 and dt != "f32")


@pytest.mark.parametrize("seed", range(400))
def test_reduction(gb, seed):
    rng = np.random.default_rng(8000 + seed)
    k = int(rng.integers(1, 17))
    n = int(rng.integers(1, 200_000))
    dt = str(rng.choice(list(TORCH)))
    ops = [0, 2, 3] if dt in ("i8", "u8", "i32", "i64") else [0, 1, 2, 3]
    op = int(rng.choice(ops))
    divisor = int(rng.choice([1, 2, 3, 8, 12, 1000, 1 << 24])) if op == 1 else 1
    in_place = rng.random() < 0.3
    what = f"seed={seed} k={k} n={n} dt={dt} op={op} divisor={divisor} in_place={in_place}"
    xs = [draw_values(rng, dt, n) for _ in range(k)]
    d = [to_dev(x, dt) for x in xs]
    out = d[0] if in_place else torch.empty(n, dtype=TORCH[dt], device=DEV)
    gb.gb_reduce_typed(out, d, op, divisor)
    torch.cuda.synchronize()
    same(to_host(out), O.reduce_typed(xs, dt, op, divisor), dt, what, nan_as_nan=dt != "f32")


@pytest.mark.parametrize("seed", range(160))
def test_encode_decode(gb, seed):
    rng = np.random.default_rng(9000 + seed)
    k = int(rng.integers(1, 9))
    n = int(rng.integers(1, 300_000))
    codec = int(rng.integers(1, 3))
    mode = int(rng.integers(0, 2))
    dt = str(rng.choice(["f32", "f16", "bf16", "f64"]))
    what = f"seed={seed} k={k} n={n} codec={codec} mode={mode} dt={dt}"
    xs = [draw_values(rng, dt, n) for _ in range(k)]
    codes, scales = [], []
    for x in xs:
        c = torch.empty(n, dtype=torch.uint16 if codec == 1 else torch.uint8, device=DEV)
        s = torch.empty(O.nblocks(n), device=DEV) if codec == 2 else None
        gb.gb_encode(codec, c, s, to_dev(x, dt), mode)
        codes.append(c)
        scales.append(s)
    out = torch.empty(n, dtype=TORCH[dt], device=DEV)
    gb.gb_decode_sum(out, codes, scales if codec == 2 else None, codec)
    torch.cuda.synchronize()
    enc = [O.encode_typed(x, dt, codec, mode) for x in xs]
    for r in range(k):
        got = codes[r].view(torch.int16).cpu().numpy().view(np.uint16) if codec == 1 else codes[r].cpu().numpy()
        assert (got == enc[r][0]).all(), what + f" codes {r}"
        if codec == 2:
            assert (scales[r].cpu().numpy().view(np.uint32) == enc[r][1].view(np.uint32)).all(), what + f" scales {r}"
    want = O.decode_sum_typed([c for c, _ in enc], [s for _, s in enc] if codec == 2 else None, codec, dt)
    same(to_host(out), want, dt, what)
