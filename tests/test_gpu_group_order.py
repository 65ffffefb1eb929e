"""Launches whose workgroups take another shape than the small-launch path:
- the permuted workgroup order of the streaming kernels, from 16 runs of
  2048 groups (about 3.4e7 values) for the kernels over 1024-value vector
  groups, from 8 runs (about 1.7e7 values) for the fused bf16-codec passes
  over float32 gradients of one or two ranks and the batch kernels, from 4
  runs (2^23 values) for the bf16 decode into float32, from 64 MiB per rank
  for the reductions, and from about 4e8 values for the kernels over
  4096-value fp8 groups;
- the wide four-rank sum, from 2^28 values;
- the fused fp8 pass in 128-lane workgroups (float32 gradients from 2^27
  values, 2^28 over two ranks, but not over 4; float64 gradients from
  3 * 2^21 values), and one block per 64-lane workgroup (float32 gradients
  of 4 ranks from 2^22 values, with error feedback also over float16 and
  bfloat16 gradients, the batch of such a bucket too; the decode of 4
  payloads into float32 from 2^24);
- the fused bf16 pass in 64-lane workgroups (float32 gradients from 3
  ranks; float16 and bfloat16 gradients from 5 ranks and 2^22 values, and
  over 4 ranks from 2^22 with 8 values per lane; with error feedback, over
  float32 gradients from 1 rank and over the other types by rank count and
  size).

Each must give, bit for bit, what the same arithmetic gives in another
shape: over slices of the stream small enough to keep the index order and
the narrow shape, or through the batch kernel; the new shapes are also
checked against the oracle on sampled windows.

Every result is elementwise (per value, or per 256-value fp8 block), so a
call over a slice that starts on a bucket boundary computes exactly that
slice of the whole call; the small-launch path is checked against the oracle
by the other GPU tests, and the 1e9-value fp8 bucket stream against the
oracle on every value.  Outputs start filled with a sentinel, so a group
that no workgroup took shows as a difference.  Sizes end in a ragged tail
that is not a whole number of runs of the permutation."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W  # noqa: E402

DEV = "cuda:0"
B = W.DDP_BUCKET  # 6,553,600 values: a multiple of 4096
N_VEC = 72_000_000 + 1234  # > 16 runs of 2048 groups of 2048 values
N_BLK = 410_000_000 + 4096 * 7 + 99  # > 96 runs of 1024 groups of 4096 values
STEP_VEC = 5 * B  # 32,768,000 values: fewer than 16 runs of 1024-value groups
STEP_DEC = B  # 6,553,600 values: fewer than the bf16 decode's 4 runs (2^23 values)
STEP_RED = 2 * B  # 13,107,200 values: fewer than 8 runs of the reductions' 4 KiB groups (float32)
STEP_BLK = 50 * B  # 327,680,000 values: fewer than 96 runs of 4096-value groups
STEP_HALF = 20 * B  # 131,072,000 values: below 2^27, where the fused fp8 pass keeps 256-lane workgroups
SENTINEL = 0x7FBADBAD  # a float32 NaN no kernel writes


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def slices(n, step):
    return [(s, min(s + step, n)) for s in range(0, n, step)]


def filled(n, dtype=torch.float32):
    t = torch.empty(n, dtype=dtype, device=DEV)
    if t.element_size() == 4:
        t.view(torch.int32).fill_(SENTINEL)
    else:
        t.view(torch.uint8).fill_(0xFF)
    return t


def bits(t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()])


def same(a, b, what):
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b)), what


def test_vector_group_kernels(gb):
    n = N_VEC
    x = [W.device_gradients(n, 900 + r, DEV) for r in range(3)]
    parts = slices(n, STEP_VEC)

    # fixed-order sum and AVG
    for op, div in ((None, 1), (gb.GB_OP_AVG, 3)):
        whole, ref = filled(n), filled(n)
        call = (lambda o, s: gb.gb_reduce_sum(o, s)) if op is None else (lambda o, s: gb.gb_reduce(o, s, op, div))
        call(whole, x)
        for s, e in slices(n, STEP_RED):
            call(ref[s:e], [t[s:e] for t in x])
        same(whole, ref, f"reduce op={op}")

    # bf16 encode (two vectors per lane at this size) and decode-accumulate
    cw, cr = filled(n, torch.uint16), filled(n, torch.uint16)
    gb.gb_encode_bf16(cw, x[0])
    for s, e in parts:
        gb.gb_encode_bf16(cr[s:e], x[0][s:e])
    same(cw, cr, "encode bf16")
    c2 = torch.empty(n, dtype=torch.uint16, device=DEV)
    gb.gb_encode_bf16(c2, x[1])
    whole, ref = filled(n), filled(n)
    gb.gb_decode_accumulate(whole, [cw, c2], None, gb.GB_CODEC_BF16)
    for s, e in slices(n, STEP_DEC):
        gb.gb_decode_accumulate(ref[s:e], [cw[s:e], c2[s:e]], None, gb.GB_CODEC_BF16)
    same(whole, ref, "decode bf16")

    # the bf16 bucket stream, plain and with error feedback (float32
    # gradients: permuted from 8 runs, so the reference slices stay below)
    ws = torch.empty(gb.gb_bucket_workspace_bytes(gb.GB_CODEC_BF16, 3, n, B), dtype=torch.uint8, device=DEV)
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local(whole, x, B, gb.GB_CODEC_BF16, 0, ws)
    for s, e in slices(n, STEP_RED):
        gb.gb_bucket_allreduce_local(ref[s:e], [t[s:e] for t in x], B, gb.GB_CODEC_BF16, 0, ws)
    same(whole, ref, "bf16 bucket stream")
    rw = [torch.full((n,), 1e-5, device=DEV) for _ in range(3)]
    rr = [t.clone() for t in rw]
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local_ef(whole, x, rw, B, gb.GB_CODEC_BF16, 0, ws)
    for s, e in slices(n, STEP_RED):
        gb.gb_bucket_allreduce_local_ef(ref[s:e], [t[s:e] for t in x], [t[s:e] for t in rr], B,
                                        gb.GB_CODEC_BF16, 0, ws)
    same(whole, ref, "bf16 bucket stream with error feedback")
    for r in range(3):
        same(rw[r], rr[r], f"bf16 residual {r}")
    del rw, rr

    # island sum with its bf16 payload
    sw, sr = filled(n), filled(n)
    cw.view(torch.uint8).fill_(0xFF)
    cr.view(torch.uint8).fill_(0xFF)
    gb.gb_reduce_encode(gb.GB_CODEC_BF16, cw, None, x, sum=sw)
    for s, e in parts:
        gb.gb_reduce_encode(gb.GB_CODEC_BF16, cr[s:e], None, [t[s:e] for t in x], sum=sr[s:e])
    same(sw, sr, "reduce_encode bf16 sum")
    same(cw, cr, "reduce_encode bf16 codes")


def test_wide_four_rank_sum(gb):
    """The four-rank float32 sum from 2^28 values (4 vectors per lane, one
    workgroup per compute unit, its own order), with a ragged last group and
    in place, against the narrow kernel over slices below 2^28 and against
    the oracle on sampled windows (the first and last values included)."""
    import numpy as np
    from oracle import oracle as O
    n = (1 << 28) + 4096 * 3 + 77
    x = [W.device_gradients(n, 1100 + r, DEV) for r in range(4)]
    whole, ref = filled(n), filled(n)
    gb.gb_reduce_sum(whole, x)
    for s, e in slices(n, STEP_BLK // 4):
        gb.gb_reduce_sum(ref[s:e], [t[s:e] for t in x])
    same(whole, ref, "wide four-rank sum")
    rng = np.random.default_rng(5)
    for s in [0, n - 100_000] + [int(v) for v in rng.integers(0, n - 100_000, 6)]:
        got = whole[s:s + 100_000].cpu().numpy()
        want = O.reduce_sum([t[s:s + 100_000].cpu().numpy() for t in x])
        assert (got.view(np.uint32) == want.view(np.uint32)).all(), f"oracle window at {s}"
    x0 = x[0].clone()
    gb.gb_reduce_sum(x0, [x0] + x[1:])
    same(x0, ref, "wide four-rank sum in place")


@pytest.mark.parametrize("k", [2, 3, 5, 8])
def test_fused_fp8_half_workgroups(gb, k):
    """The fused fp8 bucket stream over float32 gradients from 2^27 values
    per rank (2^28 over two ranks; 4 ranks take the 64-lane shape below) runs
    in 128-lane workgroups in index order.  With a ragged last workgroup and
    block it must equal the 256-lane kernel over slices below 2^27, and the
    oracle on sampled windows (the first and the last values included):
    totals, codes and scales."""
    import numpy as np
    from oracle import oracle as O
    fp8 = gb.GB_CODEC_FP8_E4M3_B256
    n = ((1 << 28) if k == 2 else (1 << 27)) + 2048 * 5 + 77
    x = [W.device_gradients(n, 1200 + 10 * k + r, DEV) for r in range(k)]
    lay = gb.gb_bucket_workspace_layout(fp8, k, n, B)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local(whole, x, B, fp8, 0, ws)
    wss = torch.empty(gb.gb_bucket_workspace_bytes(fp8, k, STEP_HALF, B), dtype=torch.uint8, device=DEV)
    for s, e in slices(n, STEP_HALF):
        gb.gb_bucket_allreduce_local(ref[s:e], [t[s:e] for t in x], B, fp8, 0, wss)
    same(whole, ref, f"fused fp8 pass over {k} ranks")
    del ref, wss
    nb = (n + 255) // 256
    codes = [ws[r * lay["codes_stride"]:][:n] for r in range(k)]
    scales = [ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32) for r in range(k)]
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    length = 65536
    rng = np.random.default_rng(70 + k)
    last = (n - length) // 256 * 256
    for s in [0, last] + [int(v) * 256 for v in rng.integers(0, last // 256, 4)]:
        e = n if s == last else s + length
        want, wc, wsc = O.bucket_allreduce([t[s:e].cpu().numpy() for t in x], B, O.CODEC_FP8,
                                           O.SCALE_ABSMAX_DIV_448)
        assert (u32(whole[s:e].cpu().numpy()) == u32(want)).all(), f"oracle total window at {s}"
        for r in range(k):
            assert (codes[r][s:e].cpu().numpy() == wc[r]).all(), f"oracle codes, rank {r}, window at {s}"
            got = scales[r][s // 256:(e + 255) // 256].cpu().numpy()
            assert (u32(got) == u32(wsc[r])).all(), f"oracle scales, rank {r}, window at {s}"


F64_LO = 3 << 21


@pytest.mark.parametrize("dt,k,n", [
    ("f64", 2, F64_LO + 2048 * 5 + 77), ("f64", 3, F64_LO + 2048 * 5 + 77), ("f64", 4, F64_LO + 2048 * 5 + 77),
    ("f64", 8, F64_LO + 2048 * 5 + 77), ("f64", 4, F64_LO - 2048 - 77)])
def test_fused_fp8_half_typed_workgroups(gb, dt, k, n):
    """The fused fp8 bucket stream runs in 128-lane workgroups in index order
    over float64 gradients from 3 * 2^21 values per rank (2 per CU; over 4
    or more ranks below 2^29), in 256-lane ones below.  On either side of
    the threshold, with a ragged last workgroup and block, it must equal the
    256-lane batch kernel on the same buffers (a batch of one bucket), and
    the oracle on sampled windows (the first and the last values included):
    totals, codes and scales."""
    import numpy as np
    from oracle import oracle as O
    fp8 = gb.GB_CODEC_FP8_E4M3_B256
    x = [W.device_gradients_typed(n, 1700 + 10 * k + r, DEV, dt) for r in range(k)]
    lay = gb.gb_bucket_workspace_layout(fp8, k, n, B)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
    gb.gb_bucket_allreduce_local_typed(whole, x, B, fp8, 0, ws)
    wsb = torch.empty(gb.gb_bucket_batch_workspace_bytes(fp8, k, [n]), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch([ref], [x], fp8, workspace=wsb)
    same(whole, ref, f"fused fp8 pass over {k} ranks of {dt} against the batch kernel")
    del ref, wsb
    nb = (n + 255) // 256
    codes = [ws[r * lay["codes_stride"]:][:n] for r in range(k)]
    scales = [ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32) for r in range(k)]
    host = lambda t: bits(t).cpu().numpy()
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    length = 65536
    rng = np.random.default_rng(150 + k)
    last = (n - length) // 256 * 256
    for s in [0, last] + [int(v) * 256 for v in rng.integers(0, last // 256, 3)]:
        e = n if s == last else s + length
        xs = [host(t[s:e]).view(np.uint16) if dt != "f64" else t[s:e].cpu().numpy() for t in x]
        want, wc, wsc = O.bucket_allreduce_typed(xs, dt, B, O.CODEC_FP8, O.SCALE_ABSMAX_DIV_448)
        assert (host(whole[s:e]) == np.ascontiguousarray(want).view(host(whole[:1]).dtype)).all(), \
            f"oracle total window at {s}"
        for r in range(k):
            assert (codes[r][s:e].cpu().numpy() == wc[r]).all(), f"oracle codes, rank {r}, window at {s}"
            got = scales[r][s // 256:(e + 255) // 256].cpu().numpy()
            assert (u32(got) == u32(wsc[r])).all(), f"oracle scales, rank {r}, window at {s}"


def plant_specials(x, n, last):
    """NaN, Inf, a block whose scale is subnormal, a block of negative zeros
    and the largest finite magnitude, in the first window and the last, and
    a NaN in the ragged last block."""
    for base in (0, last):
        x[0][base + 3 * 256 + 17] = float("nan")
        x[1][base + 5 * 256 + 200] = float("inf")
        x[2][base + 5 * 256 + 9] = -float("inf")
        x[3][base + 7 * 256:base + 8 * 256] = 3e-41  # scale 3e-41 / 448, subnormal
        x[1][base + 9 * 256:base + 10 * 256] = -0.0
        x[2][base + 11 * 256 + 63] = -3.4028234663852886e38
        x[0][base + 11 * 256 + 64] = float("nan")
    x[3][n - 1] = float("nan")


@pytest.mark.parametrize("n", [(1 << 22) + 256 * 5 + 77, (1 << 22) - 77, (1 << 27) + 256 * 5 + 77])
def test_fused_fp8_wave_workgroups(gb, n):
    """The fused fp8 bucket stream over float32 gradients of 4 ranks runs one
    256-value block per 64-lane workgroup from 2^22 values per rank, in
    256-lane workgroups below.  On either side of the threshold and at 2^27,
    with a ragged last block and special values planted in the first and the
    last window, it must equal the 256-lane kernel over slices below 2^22,
    and the oracle on the first, the last and sampled windows: totals, codes
    and scales.  A batch of that one bucket takes the same shape and must give
    the same bits, and its AVG the oracle's AVG of that total."""
    import numpy as np
    from oracle import oracle as O
    fp8, k = gb.GB_CODEC_FP8_E4M3_B256, 4
    x = [W.device_gradients(n, 1900 + r, DEV) for r in range(k)]
    last = (n - 65536) // 256 * 256
    plant_specials(x, n, last)
    lay = gb.gb_bucket_workspace_layout(fp8, k, n, B)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=DEV)
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local(whole, x, B, fp8, 0, ws)
    step = 3 * (1 << 20)  # below 2^22, a multiple of 256
    wss = torch.empty(gb.gb_bucket_workspace_bytes(fp8, k, step, step), dtype=torch.uint8, device=DEV)
    for s, e in slices(n, step):
        gb.gb_bucket_allreduce_local(ref[s:e], [t[s:e] for t in x], step, fp8, 0, wss)
    same(whole, ref, "fused fp8 pass over 4 ranks against 256-lane slices")
    del wss
    need = gb.gb_bucket_batch_workspace_bytes(fp8, k, [n])
    assert need == lay["total"]
    wsb = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ref.fill_(0.0)
    gb.gb_bucket_allreduce_local_batch([ref], [x], fp8, workspace=wsb)
    same(whole, ref, "a batch of the one bucket")
    assert torch.equal(ws, wsb), "the batch's payloads"
    del wsb
    nb = (n + 255) // 256
    codes = [ws[r * lay["codes_stride"]:][:n] for r in range(k)]
    scales = [ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32) for r in range(k)]
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    rng = np.random.default_rng(190)
    for s in [0, last] + [int(v) * 256 for v in rng.integers(0, last // 256, 3)]:
        e = n if s == last else s + 65536
        want, wc, wsc = O.bucket_allreduce([t[s:e].cpu().numpy() for t in x], B, O.CODEC_FP8,
                                           O.SCALE_ABSMAX_DIV_448)
        assert (u32(whole[s:e].cpu().numpy()) == u32(want)).all(), f"oracle total window at {s}"
        for r in range(k):
            assert (codes[r][s:e].cpu().numpy() == wc[r]).all(), f"oracle codes, rank {r}, window at {s}"
            got = scales[r][s // 256:(e + 255) // 256].cpu().numpy()
            assert (u32(got) == u32(wsc[r])).all(), f"oracle scales, rank {r}, window at {s}"
    total = whole.cpu().numpy()
    for d in (4, 3):  # the exact reciprocal of a power of two, and a divide
        wsb = torch.empty(need, dtype=torch.uint8, device=DEV)
        ref.fill_(0.0)
        gb.gb_bucket_allreduce_local_batch([ref], [x], fp8, workspace=wsb, divisor=d)
        want = O.reduce([total], O.OP_AVG, d)
        assert (u32(ref.cpu().numpy()) == u32(want)).all(), f"AVG over {d}"
        del wsb


@pytest.mark.parametrize("n", [(1 << 22) + 256 * 5 + 77, (1 << 22) - 77, (1 << 27) + 256 * 5 + 77])
def test_fused_fp8_ef_wave_workgroups(gb, n):
    """The fp8 bucket stream with error feedback over float32 gradients of 4
    ranks runs one 256-value block per 64-lane workgroup from 2^22 values per
    rank, in 256-lane workgroups below.  On either side of the threshold and
    at 2^27, with a ragged last block and special values planted in
    gradients and a residual, it must equal the 256-lane kernel over slices
    below 2^22 from the same residuals, and the oracle on the first, the last and sampled
    windows: totals, codes, scales and the new residuals.  A batch of that
    one bucket takes the same shape and must give the same bits, and its AVG
    the oracle's AVG of that total."""
    import numpy as np
    from oracle import oracle as O
    fp8, k = gb.GB_CODEC_FP8_E4M3_B256, 4
    x = [W.device_gradients(n, 2000 + r, DEV) for r in range(k)]
    last = (n - 65536) // 256 * 256
    plant_specials(x, n, last)
    r0 = [W.device_gradients(n, 2100 + r, DEV) * 1e-2 for r in range(k)]
    for base in (0, last):
        r0[2][base + 13 * 256 + 5] = float("nan")
        r0[0][base + 14 * 256:base + 15 * 256] = -3e-41
    lay = gb.gb_bucket_workspace_layout(fp8, k, n, B)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=DEV)
    rw = [t.clone() for t in r0]
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local_ef(whole, x, rw, B, fp8, 0, ws)
    rs = [t.clone() for t in r0]
    step = 3 * (1 << 20)  # below 2^22, a multiple of 256
    wss = torch.empty(gb.gb_bucket_workspace_bytes(fp8, k, step, step), dtype=torch.uint8, device=DEV)
    for s, e in slices(n, step):
        gb.gb_bucket_allreduce_local_ef(ref[s:e], [t[s:e] for t in x], [t[s:e] for t in rs], step, fp8, 0, wss)
    same(whole, ref, "fp8 pass with error feedback against 256-lane slices")
    for r in range(k):
        same(rw[r], rs[r], f"residual {r} against 256-lane slices")
    del wss, rs
    need = gb.gb_bucket_batch_workspace_bytes(fp8, k, [n])
    assert need == lay["total"]
    wsb = torch.zeros(need, dtype=torch.uint8, device=DEV)
    rb = [t.clone() for t in r0]
    ref.fill_(0.0)
    gb.gb_bucket_allreduce_local_batch_ef([ref], [x], [rb], fp8, 0, wsb)
    same(whole, ref, "a batch of the one bucket")
    assert torch.equal(ws, wsb), "the batch's payloads"
    for r in range(k):
        same(rw[r], rb[r], f"the batch's residual {r}")
    del wsb, rb
    nb = (n + 255) // 256
    codes = [ws[r * lay["codes_stride"]:][:n] for r in range(k)]
    scales = [ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32) for r in range(k)]
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    rng = np.random.default_rng(200)
    for s in [0, last] + [int(v) * 256 for v in rng.integers(0, last // 256, 3)]:
        e = n if s == last else s + 65536
        want, wc, wsc, wres = O.bucket_allreduce_ef([t[s:e].cpu().numpy() for t in x],
                                                    [t[s:e].cpu().numpy() for t in r0], B, O.CODEC_FP8,
                                                    O.SCALE_ABSMAX_DIV_448)
        assert (u32(whole[s:e].cpu().numpy()) == u32(want)).all(), f"oracle total window at {s}"
        for r in range(k):
            assert (codes[r][s:e].cpu().numpy() == wc[r]).all(), f"oracle codes, rank {r}, window at {s}"
            got = scales[r][s // 256:(e + 255) // 256].cpu().numpy()
            assert (u32(got) == u32(wsc[r])).all(), f"oracle scales, rank {r}, window at {s}"
            assert (u32(rw[r][s:e].cpu().numpy()) == u32(wres[r])).all(), f"oracle residual {r}, window at {s}"
    total = whole.cpu().numpy()
    for d in (4, 3):  # the exact reciprocal of a power of two, and a divide
        wsb = torch.empty(need, dtype=torch.uint8, device=DEV)
        rb = [t.clone() for t in r0]
        ref.fill_(0.0)
        gb.gb_bucket_allreduce_local_batch_ef([ref], [x], [rb], fp8, 0, wsb, divisor=d)
        want = O.reduce([total], O.OP_AVG, d)
        assert (u32(ref.cpu().numpy()) == u32(want)).all(), f"AVG over {d}"
        del wsb, rb


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("n", [(1 << 22) + 256 * 5 + 77, (1 << 22) - 77])
def test_fused_fp8_ef_wave_typed_workgroups(gb, dt, n):
    """The fp8 bucket stream with error feedback over bfloat16 and float16
    gradients of 4 ranks runs one 256-value block per 64-lane workgroup from
    2^22 values per rank, in 256-lane workgroups below.  On either side of
    the threshold, with a ragged last block and special values planted in a
    residual, it must equal the 256-lane kernel over slices below 2^22 from
    the same residuals, a batch of that one bucket, and the oracle on the
    first, the last and sampled windows: totals, codes, scales and the new
    residuals."""
    import numpy as np
    from oracle import oracle as O
    fp8, k = gb.GB_CODEC_FP8_E4M3_B256, 4
    x = [W.device_gradients_typed(n, 2400 + r, DEV, dt) for r in range(k)]
    last = (n - 65536) // 256 * 256
    x[1][n - 1] = float("inf")
    r0 = [W.device_gradients(n, 2500 + r, DEV) * 1e-2 for r in range(k)]
    for base in (0, last):
        r0[2][base + 13 * 256 + 5] = float("nan")
        r0[0][base + 14 * 256:base + 15 * 256] = -3e-41
        r0[3][base + 15 * 256 + 7] = 3e38
    lay = gb.gb_bucket_workspace_layout(fp8, k, n, B)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=DEV)
    rw = [t.clone() for t in r0]
    whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
    gb.gb_bucket_allreduce_local_ef_typed(whole, x, rw, B, fp8, 0, ws)
    rs = [t.clone() for t in r0]
    step = 3 * (1 << 20)  # below 2^22, a multiple of 256
    wss = torch.empty(gb.gb_bucket_workspace_bytes(fp8, k, step, step), dtype=torch.uint8, device=DEV)
    for s, e in slices(n, step):
        gb.gb_bucket_allreduce_local_ef_typed(ref[s:e], [t[s:e] for t in x], [t[s:e] for t in rs], step, fp8, 0, wss)
    same(whole, ref, f"{dt} error feedback against 256-lane slices")
    for r in range(k):
        same(rw[r], rs[r], f"{dt} residual {r} against 256-lane slices")
    del wss, rs
    wsb = torch.zeros(gb.gb_bucket_batch_workspace_bytes(fp8, k, [n]), dtype=torch.uint8, device=DEV)
    rb = [t.clone() for t in r0]
    ref.view(torch.int16).fill_(0)
    gb.gb_bucket_allreduce_local_batch_ef([ref], [x], [rb], fp8, 0, wsb)
    same(whole, ref, f"{dt}: a batch of the one bucket")
    assert torch.equal(ws, wsb), "the batch's payloads"
    for r in range(k):
        same(rw[r], rb[r], f"{dt}: the batch's residual {r}")
    del wsb, rb
    nb = (n + 255) // 256
    codes = [ws[r * lay["codes_stride"]:][:n] for r in range(k)]
    scales = [ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32) for r in range(k)]
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    rng = np.random.default_rng(220)
    for s in [0, last] + [int(v) * 256 for v in rng.integers(0, last // 256, 3)]:
        e = n if s == last else s + 65536
        xs = [bits(t[s:e]).cpu().numpy().view(np.uint16) for t in x]
        want, wc, wsc, wres = O.bucket_allreduce_ef_typed(xs, [t[s:e].cpu().numpy() for t in r0], dt, B,
                                                          O.CODEC_FP8, O.SCALE_ABSMAX_DIV_448)
        got = bits(whole[s:e]).cpu().numpy().view(np.uint16)
        assert (got == np.ascontiguousarray(want).view(np.uint16)).all(), f"oracle total window at {s}"
        for r in range(k):
            assert (codes[r][s:e].cpu().numpy() == wc[r]).all(), f"oracle codes, rank {r}, window at {s}"
            sc = scales[r][s // 256:(e + 255) // 256].cpu().numpy()
            assert (u32(sc) == u32(wsc[r])).all(), f"oracle scales, rank {r}, window at {s}"
            assert (u32(rw[r][s:e].cpu().numpy()) == u32(wres[r])).all(), f"oracle residual {r}, window at {s}"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("n", [(1 << 22) + 256 * 5 + 77, (1 << 22) - 77])
def test_fused_bf16_eight_per_lane(gb, dt, n):
    """The bf16-codec bucket stream over bfloat16 and float16 gradients of 4
    ranks takes 8 values per lane in 64-lane workgroups from 2^22 values per
    rank.  On either side of the threshold, with a ragged last lane and
    special values (Inf, NaN, the largest finite magnitude), it must equal
    the kernels below the threshold over slices, and the oracle on the
    first, the last and sampled windows: totals and codes."""
    import numpy as np
    from oracle import oracle as O
    bf16, k = gb.GB_CODEC_BF16, 4
    x = [W.device_gradients_typed(n, 2600 + r, DEV, dt) for r in range(k)]
    last = (n - 65536) // 256 * 256
    for base in (0, last):
        x[0][base + 17] = float("inf")
        x[1][base + 300] = float("nan")
        x[2][base + 301] = -65504.0
    x[3][n - 1] = float("nan")
    lay = gb.gb_bucket_workspace_layout(bf16, k, n, B)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=DEV)
    whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
    gb.gb_bucket_allreduce_local_typed(whole, x, B, bf16, 0, ws)
    step = 3 * (1 << 20)  # below 2^22
    wss = torch.empty(gb.gb_bucket_workspace_bytes(bf16, k, step, step), dtype=torch.uint8, device=DEV)
    for s, e in slices(n, step):
        gb.gb_bucket_allreduce_local_typed(ref[s:e], [t[s:e] for t in x], step, bf16, 0, wss)
    same(whole, ref, f"{dt} bf16-codec stream against slices below 2^22")
    codes = [ws[r * lay["codes_stride"]:][:2 * n].view(torch.int16) for r in range(k)]
    rng = np.random.default_rng(230)
    for s in [0, last] + [int(v) * 256 for v in rng.integers(0, last // 256, 3)]:
        e = n if s == last else s + 65536
        xs = [bits(t[s:e]).cpu().numpy().view(np.uint16) for t in x]
        want, wc, _ = O.bucket_allreduce_typed(xs, dt, B, O.CODEC_BF16)
        got = bits(whole[s:e]).cpu().numpy().view(np.uint16)
        assert (got == np.ascontiguousarray(want).view(np.uint16)).all(), f"oracle total window at {s}"
        for r in range(k):
            assert (codes[r][s:e].cpu().numpy().view(np.uint16) == wc[r]).all(), f"oracle codes {r}, window at {s}"


@pytest.mark.parametrize("acc", [False, True])
@pytest.mark.parametrize("n", [(1 << 24) + 256 * 3 + 77, (1 << 24) - 77])
def test_decode_fp8_wave_workgroups(gb, n, acc):
    """The fp8 decode of 4 payloads into a float32 total runs one 256-value
    block per 64-lane workgroup from 2^24 values, in 256-lane workgroups
    below.  On either side of the threshold, with a ragged last block and
    payloads of special values (NaN and Inf codes, a subnormal scale, zero
    blocks), with and without accumulation, it must equal the 256-lane
    kernel over slices below 2^24, and the oracle on the first, the last and
    sampled windows."""
    import numpy as np
    from oracle import oracle as O
    fp8, k = gb.GB_CODEC_FP8_E4M3_B256, 4
    x = [W.device_gradients(n, 2200 + r, DEV) for r in range(k)]
    last = (n - 65536) // 256 * 256
    plant_specials(x, n, last)
    nb = (n + 255) // 256
    codes = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(k)]
    scales = [torch.empty(nb, dtype=torch.float32, device=DEV) for _ in range(k)]
    for r in range(k):
        gb.gb_encode_fp8_e4m3_blockscaled(codes[r], scales[r], x[r], 0)
    start = W.device_gradients(n, 2300, DEV)
    whole = start.clone() if acc else filled(n)
    ref = start.clone() if acc else filled(n)
    gb.gb_decode_accumulate(whole, codes, scales, fp8, accumulate=acc)
    step = 3 * (1 << 22)  # below 2^24, a multiple of 256
    for s, e in slices(n, step):
        gb.gb_decode_accumulate(ref[s:e], [c[s:e] for c in codes], [t[s // 256:(e + 255) // 256] for t in scales],
                                fp8, accumulate=acc)
    same(whole, ref, f"decode of 4 payloads (accumulate={acc}) against 256-lane slices")
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    rng = np.random.default_rng(210)
    for s in [0, last] + [int(v) * 256 for v in rng.integers(0, last // 256, 3)]:
        e = n if s == last else s + 65536
        want = O.decode_accumulate([c[s:e].cpu().numpy() for c in codes],
                                   [t[s // 256:(e + 255) // 256].cpu().numpy() for t in scales], O.CODEC_FP8,
                                   start[s:e].cpu().numpy() if acc else None)
        assert (u32(whole[s:e].cpu().numpy()) == u32(want)).all(), f"oracle window at {s}"


@pytest.mark.parametrize("k", [3, 4, 6, 8])
@pytest.mark.parametrize("n", [(3 << 21) + 256 * 5 + 77, (1 << 21) + 3 * 64 + 5])
def test_fused_bf16_wave_workgroups(gb, k, n):
    """The fused bf16 bucket stream over float32 gradients from 3 ranks runs
    in 64-lane workgroups (256 values each) in index order, capped by rank
    count from 3 * 2^21 values and uncapped below.  With a ragged last
    workgroup it must equal the 256-lane batch kernel on the same buffers (a
    batch of one bucket), and the oracle on sampled windows (the first and
    last values included): totals and codes."""
    import numpy as np
    from oracle import oracle as O
    bf16 = gb.GB_CODEC_BF16
    x = [W.device_gradients(n, 1300 + 10 * k + r, DEV) for r in range(k)]
    lay = gb.gb_bucket_workspace_layout(bf16, k, n, B)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local(whole, x, B, bf16, 0, ws)
    wsb = torch.empty(gb.gb_bucket_batch_workspace_bytes(bf16, k, [n]), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch([ref], [x], bf16, workspace=wsb)
    same(whole, ref, f"fused bf16 pass over {k} ranks against the batch kernel")
    del ref, wsb
    codes = [ws[r * lay["codes_stride"]:][:2 * n].view(torch.int16) for r in range(k)]
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    length = 65536
    rng = np.random.default_rng(90 + k)
    last = n - length
    for s in [0, last] + [int(v) * 4 for v in rng.integers(0, last // 4, 4)]:
        e = n if s == last else s + length
        want, wc, _ = O.bucket_allreduce([t[s:e].cpu().numpy() for t in x], B, O.CODEC_BF16)
        assert (u32(whole[s:e].cpu().numpy()) == u32(want)).all(), f"oracle total window at {s}"
        for r in range(k):
            got = codes[r][s:e].cpu().numpy().view(np.uint16)
            assert (got == wc[r]).all(), f"oracle codes, rank {r}, window at {s}"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("k,n", [(k, (1 << 22) + 256 * 5 + 77) for k in (5, 6, 7, 8)]
                         + [(5, (1 << 22) - 3 * 64 - 5), (4, (1 << 29) + 256 * 5 + 77), (4, (1 << 29) - 3 * 64 - 5)])
def test_fused_bf16_half_wave_workgroups(gb, dt, k, n):
    """The fused bf16 bucket stream over float16 and bfloat16 gradients runs
    in 64-lane workgroups in index order, capped by rank count, over 5 to 8
    ranks from 2^22 values and over 4 from 2^29; in 256-lane workgroups
    below.  With a ragged last workgroup, on either side of each threshold,
    it must equal the 256-lane batch kernel on the same buffers (a batch of
    one bucket), and the oracle on sampled windows (the first and last values
    included): totals and codes."""
    import numpy as np
    from oracle import oracle as O
    bf16 = gb.GB_CODEC_BF16
    x = [W.device_gradients_typed(n, 1600 + 10 * k + r, DEV, dt) for r in range(k)]
    lay = gb.gb_bucket_workspace_layout(bf16, k, n, B)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
    gb.gb_bucket_allreduce_local_typed(whole, x, B, bf16, 0, ws)
    wsb = torch.empty(gb.gb_bucket_batch_workspace_bytes(bf16, k, [n]), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch([ref], [x], bf16, workspace=wsb)
    same(whole, ref, f"fused bf16 pass over {k} ranks of {dt} against the batch kernel")
    del ref, wsb
    codes = [ws[r * lay["codes_stride"]:][:2 * n].view(torch.int16) for r in range(k)]
    u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    length = 65536
    rng = np.random.default_rng(130 + k)
    last = n - length
    for s in [0, last] + [int(v) * 4 for v in rng.integers(0, last // 4, 3)]:
        e = n if s == last else s + length
        want, wc, _ = O.bucket_allreduce_typed([u16(t[s:e]) for t in x], dt, B, O.CODEC_BF16)
        assert (u16(whole[s:e]) == want).all(), f"oracle total window at {s}"
        for r in range(k):
            assert (u16(codes[r][s:e]) == wc[r]).all(), f"oracle codes, rank {r}, window at {s}"


@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("n", [(3 << 21) + 256 * 5 + 77, (1 << 20) + 3 * 64 + 5])
def test_fused_bf16_ef_wave_workgroups(gb, k, n):
    """The fused bf16 bucket stream with error feedback over float32
    gradients runs in 64-lane workgroups in index order at every size.  With
    a ragged last workgroup it must equal the 256-lane batch kernel from the
    same residuals (a batch of one bucket), and the oracle on sampled windows
    (the first and last values included): totals, codes and new residuals."""
    import numpy as np
    from oracle import oracle as O
    bf16 = gb.GB_CODEC_BF16
    x = [W.device_gradients(n, 1400 + 10 * k + r, DEV) for r in range(k)]
    r0 = [W.device_gradients(n, 1500 + 10 * k + r, DEV) * 1e-3 for r in range(k)]
    lay = gb.gb_bucket_workspace_layout(bf16, k, n, B)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    res = [t.clone() for t in r0]
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local_ef(whole, x, res, B, bf16, 0, ws)
    resb = [t.clone() for t in r0]
    wsb = torch.empty(gb.gb_bucket_batch_workspace_bytes(bf16, k, [n]), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch_ef([ref], [x], [resb], bf16, workspace=wsb)
    same(whole, ref, f"fused bf16 pass with feedback over {k} ranks against the batch kernel")
    for r in range(k):
        same(res[r], resb[r], f"residual {r} against the batch kernel")
    del ref, wsb, resb
    codes = [ws[r * lay["codes_stride"]:][:2 * n].view(torch.int16) for r in range(k)]
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    length = 65536
    rng = np.random.default_rng(110 + k)
    last = n - length
    for s in [0, last] + [int(v) * 4 for v in rng.integers(0, last // 4, 3)]:
        e = n if s == last else s + length
        want, wc, _, wr = O.bucket_allreduce_ef([t[s:e].cpu().numpy() for t in x],
                                                [t[s:e].cpu().numpy() for t in r0], B, O.CODEC_BF16)
        assert (u32(whole[s:e].cpu().numpy()) == u32(want)).all(), f"oracle total window at {s}"
        for r in range(k):
            assert (codes[r][s:e].cpu().numpy().view(np.uint16) == wc[r]).all(), f"oracle codes {r} at {s}"
            assert (u32(res[r][s:e].cpu().numpy()) == u32(wr[r])).all(), f"oracle residual {r} at {s}"


@pytest.mark.parametrize("dt,k,n", [
    ("bf16", 1, (1 << 22) + 256 * 5 + 77), ("bf16", 2, (1 << 22) + 256 * 5 + 77), ("bf16", 2, (1 << 22) - 3 * 64 - 5), ("bf16", 3, (1 << 22) + 256 * 5 + 77), ("bf16", 4, (1 << 20) + 3 * 64 + 5), ("bf16", 8, (1 << 20) + 3 * 64 + 5),
    ("f16", 2, (1 << 22) + 256 * 5 + 77), ("f16", 5, (1 << 20) + 3 * 64 + 5),
    ("f64", 1, (1 << 22) + 256 * 5 + 77), ("f64", 1, (1 << 22) - 3 * 64 - 5), ("f64", 2, (1 << 20) + 3 * 64 + 5), ("f64", 3, (1 << 22) + 256 * 5 + 77), ("f64", 4, (1 << 20) + 3 * 64 + 5), ("f64", 8, (1 << 20) + 3 * 64 + 5)])
def test_fused_bf16_ef_wave_typed_workgroups(gb, dt, k, n):
    """The fused bf16 bucket stream with error feedback runs in 64-lane
    workgroups in index order, capped by rank count: over float16 and
    bfloat16 gradients from 4 ranks at every size and over 2 or 3 from 2^22
    values (one rank keeps 256 lanes), over float64 gradients over 2 and 4 to
    8 ranks at every size and over 1 or 3 from 2^22 values (a float64 lane
    holds values 512 apart, so its workgroup is whole only with its vector
    group).  On either side of each threshold, with a ragged last vector
    group, it must equal the same step as separate 256-lane launches (each
    rank's error-feedback encode, then the decode-and-add) and the batch
    kernel (a batch of one bucket, which takes the same rule) from the same
    residuals, and the oracle on sampled windows (the first and last values
    included): totals, codes and new residuals."""
    import numpy as np
    from oracle import oracle as O
    bf16 = gb.GB_CODEC_BF16
    x = [W.device_gradients_typed(n, 1800 + 10 * k + r, DEV, dt) for r in range(k)]
    r0 = [W.device_gradients(n, 1900 + 10 * k + r, DEV) * 1e-3 for r in range(k)]
    lay = gb.gb_bucket_workspace_layout(bf16, k, n, B)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    res = [t.clone() for t in r0]
    whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
    gb.gb_bucket_allreduce_local_ef_typed(whole, x, res, B, bf16, 0, ws)
    codes = [ws[r * lay["codes_stride"]:][:2 * n].view(torch.int16) for r in range(k)]
    ress = [t.clone() for t in r0]
    codess = [torch.empty(n, dtype=torch.uint16, device=DEV) for _ in range(k)]
    for r in range(k):
        gb.gb_encode_ef(bf16, codess[r], None, ress[r], x[r])
    gb.gb_decode_sum(ref, codess, None, bf16)
    same(whole, ref, f"fused bf16 pass with feedback over {k} ranks of {dt} against the separate launches")
    for r in range(k):
        same(codes[r], codess[r].view(torch.int16), f"codes {r} against the separate encode")
        same(res[r], ress[r], f"residual {r} against the separate encode")
    del codess, ress
    ref.view(torch.uint8).fill_(0xFF)
    resb = [t.clone() for t in r0]
    wsb = torch.empty(gb.gb_bucket_batch_workspace_bytes(bf16, k, [n]), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_batch_ef([ref], [x], [resb], bf16, workspace=wsb)
    same(whole, ref, f"fused bf16 pass with feedback over {k} ranks of {dt} against the batch kernel")
    for r in range(k):
        same(res[r], resb[r], f"residual {r} against the batch kernel")
    del ref, wsb, resb
    host = lambda t: bits(t).cpu().numpy()
    u32 = lambda a: np.ascontiguousarray(a).view(np.uint32)
    length = 65536
    rng = np.random.default_rng(170 + k)
    last = (n - length) // 1024 * 1024
    for s in [0, last] + [int(v) * 1024 for v in rng.integers(0, last // 1024, 3)]:
        e = n if s == last else s + length
        xs = [host(t[s:e]).view(np.uint16) if dt != "f64" else t[s:e].cpu().numpy() for t in x]
        want, wc, _, wr = O.bucket_allreduce_ef_typed(xs, [t[s:e].cpu().numpy() for t in r0], dt, B, O.CODEC_BF16)
        assert (host(whole[s:e]) == np.ascontiguousarray(want).view(host(whole[:1]).dtype)).all(), \
            f"oracle total window at {s}"
        for r in range(k):
            assert (host(codes[r][s:e]).view(np.uint16) == wc[r]).all(), f"oracle codes {r} at {s}"
            assert (u32(res[r][s:e].cpu().numpy()) == u32(wr[r])).all(), f"oracle residual {r} at {s}"


@pytest.mark.parametrize("dt", ["bf16", "f16", "f64"])
def test_typed_reduce(gb, dt):
    n = N_VEC
    x = [W.device_gradients_typed(n, 950 + r, DEV, dt) for r in range(2)]
    whole = filled(n, x[0].dtype)
    ref = filled(n, x[0].dtype)
    gb.gb_reduce_typed(whole, x, gb.GB_OP_AVG, 2)
    step = STEP_RED * 4 // x[0].element_size() // 2  # below 8 runs of 4 KiB groups for the type
    for s, e in slices(n, step):
        gb.gb_reduce_typed(ref[s:e], [t[s:e] for t in x], gb.GB_OP_AVG, 2)
    same(whole, ref, f"typed AVG {dt}")


def test_fp8_group_kernels(gb):
    n = N_BLK
    k = 4
    x = [W.device_gradients(n, 970 + r, DEV) for r in range(k)]
    parts = slices(n, STEP_BLK)
    nb = (n + 255) // 256

    # encode, then decode-accumulate of two ranks' payloads
    codes = [filled(n, torch.uint8) for _ in range(2)]
    scales = [filled(nb) for _ in range(2)]
    cr, sr = filled(n, torch.uint8), filled(nb)
    for r in range(2):
        gb.gb_encode_fp8_e4m3_blockscaled(codes[r], scales[r], x[r], 0)
    for s, e in parts:
        gb.gb_encode_fp8_e4m3_blockscaled(cr[s:e], sr[s // 256:(e + 255) // 256], x[0][s:e], 0)
    same(codes[0], cr, "encode fp8 codes")
    same(scales[0], sr, "encode fp8 scales")
    del cr, sr
    whole, ref = filled(n), filled(n)
    gb.gb_decode_accumulate(whole, codes, scales, gb.GB_CODEC_FP8_E4M3_B256)
    for s, e in parts:
        gb.gb_decode_accumulate(ref[s:e], [c[s:e] for c in codes], [t[s // 256:(e + 255) // 256] for t in scales],
                                gb.GB_CODEC_FP8_E4M3_B256)
    same(whole, ref, "decode fp8")

    # island sum with its fp8 payload, the sum written over the first source
    x0 = x[0].clone()
    cw, sw = codes[0], scales[0]
    cr, sr = filled(n, torch.uint8), filled(nb)
    cw.fill_(0xFF)
    sw.view(torch.int32).fill_(SENTINEL)
    srcs = [x0] + x[1:2]
    ref = filled(n)
    for s, e in parts:
        gb.gb_reduce_encode(gb.GB_CODEC_FP8_E4M3_B256, cr[s:e], sr[s // 256:(e + 255) // 256],
                            [t[s:e] for t in srcs], sum=ref[s:e], scale_mode=1)
    gb.gb_reduce_encode(gb.GB_CODEC_FP8_E4M3_B256, cw, sw, srcs, sum=x0, scale_mode=1)
    same(x0, ref, "reduce_encode fp8 sum in place")
    same(cw, cr, "reduce_encode fp8 codes")
    same(sw, sr, "reduce_encode fp8 scales")
    del x0, cr, sr, codes, scales, cw, sw, ref

    # the fp8 bucket stream over 4 ranks, and with error feedback over 2
    ws = torch.empty(gb.gb_bucket_workspace_bytes(gb.GB_CODEC_FP8_E4M3_B256, k, n, B), dtype=torch.uint8,
                     device=DEV)
    whole, ref = filled(n), filled(n)
    gb.gb_bucket_allreduce_local(whole, x, B, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    for s, e in slices(n, STEP_HALF):  # one block per wavefront here and in the whole launch
        gb.gb_bucket_allreduce_local(ref[s:e], [t[s:e] for t in x], B, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    same(whole, ref, "fp8 bucket stream")
    rw = [torch.full((n,), -2e-5, device=DEV) for _ in range(2)]
    rr = [t.clone() for t in rw]
    whole.view(torch.int32).fill_(SENTINEL)
    ref.view(torch.int32).fill_(SENTINEL)
    gb.gb_bucket_allreduce_local_ef(whole, x[:2], rw, B, gb.GB_CODEC_FP8_E4M3_B256, 1, ws)
    for s, e in parts:
        gb.gb_bucket_allreduce_local_ef(ref[s:e], [t[s:e] for t in x[:2]], [t[s:e] for t in rr], B,
                                        gb.GB_CODEC_FP8_E4M3_B256, 1, ws)
    same(whole, ref, "fp8 bucket stream with error feedback")
    for r in range(2):
        same(rw[r], rr[r], f"fp8 residual {r}")


@pytest.mark.parametrize("dt,codec,n,step", [("bf16", 2, N_BLK, STEP_BLK), ("f64", 1, N_VEC, STEP_VEC)])
def test_typed_error_feedback(gb, dt, codec, n, step):
    """Error feedback over bfloat16 gradients with the fp8 codec, and over
    float64 gradients (their own lane map) with the bf16 codec, above the
    thresholds."""
    x = [W.device_gradients_typed(n, 990 + r, DEV, dt) for r in range(2)]
    rw = [torch.full((n,), 1.5e-5, device=DEV) for _ in range(2)]
    rr = [t.clone() for t in rw]
    whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
    ws = torch.empty(gb.gb_bucket_workspace_bytes(codec, 2, n, B), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_ef_typed(whole, x, rw, B, codec, 0, ws)
    for s, e in slices(n, step):
        gb.gb_bucket_allreduce_local_ef_typed(ref[s:e], [t[s:e] for t in x], [t[s:e] for t in rr], B, codec, 0, ws)
    same(whole, ref, f"{dt} error-feedback stream")
    for r in range(2):
        same(rw[r], rr[r], f"{dt} residual {r}")
