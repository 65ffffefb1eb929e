"""GPU parity at the workloads' full sizes, through the same calls and launch
configuration bench.py times, checked against the CPU oracle: the 1e9-value
fp8 bucket stream on every value (bucket by bucket on the host's cores), the
other workloads on their whole outputs here or through the golden hashes of
tests/golden, and the typed streams on sampled outputs.

Sampling is by whole 256-value blocks: a block is the unit of every
computation here (an fp8 scale covers one block; every other step is
elementwise), so the oracle run on the concatenation of sampled blocks gives
exactly those blocks' results.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def u32(a):
    return np.ascontiguousarray(a).view(np.uint32)


def gather_blocks(t, blocks):
    """Values of the given 256-value blocks of a device tensor, on the host."""
    idx = (torch.as_tensor(blocks, device=t.device, dtype=torch.int64)[:, None] * 256
           + torch.arange(256, device=t.device)[None, :]).reshape(-1)
    return t[idx].cpu().numpy()


def sample_blocks(nblocks, count, seed, must=()):
    rng = np.random.default_rng(seed)
    b = set(int(x) for x in rng.choice(nblocks, min(count, nblocks), replace=False))
    b.update(int(m) for m in must if 0 <= m < nblocks)
    return np.array(sorted(b), dtype=np.int64)


def test_two_rank_4mib_whole(gb):
    xs = W.normal_ranks(2, W.TWO_RANK_N)
    d = [torch.from_numpy(x).to(DEV) for x in xs]
    s = torch.empty(W.TWO_RANK_N, device=DEV)
    c = torch.empty(W.TWO_RANK_N, dtype=torch.uint16, device=DEV)
    dec = torch.empty(W.TWO_RANK_N, device=DEV)
    gb.gb_reduce_sum(s, d)
    gb.gb_encode_bf16(c, s)
    gb.gb_decode_accumulate(dec, [c], None, gb.GB_CODEC_BF16)
    ws = O.reduce_sum(xs)
    wc = O.encode_bf16(ws)
    wd = O.decode_accumulate([wc], None, O.CODEC_BF16)
    assert (u32(s.cpu().numpy()) == u32(ws)).all()
    assert (c.view(torch.int16).cpu().numpy().view(np.uint16) == wc).all()
    assert (u32(dec.cpu().numpy()) == u32(wd)).all()


def test_two_island_sweep_every_size_whole(gb):
    for n in W.SWEEP_SIZES:
        xs = W.normal_ranks(2, n)
        d = [torch.from_numpy(x).to(DEV) for x in xs]
        out = torch.empty(n, device=DEV)
        gb.gb_reduce_sum(out, d)
        assert (u32(out.cpu().numpy()) == u32(O.reduce_sum(xs))).all(), n


def test_gradients_64mib_bf16_sampled(gb):
    k, n = 4, W.GRAD64_N
    xs = W.gradient_ranks(k, n)
    d = [torch.from_numpy(x).to(DEV) for x in xs]
    codes = [torch.empty(n, dtype=torch.uint16, device=DEV) for _ in range(k)]
    out = torch.empty(n, device=DEV)
    for r in range(k):
        gb.gb_encode_bf16(codes[r], d[r])
    gb.gb_decode_accumulate(out, codes, None, gb.GB_CODEC_BF16)
    torch.cuda.synchronize()
    blocks = sample_blocks(n // 256, 4000, 1, must=(0, n // 256 - 1))
    sx = [x.reshape(-1, 256)[blocks].reshape(-1) for x in xs]
    wc = [O.encode_bf16(x) for x in sx]
    wo = O.decode_accumulate(wc, None, O.CODEC_BF16)
    for r in range(k):
        got = gather_blocks(codes[r].view(torch.int16), blocks).view(np.uint16)
        assert (got == wc[r]).all(), r
    assert (u32(gather_blocks(out, blocks)) == u32(wo)).all()


@pytest.mark.parametrize("mode", [0, 1])
def test_gradients_256mib_fp8_sampled(gb, mode):
    k, n = 4, W.GRAD256_N
    xs = W.gradient_ranks(k, n)
    d = [torch.from_numpy(x).to(DEV) for x in xs]
    nb = n // 256
    codes = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(k)]
    scales = [torch.empty(nb, device=DEV) for _ in range(k)]
    out = torch.empty(n, device=DEV)
    for r in range(k):
        gb.gb_encode_fp8_e4m3_blockscaled(codes[r], scales[r], d[r], mode)
    gb.gb_decode_accumulate(out, codes, scales, gb.GB_CODEC_FP8_E4M3_B256)
    torch.cuda.synchronize()
    blocks = sample_blocks(nb, 4000, 2, must=(0, nb - 1))
    enc = [O.encode_fp8(x.reshape(-1, 256)[blocks].reshape(-1), mode) for x in xs]
    wo = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8)
    bt = torch.as_tensor(blocks, device=DEV)
    for r in range(k):
        assert (gather_blocks(codes[r], blocks) == enc[r][0]).all(), r
        assert (u32(scales[r][bt].cpu().numpy()) == u32(enc[r][1])).all(), r
    assert (u32(gather_blocks(out, blocks)) == u32(wo)).all()


def test_ddp_1b_buckets_fp8_every_value(gb):
    """The benchmark's default workload: 4 x 1e9 values, 153 buckets of
    25 MiB, one gb_bucket_allreduce_local call in the launch configuration
    the benchmark times, then every output value, every code and every
    scale of every bucket against the oracle (gpubridge README, "Bridge
    compression": the compression kernels match the CPU reference bit for
    bit).  The oracle runs bucket by bucket on a pool of the host's cores
    (ctypes releases the GIL), each bucket's inputs and results copied to the
    host and dropped once compared; finite inputs must also give no NaN
    code, positive finite scales and finite outputs."""
    import concurrent.futures as cf
    import os
    k, n, bucket = 4, W.DDP_N, W.DDP_BUCKET
    x = [W.device_gradients(n, W.BASE_SEED + r, DEV) for r in range(k)]
    out = torch.empty(n, device=DEV)
    lay = gb.gb_bucket_workspace_layout(gb.GB_CODEC_FP8_E4M3_B256, k, n, bucket)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local(out, x, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    torch.cuda.synchronize()
    nb = n // 256
    codes = [ws[r * lay["codes_stride"]:r * lay["codes_stride"] + n] for r in range(k)]
    scales = [ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32) for r in range(k)]
    buckets = W.ddp_buckets()
    assert len(buckets) == 153

    def check(b):
        s, length = buckets[b]
        xs = [t[s:s + length].cpu().numpy() for t in x]
        want, wc, wsc = O.bucket_allreduce(xs, bucket, O.CODEC_FP8, O.SCALE_ABSMAX_DIV_448)
        bad = [int((u32(out[s:s + length].cpu().numpy()) != u32(want)).sum())]
        for r in range(k):
            c = codes[r][s:s + length].cpu().numpy()
            sc = scales[r][s // 256:(s + length) // 256].cpu().numpy()
            bad += [int((c != wc[r]).sum()), int((u32(sc) != u32(wsc[r])).sum()),
                    int(((c & 0x7F) == 0x7F).sum()), int((~np.isfinite(sc) | (sc <= 0)).sum())]
        bad.append(int((~np.isfinite(want)).sum()))
        return b, bad

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(check, range(len(buckets))))
    failed = [(b, bad) for b, bad in results if any(bad)]
    assert not failed, f"{len(failed)} of {len(buckets)} buckets differ, first: {failed[:3]}"


def raw(t):
    """A device tensor's bits as an integer view (16-bit floats as their codes)."""
    return t.view({2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]) if t.is_floating_point() else t


@pytest.mark.parametrize("dt", ["bf16", "f16", "f64"])
def test_ddp_1b_buckets_fp8_typed_sampled(gb, dt):
    """The benchmark's --dtype runs: 4 x 1e9 gradients of the type (float64
    at 5e8, as large in bytes), the same buckets and one
    gb_bucket_allreduce_local_typed call, checked against the oracle on
    random blocks and on the first and last block of every bucket: the total
    rounded to the type, every code and every scale."""
    k, bucket = 4, W.DDP_BUCKET
    n = W.DDP_N if dt != "f64" else W.DDP_N // 2
    x = [W.device_gradients_typed(n, W.BASE_SEED + r, DEV, dt) for r in range(k)]
    out = torch.empty(n, dtype=x[0].dtype, device=DEV)
    lay = gb.gb_bucket_workspace_layout(gb.GB_CODEC_FP8_E4M3_B256, k, n, bucket)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local_typed(out, x, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    torch.cuda.synchronize()
    nb = n // 256
    edges = [e for s, l in W.ddp_buckets(n, bucket) for e in (s // 256, (s + l) // 256 - 1)]
    blocks = sample_blocks(nb, 2000, 4, must=edges)
    # the gathered bits, reinterpreted as the oracle's arrays of the type
    as_type = (lambda a: a.view(np.uint16)) if dt in ("bf16", "f16") else (lambda a: a.view(np.float64))
    xs = [as_type(gather_blocks(raw(t), blocks)) for t in x]
    want, codes, scales = O.bucket_allreduce_typed(xs, dt, 256, O.CODEC_FP8, O.SCALE_ABSMAX_DIV_448)
    got = gather_blocks(raw(out), blocks)
    bad = int((got != np.ascontiguousarray(want).view(got.dtype)).sum())
    assert bad == 0, f"{bad} of {got.size} sampled values differ from the oracle"

    bt = torch.as_tensor(blocks, device=DEV)
    for r in range(k):
        c = ws[r * lay["codes_stride"]:r * lay["codes_stride"] + n]
        s = ws[lay["scales_offset"] + r * lay["scales_stride"]:][:4 * nb].view(torch.float32)
        assert int((gather_blocks(c, blocks) != codes[r]).sum()) == 0, f"codes of rank {r}"
        assert int((u32(s[bt].cpu().numpy()) != u32(scales[r])).sum()) == 0, f"scales of rank {r}"


def test_ddp_per_bucket_calls_in_a_replayed_graph(gb):
    """One call per bucket (as a DDP hook issues them), captured in a HIP graph
    and replayed several times with eager work in between: every replay gives
    the single-call result."""
    k, bucket, nbuckets = 4, W.DDP_BUCKET, 6
    n = bucket * nbuckets - 256 * 7  # last bucket partial
    x = [W.device_gradients(n, 100 + r, DEV) for r in range(k)]
    whole = torch.empty(n, device=DEV)
    lay = gb.gb_bucket_workspace_layout(gb.GB_CODEC_FP8_E4M3_B256, k, n, bucket)
    ws = torch.empty(lay["total"] + 4096 * nbuckets, dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local(whole, x, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
    torch.cuda.synchronize()
    want = whole.clone()
    out = torch.empty(n, device=DEV)
    calls, off = [], 0
    for start in range(0, n, bucket):
        length = min(bucket, n - start)
        need = gb.gb_bucket_workspace_bytes(gb.GB_CODEC_FP8_E4M3_B256, k, length, bucket)
        calls.append((out[start:start + length], [t[start:start + length] for t in x], ws[off:off + need]))
        off += need

    def step():
        for o, xs, w in calls:
            gb.gb_bucket_allreduce_local(o, xs, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, w)

    step()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), want.view(torch.int32))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(float(rep))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), rep
        gb.gb_reduce_sum(whole, [x[0]])  # eager work between replays
        torch.cuda.synchronize()
