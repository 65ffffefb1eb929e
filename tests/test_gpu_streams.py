"""The library's calls on several streams, from several host threads and
inside replayed HIP graphs: results equal the oracle's in every case.

Every call enqueues on the stream it is given (torch's current stream by
default), so independent calls on two streams may overlap on the GPU; the
staged calls share one per-device set of copy streams, which a lock keeps
whole per call."""
import threading

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


def test_two_streams_overlap(gb):
    """A bucket stream on one stream and a bf16 encode plus sum on another,
    issued interleaved without synchronisation in between."""
    k, n, bucket = 4, 4096 * 40 + 17, 4096 * 8
    xs = W.gradient_ranks(k, n, 6000)
    ys = W.normal_ranks(2, n, 6100)
    dx = [torch.from_numpy(x).to(DEV) for x in xs]
    dy = [torch.from_numpy(y).to(DEV) for y in ys]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    out1 = torch.empty(n, device=DEV)
    ws = torch.empty(gb.gb_bucket_workspace_bytes(2, k, n, bucket), dtype=torch.uint8, device=DEV)
    out2 = torch.empty(n, device=DEV)
    codes = torch.empty(n, dtype=torch.uint16, device=DEV)
    for rep in range(5):
        gb.gb_bucket_allreduce_local(out1, dx, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, ws, stream=s1)
        gb.gb_reduce_sum(out2, dy, stream=s2)
        gb.gb_encode_bf16(codes, out2, stream=s2)
    torch.cuda.synchronize()
    want1, _, _ = O.bucket_allreduce(xs, bucket, O.CODEC_FP8)
    want2 = O.reduce_sum(ys)
    assert (u32(out1.cpu().numpy()) == u32(want1)).all()
    assert (u32(out2.cpu().numpy()) == u32(want2)).all()
    assert (codes.view(torch.int16).cpu().numpy().view(np.uint16) == O.encode_bf16(want2)).all()


def test_staged_calls_from_two_threads(gb):
    """Two host threads run staged encodes of different buffers on their own
    streams at the same time; each one's host payload is its own."""
    n, chunk = 3 * 65536 + 9, 65536
    xs = [W.gradients(n, 6200 + t) for t in range(2)]
    nb = O.nblocks(n)
    bufs = []
    for t in range(2):
        bufs.append(dict(x=torch.from_numpy(xs[t]).to(DEV), cd=torch.empty(n, dtype=torch.uint8, device=DEV),
                         sd=torch.empty(nb, device=DEV), ch=torch.empty(n, dtype=torch.uint8, pin_memory=True),
                         sh=torch.empty(nb, dtype=torch.float32, pin_memory=True), stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []

    def work(b):
        try:
            for _ in range(10):
                gb.gb_encode_staged(gb.GB_CODEC_FP8_E4M3_B256, b["cd"], b["sd"], b["ch"], b["sh"], b["x"], chunk,
                                    0, stream=b["stream"])
            b["stream"].synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)
    threads = [threading.Thread(target=work, args=(b,)) for b in bufs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(2):
        wc, ws = O.encode_fp8(xs[t], 0)
        assert (bufs[t]["ch"].numpy() == wc).all(), t
        assert (u32(bufs[t]["sh"].numpy()) == u32(ws)).all(), t


def test_typed_calls_in_a_replayed_graph(gb):
    """bfloat16 bucket stream and float16 AVG captured once, replayed with
    eager work and new inputs between replays: every replay is right."""
    k, n, bucket = 4, 4096 * 6 + 256 * 3, 4096
    xb = W.typed_ranks(k, n, "bf16", 6300)
    xh = W.typed_ranks(3, n, "f16", 6400)
    db = [torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16) for x in xb]
    dh = [torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.float16) for x in xh]
    ob = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    oh = torch.empty(n, dtype=torch.float16, device=DEV)
    ws = torch.empty(gb.gb_bucket_workspace_bytes(2, k, n, bucket), dtype=torch.uint8, device=DEV)

    def step():
        gb.gb_bucket_allreduce_local_typed(ob, db, bucket, gb.GB_CODEC_FP8_E4M3_B256, 0, ws)
        gb.gb_reduce_typed(oh, dh, gb.GB_OP_AVG, 3)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        # new inputs, written in place, before each replay
        xb = W.typed_ranks(k, n, "bf16", 6500 + rep)
        xh = W.typed_ranks(3, n, "f16", 6600 + rep)
        for t, x in zip(db, xb):
            t.view(torch.int16).copy_(torch.from_numpy(x.view(np.int16)))
        for t, x in zip(dh, xh):
            t.view(torch.int16).copy_(torch.from_numpy(x.view(np.int16)))
        ob.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want, _, _ = O.bucket_allreduce_typed(xb, "bf16", bucket, O.CODEC_FP8)
        assert (ob.view(torch.int16).cpu().numpy().view(np.uint16) == want).all(), rep
        wh = O.reduce_typed(xh, "f16", O.OP_AVG, 3)
        gh = oh.view(torch.int16).cpu().numpy().view(np.uint16)
        nan = np.isnan(wh.view(np.float16))
        assert (np.isnan(gh.view(np.float16)) == nan).all() and (gh[~nan] == wh[~nan]).all(), rep
        gb.gb_reduce_sum(torch.empty(16, device=DEV), [torch.ones(16, device=DEV)])  # eager work between
        torch.cuda.synchronize()


@pytest.mark.parametrize("codec,k", [(O.CODEC_FP8, 3), (O.CODEC_BF16, 4)])
def test_error_feedback_in_a_replayed_graph(gb, codec, k):
    """One error-feedback bucket stream captured once and replayed three times:
    each replay reads the residuals the previous one wrote, exactly as three
    eager calls do, for float32, bfloat16 and float64 gradients; with the
    bf16 codec over 4 ranks every type runs the 64-lane kernel."""
    n, bucket = 4096 * 5 + 256 * 3 + 17, 4096
    for dt in ("f32", "bf16", "f64"):
        xs = W.typed_ranks(k, n, dt, 6700) if dt != "f32" else W.gradient_ranks(k, n, 6700)
        dx = ([torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16) for x in xs] if dt == "bf16"
              else [torch.from_numpy(x).to(DEV) for x in xs])
        res = [torch.zeros(n, device=DEV) for _ in range(k)]
        out = torch.empty(n, dtype=dx[0].dtype, device=DEV)
        ws = torch.empty(gb.gb_bucket_workspace_bytes(codec, k, n, bucket), dtype=torch.uint8, device=DEV)
        step = lambda: gb.gb_bucket_allreduce_local_ef_typed(out, dx, res, bucket, codec, 0, ws)
        # warm up on scratch residuals, then capture
        saved = [r.clone() for r in res]
        step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for r, s in zip(res, saved):
            r.copy_(s)
        torch.cuda.synchronize()
        wres = [np.zeros(n, np.float32) for _ in range(k)]
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            want, _, _, wres = O.bucket_allreduce_ef_typed(xs, wres, dt, bucket, codec)
            got = out.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else out.cpu().numpy()
            assert got.tobytes() == np.ascontiguousarray(want).tobytes(), (dt, rep)
            for r in range(k):
                assert (u32(res[r].cpu().numpy()) == u32(wres[r])).all(), (dt, rep, r)
            gb.gb_reduce_sum(torch.empty(16, device=DEV), [torch.ones(16, device=DEV)])  # eager work between
            torch.cuda.synchronize()


def test_one_block_per_wavefront_kernels_in_a_replayed_graph(gb):
    """The 4-rank kernels that take one fp8 block per 64-lane workgroup, each
    captured once and replayed three times with eager work in between: the
    fused pass over float32 gradients, the pass with error feedback over
    float32 and bfloat16 gradients (each replay reads the residuals the
    previous one wrote, as eager calls do) and the decode of 4 payloads.
    Every replay must equal the same calls made eagerly, bit for bit."""
    k, fp8 = 4, gb.GB_CODEC_FP8_E4M3_B256
    n, bucket = (1 << 22) + 256 * 3 + 17, W.DDP_BUCKET
    between = lambda: gb.gb_reduce_sum(torch.empty(16, device=DEV), [torch.ones(16, device=DEV)])

    def replays_match(step, outs, reset, eager_steps):
        """Capture step, reset the state, then compare three replays with
        the eager results of the same three steps."""
        step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        reset()
        torch.cuda.synchronize()
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            for got, want in zip(outs(), eager_steps[rep]):
                assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), rep
            between()
            torch.cuda.synchronize()

    x = [W.device_gradients(n, 7000 + r, DEV) for r in range(k)]
    ws = torch.empty(gb.gb_bucket_workspace_bytes(fp8, k, n, bucket), dtype=torch.uint8, device=DEV)
    out = torch.empty(n, device=DEV)
    gb.gb_bucket_allreduce_local(out, x, bucket, fp8, 0, ws)
    torch.cuda.synchronize()
    want = [(out.clone(), ws.clone())]
    replays_match(lambda: gb.gb_bucket_allreduce_local(out, x, bucket, fp8, 0, ws), lambda: (out, ws),
                  lambda: None, want * 3)

    for dt in ("f32", "bf16"):
        xs = x if dt == "f32" else [W.device_gradients_typed(n, 7100 + r, DEV, dt) for r in range(k)]
        r0 = [W.device_gradients(n, 7200 + r, DEV) * 1e-2 for r in range(k)]
        res = [t.clone() for t in r0]
        o = torch.empty(n, dtype=xs[0].dtype, device=DEV)
        step = lambda: gb.gb_bucket_allreduce_local_ef_typed(o, xs, res, bucket, fp8, 0, ws)
        eager = []
        for _ in range(3):
            step()
            torch.cuda.synchronize()
            eager.append([o.clone(), ws.clone()] + [t.clone() for t in res])
        for t, s in zip(res, r0):
            t.copy_(s)

        def reset():
            for t, s in zip(res, r0):
                t.copy_(s)
        replays_match(step, lambda: [o, ws] + res, reset, eager)

    m = (1 << 24) + 77
    codes = [torch.empty(m, dtype=torch.uint8, device=DEV) for _ in range(k)]
    scales = [torch.empty((m + 255) // 256, device=DEV) for _ in range(k)]
    for r in range(k):
        gb.gb_encode_fp8_e4m3_blockscaled(codes[r], scales[r], W.device_gradients(m, 7300 + r, DEV), 0)
    acc = torch.empty(m, device=DEV)
    gb.gb_decode_accumulate(acc, codes, scales, fp8)
    torch.cuda.synchronize()
    replays_match(lambda: gb.gb_decode_accumulate(acc, codes, scales, fp8), lambda: (acc,), lambda: acc.zero_(),
                  [(acc.clone(),)] * 3)
