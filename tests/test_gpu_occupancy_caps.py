"""Bucket streams over four ranks on both sides of the sizes where a kernel's
occupancy cap changes (the LDS a launch reserves, which no kernel reads):
the fused bf16 pass from 2^25 values per rank (float32 and float64
gradients), the fused fp8 pass over half-precision gradients from 2^26 and
the fused fp8 pass with error feedback from 2^28.  A call above the size
gives, bit for bit, what the same call gives over bucket-aligned slices
below it; those smaller calls are checked against the oracle by the other
GPU tests.  Outputs start filled with a sentinel, and every size ends in a
ragged tail."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W  # noqa: E402

DEV = "cuda:0"
B = W.DDP_BUCKET  # 6,553,600 values
K = 4


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def slices(n, step):
    return [(s, min(s + step, n)) for s in range(0, n, step)]


def filled(n, dtype):
    t = torch.empty(n, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xFF)  # a NaN in every floating type
    return t


def bits(t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()])


def same(a, b, what):
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b)), what


def gradients(n, dt, seed):
    return [W.device_gradients_typed(n, seed + r, DEV, dt) for r in range(K)]


@pytest.mark.parametrize("dt,codec,n,step", [
    ("f32", 1, (1 << 25) + 4096 * 3 + 77, 5 * B),    # fused bf16: 3 per CU from 2^25
    ("f64", 1, (1 << 25) + 4096 * 3 + 77, 5 * B),    # fused bf16: 2 per CU from 2^25
    ("f16", 2, (1 << 26) + 4096 * 5 + 301, 10 * B),  # fused fp8 over halves: 2 per CU from 2^26
    ("bf16", 2, (1 << 26) + 4096 * 5 + 301, 10 * B),
])
def test_bucket_stream(gb, dt, codec, n, step):
    assert step < n and all(e - s < (1 << 25 if codec == 1 else 1 << 26) for s, e in slices(n, step))
    x = gradients(n, dt, 1100)
    ws = torch.empty(gb.gb_bucket_workspace_bytes(codec, K, n, B), dtype=torch.uint8, device=DEV)
    whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
    gb.gb_bucket_allreduce_local_typed(whole, x, B, codec, 0, ws)
    for s, e in slices(n, step):
        gb.gb_bucket_allreduce_local_typed(ref[s:e], [t[s:e] for t in x], B, codec, 0, ws)
    same(whole, ref, f"{dt} codec={codec} n={n}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fp8_error_feedback(gb, dt):
    """The fused fp8 error-feedback pass: one workgroup per CU from 2^28 values
    per rank, uncapped below; residuals carried over two steps."""
    n, step = (1 << 28) + 4096 * 2 + 13, 40 * B
    assert all(e - s < (1 << 28) for s, e in slices(n, step))
    ws = torch.empty(gb.gb_bucket_workspace_bytes(2, K, n, B), dtype=torch.uint8, device=DEV)
    rw = [torch.full((n,), 2.5e-5, device=DEV) for _ in range(K)]
    rr = [t.clone() for t in rw]
    for it in range(2):
        x = gradients(n, dt, 1200 + 10 * it)
        whole, ref = filled(n, x[0].dtype), filled(n, x[0].dtype)
        gb.gb_bucket_allreduce_local_ef_typed(whole, x, rw, B, 2, 0, ws)
        for s, e in slices(n, step):
            gb.gb_bucket_allreduce_local_ef_typed(ref[s:e], [t[s:e] for t in x], [t[s:e] for t in rr], B, 2, 0, ws)
        same(whole, ref, f"{dt} step {it}")
        for r in range(K):
            same(rw[r], rr[r], f"{dt} residual {r} step {it}")
        del x, whole, ref
