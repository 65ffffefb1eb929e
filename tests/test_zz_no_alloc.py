"""gb_bucket_allreduce_local_noalloc through the C ABI: the bucket stream with
its payloads in the library's static device scratch gives the same output as
gb_bucket_allreduce_local with a workspace, bit for bit, on consecutive calls
whose sizes shrink (the scratch keeps the previous call's bytes), for both
codecs, both scale rules, more than 8 ranks (whose payloads the pass reads
back from the scratch) and in place, and captured in a HIP graph and
replayed; sizes beyond the scratch are refused with nothing written."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W  # noqa: E402

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def ranks(k, n, seed):
    return [torch.from_numpy(x).to(DEV) for x in W.gradient_ranks(k, n, seed)]


def with_workspace(gb, xs, bucket, codec, mode):
    n = xs[0].numel()
    out = torch.full((n,), float("nan"), device=DEV)
    ws = torch.empty(max(1, gb.gb_bucket_workspace_bytes(codec, len(xs), n, bucket)), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local(out, xs, bucket, codec, mode, ws)
    return out


def no_alloc(gb, xs, bucket, codec, mode):
    n = xs[0].numel()
    out = torch.full((n,), float("nan"), device=DEV)
    gb.gb_bucket_allreduce_local_noalloc(out, xs, bucket, codec, mode)
    return out


def bits(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("codec,mode", [(2, 0), (2, 1), (1, 0), (0, 0)])
@pytest.mark.parametrize("k", [1, 4, 11])
def test_two_calls_in_a_row_the_second_smaller(gb, codec, mode, k):
    bucket = 256 * 40
    # the larger call first: its payload bytes stay in the scratch for the second
    for n, seed in ((bucket * 5 + 4099, 11 + k), (bucket * 2 + 77, 23 + k)):
        xs = ranks(k, n, seed)
        want = bits(with_workspace(gb, xs, bucket, codec, mode))
        got = bits(no_alloc(gb, xs, bucket, codec, mode))
        assert (got == want).all(), f"k={k} n={n} codec={codec} mode={mode}"


def test_a_whole_ddp_bucket_at_the_scratch_limit(gb):
    """A 25 MiB bucket of 4 ranks (the DDP hook's call), then a short one."""
    for n in (6_553_600, 300_001):
        xs = ranks(4, n, 31)
        want = bits(with_workspace(gb, xs, 6_553_600, 2, 0))
        got = bits(no_alloc(gb, xs, 6_553_600, 2, 0))
        assert (got == want).all(), n


def test_in_place(gb):
    n, bucket = 256 * 33 + 5, 256 * 8
    host = W.gradient_ranks(3, n, 41)
    a = [torch.from_numpy(x).to(DEV) for x in host]
    b = [torch.from_numpy(x).to(DEV) for x in host]
    ws = torch.empty(gb.gb_bucket_workspace_bytes(2, 3, n, bucket), dtype=torch.uint8, device=DEV)
    gb.gb_bucket_allreduce_local(a[0], a, bucket, 2, 0, ws)
    gb.gb_bucket_allreduce_local_noalloc(b[0], b, bucket, 2, 0)
    assert (bits(a[0]) == bits(b[0])).all()


@pytest.mark.parametrize("codec,k", [(2, 4), (1, 4), (2, 11)])
def test_captured_in_a_graph_and_replayed(gb, codec, k):
    """The call captured once in a HIP graph (no allocation, no memset node)
    and replayed four times, new inputs copied in eagerly before each replay:
    every replay equals the eager workspace call on those inputs."""
    bucket = 256 * 40
    n = bucket * 3 + 1001
    xs = ranks(k, n, 101 + k)
    out = torch.full((n,), float("nan"), device=DEV)
    gb.gb_bucket_allreduce_local_noalloc(out, xs, bucket, codec, 0)  # the scratch's address looked up eagerly
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gb.gb_bucket_allreduce_local_noalloc(out, xs, bucket, codec, 0)
    for rep in range(4):
        for x, fresh in zip(xs, ranks(k, n, 200 + 10 * rep + k)):
            x.copy_(fresh)
        want = bits(with_workspace(gb, xs, bucket, codec, 0))
        out.fill_(float("nan"))
        graph.replay()
        assert (bits(out) == want).all(), f"replay {rep}"
    del graph


def test_sizes_beyond_the_scratch_are_refused(gb):
    k, bucket = 4, 256
    n = gb.GB_NOALLOC_SCRATCH_BYTES // 4  # 4 ranks of n codes and n / 64 scale bytes: just over the scratch
    assert gb.gb_bucket_workspace_bytes(2, k, n, bucket) > gb.GB_NOALLOC_SCRATCH_BYTES
    xs = [torch.zeros(n, device=DEV) for _ in range(k)]
    out = torch.full((n,), 7.0, device=DEV)
    with pytest.raises(gb.GbError) as e:
        gb.gb_bucket_allreduce_local_noalloc(out, xs, bucket, 2, 0)
    assert e.value.status == gb.GB_ERR_WORKSPACE
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (out == 7.0).all(), "a refused call wrote its output"
    # the uncompressed stream needs no scratch at any size
    gb.gb_bucket_allreduce_local_noalloc(out, xs, bucket, 0, 0)
    torch.cuda.synchronize()
    assert (out == 0.0).all()
