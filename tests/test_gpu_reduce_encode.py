"""GPU parity of gb_reduce_encode (the island sum and its bridge payload in
one pass) against the oracle's sum followed by its encoder, bit for bit:
every rank count up to 16, both codecs and scale modes, ragged sizes, with and
without the stored sum, in place on the first source."""
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


def inputs(k, n, seed):
    xs = W.gradient_ranks(k, n, seed)
    rng = np.random.default_rng(seed)
    pool = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-42, -3e38], np.float32)
    for x in xs:
        m = max(1, n // 500)
        x[rng.choice(n, m, replace=False)] = pool[rng.integers(0, pool.size, m)]
    return xs


def run(gb, xs, codec, mode, store_sum, in_place=False):
    n = xs[0].size
    d = [torch.from_numpy(x).to(DEV) for x in xs]
    codes = torch.empty(n, dtype=torch.uint16 if codec == 1 else torch.uint8, device=DEV)
    scales = torch.empty(O.nblocks(n), device=DEV) if codec == 2 else None
    total = d[0] if in_place else (torch.empty(n, device=DEV) if store_sum else None)
    gb.gb_reduce_encode(codec, codes, scales, d, total, mode)
    torch.cuda.synchronize()
    c = codes.view(torch.int16).cpu().numpy().view(np.uint16) if codec == 1 else codes.cpu().numpy()
    return (total.cpu().numpy() if total is not None else None), c, \
        (scales.cpu().numpy() if scales is not None else None)


def check(got, xs, codec, mode, what):
    tot, codes, scales = got
    want_sum = O.reduce_sum(xs)
    if codec == 1:
        assert (codes == O.encode_bf16(want_sum)).all(), what
    else:
        wc, ws = O.encode_fp8(want_sum, mode)
        assert (codes == wc).all(), what
        assert (u32(scales) == u32(ws)).all(), what
    if tot is not None:
        assert (u32(tot) == u32(want_sum)).all(), what


@pytest.mark.parametrize("codec,mode", [(1, 0), (2, 0), (2, 1)])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 8, 9, 16])
@pytest.mark.parametrize("n", [1, 255, 4096 + 77, 3 * 65536 + 300])
def test_reduce_encode(gb, k, n, codec, mode):
    xs = inputs(k, n, 7100 + k + n % 97)
    store = k > 8 or (n % 2 == 1)
    check(run(gb, xs, codec, mode, store), xs, codec, mode, f"k={k} n={n} codec={codec} mode={mode}")


@pytest.mark.parametrize("codec", [1, 2])
def test_in_place_on_the_first_source(gb, codec):
    xs = inputs(4, 65536 + 5, 7200)
    check(run(gb, xs, codec, 0, True, in_place=True), xs, codec, 0, "in place")


def test_equals_sum_then_encode_at_the_two_rank_size(gb):
    """The 4 MiB two-rank workload's path: the fused call gives the same sum
    and codes as gb_reduce_sum followed by gb_encode_bf16."""
    xs = W.normal_ranks(2, W.TWO_RANK_N)
    d = [torch.from_numpy(x).to(DEV) for x in xs]
    s1, s2 = torch.empty(W.TWO_RANK_N, device=DEV), torch.empty(W.TWO_RANK_N, device=DEV)
    c1 = torch.empty(W.TWO_RANK_N, dtype=torch.uint16, device=DEV)
    c2 = torch.empty(W.TWO_RANK_N, dtype=torch.uint16, device=DEV)
    gb.gb_reduce_sum(s1, d)
    gb.gb_encode_bf16(c1, s1)
    gb.gb_reduce_encode(gb.GB_CODEC_BF16, c2, None, d, s2)
    torch.cuda.synchronize()
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_rejects_many_sources_without_a_sum(gb):
    xs = [torch.zeros(512, device=DEV) for _ in range(9)]
    codes = torch.empty(512, dtype=torch.uint16, device=DEV)
    with pytest.raises(gb.GbError, match="sum first"):
        gb.gb_reduce_encode(gb.GB_CODEC_BF16, codes, None, xs)
