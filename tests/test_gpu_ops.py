"""GPU parity of gb_reduce (SUM, AVG, MAX, MIN) against the CPU oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"
SIZES = [1, 3, 257, 1024, 4096 + 7, 3 * 262144 + 5]


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def same(got, want, what):
    """Every bit, NaN included (the canonical NaN on both sides)."""
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"{what}: {bad.size} mismatches at {bad[:5]}"


def inputs(k, n, seed):
    xs = W.normal_ranks(k, n, seed)
    rng = np.random.default_rng(seed)
    pool = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45], dtype=np.float32)
    for x in xs:
        m = max(1, n // 20)
        idx = rng.choice(n, m, replace=False)
        x[idx] = pool[rng.integers(0, pool.size, m)]
    return xs


@pytest.mark.parametrize("op", [0, 1, 2, 3])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n", SIZES)
def test_reduce_ops(gb, n, k, op):
    xs = inputs(k, n, 1000 + 10 * k + op)
    divisor = {1: 1, 2: 2, 3: 6, 4: 12, 8: 64}[k]
    out = torch.empty(n, device=DEV)
    gb.gb_reduce(out, [dev(x) for x in xs], op, divisor)
    torch.cuda.synchronize()
    same(out.cpu().numpy(), O.reduce(xs, op, divisor), f"op={op} k={k} n={n}")


@pytest.mark.parametrize("divisor", [3, 7, 1000, 1 << 24])
def test_avg_divisors_and_in_place(gb, divisor):
    xs = W.normal_ranks(4, 10007, 77)
    d = [dev(x) for x in xs]
    gb.gb_reduce(d[0], d, gb.GB_OP_AVG, divisor)
    torch.cuda.synchronize()
    same(d[0].cpu().numpy(), O.reduce(xs, O.OP_AVG, divisor), f"avg d={divisor}")


@pytest.mark.parametrize("codec", [1, 2])
def test_compressed_avg_is_decode_then_divide(gb, codec):
    """A compressed AVG: decode-accumulate the payloads, then divide in place."""
    k, n, world = 4, 65536 + 9, 16
    xs = W.gradient_ranks(k, n, 88)
    if codec == 1:
        codes = [O.encode_bf16(x) for x in xs]
        dcodes = [dev(c.view(np.int16)).view(torch.uint16) for c in codes]
        dscales, scales = None, None
    else:
        enc = [O.encode_fp8(x, 0) for x in xs]
        codes, scales = [c for c, _ in enc], [s for _, s in enc]
        dcodes, dscales = [dev(c) for c in codes], [dev(s) for s in scales]
    acc = torch.empty(n, device=DEV)
    gb.gb_decode_accumulate(acc, dcodes, dscales, codec)
    gb.gb_reduce(acc, [acc], gb.GB_OP_AVG, world)
    torch.cuda.synchronize()
    summed = O.decode_accumulate(codes, scales, codec)
    same(acc.cpu().numpy(), O.reduce([summed], O.OP_AVG, world), "compressed avg")


@pytest.mark.parametrize("divisor", [2, 1024, 1 << 24, 3, (1 << 24) - 1])
def test_avg_over_every_binade(gb, divisor):
    """AVG of one rank over random bit patterns spanning every binade,
    subnormals included: a power-of-two divisor (taken as a multiply by its
    exact reciprocal) and any other divisor both give the once-rounded
    quotient, also where it underflows."""
    rng = np.random.default_rng(1100 + divisor % 1000)
    x = rng.integers(0, 1 << 32, 300007, dtype=np.uint64).astype(np.uint32).view(np.float32)
    out = torch.empty(x.size, device=DEV)
    gb.gb_reduce(out, [dev(x)], gb.GB_OP_AVG, divisor)
    torch.cuda.synchronize()
    same(out.cpu().numpy(), O.reduce([x], O.OP_AVG, divisor), f"avg d={divisor}")
