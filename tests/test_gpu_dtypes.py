"""GPU parity of gb_reduce_typed over float16, bfloat16, float64, int8, uint8,
int32 and int64 against the CPU oracle's reduce_typed: bit for bit (NaN
compares as NaN), at sizes spanning several workgroups with ragged tails,
every 16-bit code as a first operand, divisors up to 2^24 for AVG, and the
sweep's largest size in the benchmark's launch configuration."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"
FLOATS = ["f16", "bf16", "f64"]
INTS = ["i8", "u8", "i32", "i64"]
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64, "i8": torch.int8,
         "u8": torch.uint8, "i32": torch.int32, "i64": torch.int64}
# 16-bit codes travel as int16 (numpy has no bfloat16), then are viewed as the type
CARRIER = {"f16": (np.int16, torch.int16), "bf16": (np.int16, torch.int16)}
SIZES = [1, 5, 3 * 4096 + 5, 3 * 262144 + 7]


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def to_dev(a, dt):
    if dt in CARRIER:
        npc, tc = CARRIER[dt]
        return torch.from_numpy(np.ascontiguousarray(a).view(npc).copy()).to(DEV).view(TORCH[dt])
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t, dt):
    if dt in CARRIER:
        return t.view(CARRIER[dt][1]).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def values(a, dt):
    """Floating values of raw arrays, for locating NaN."""
    if dt == "f16":
        return a.view(np.float16).astype(np.float64)
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a


def same(got, want, dt, what):
    if dt in FLOATS:
        gn, wn = np.isnan(values(got, dt)), np.isnan(values(want, dt))
        assert (gn == wn).all(), f"{what}: NaN positions differ"
        got, want = got[~gn], want[~wn]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:4]}: {got[bad[:4]]} vs {want[bad[:4]]}"


def inputs(dt, k, n, seed):
    """k arrays of type dt: gradient-like values with every special value
    mixed in (floats), or the type's whole range (integers)."""
    rng = np.random.default_rng(seed)
    xs = []
    for r in range(k):
        if dt == "f16":
            x = (rng.standard_normal(n) * 3.0).astype(np.float16).view(np.uint16)
            m = rng.random(n) < 0.25
            x[m] = rng.integers(0, 1 << 16, int(m.sum())).astype(np.uint16)  # any code
        elif dt == "bf16":
            f = (rng.standard_normal(n) * 1e-3).astype(np.float32).view(np.uint32)
            x = (f >> 16).astype(np.uint16)
            m = rng.random(n) < 0.25
            x[m] = rng.integers(0, 1 << 16, int(m.sum())).astype(np.uint16)
        elif dt == "f64":
            x = rng.standard_normal(n) * 10.0 ** rng.integers(-300, 300, n)
            pool = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 5e-324, -5e-324, 1.7e308, -1.7e308])
            m = rng.random(n) < 0.05
            x[m] = pool[rng.integers(0, pool.size, int(m.sum()))]
        else:
            info = np.iinfo(O.NP_DTYPES[dt])
            x = rng.integers(info.min, info.max, n, endpoint=True, dtype=O.NP_DTYPES[dt])
        xs.append(x)
    return xs


def run(gb, xs, dt, op, divisor=1):
    out = torch.empty(xs[0].size, dtype=TORCH[dt], device=DEV)
    gb.gb_reduce_typed(out, [to_dev(x, dt) for x in xs], op, divisor)
    torch.cuda.synchronize()
    return to_host(out, dt)


CASES = [(dt, op) for dt in FLOATS for op in (0, 1, 2, 3)] + [(dt, op) for dt in INTS for op in (0, 2, 3)]


@pytest.mark.parametrize("dt,op", CASES)
@pytest.mark.parametrize("k", [1, 2, 5, 8])
@pytest.mark.parametrize("n", SIZES)
def test_reduce_typed(gb, dt, op, k, n):
    xs = inputs(dt, k, n, 2000 + 17 * k + op + 100 * list(TORCH).index(dt))
    divisor = {1: 1, 2: 2, 5: 7, 8: 64}[k]
    same(run(gb, xs, dt, op, divisor), O.reduce_typed(xs, dt, op, divisor), dt, f"{dt} op={op} k={k} n={n}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("op", [0, 2, 3])
def test_every_code_as_first_operand(gb, dt, op):
    rng = np.random.default_rng(2100 + op)
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for rep in range(4):
        b = rng.integers(0, 1 << 16, a.size).astype(np.uint16)
        xs = [a, b]
        same(run(gb, xs, dt, op), O.reduce_typed(xs, dt, op), dt, f"{dt} op={op} rep={rep}")


@pytest.mark.parametrize("dt,divisor", [("f16", 3), ("f16", 99991), ("f16", (1 << 24) - 1), ("f16", 1 << 24),
                                        ("f16", 64), ("bf16", 2), ("bf16", 1 << 24),
                                        ("bf16", 257), ("bf16", 12345679), ("bf16", (1 << 24) - 1),
                                        ("f64", 3), ("f64", (1 << 24) - 1), ("f64", 1 << 24)])
def test_avg_every_value_and_large_divisors(gb, dt, divisor):
    """AVG of one rank divides each value once; for bfloat16 near the
    subnormal range a binary32 quotient rounded to nearest would double-round
    at divisor 2^24 - 1, so this pins the kernel's rounding of the quotient.
    Powers of two (a multiply by the reciprocal) reach the subnormals too."""
    if dt == "f64":
        x = inputs("f64", 1, 1 << 16, 2200 + divisor % 97)[0]
    else:
        x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    same(run(gb, [x], dt, 1, divisor), O.reduce_typed([x], dt, 1, divisor), dt, f"{dt} avg d={divisor}")


@pytest.mark.parametrize("dt", ["i32", "bf16"])
def test_in_place_on_the_first_source(gb, dt):
    xs = inputs(dt, 3, 4096 * 5 + 3, 2300)
    op = 0 if dt == "i32" else 1
    d = [to_dev(x, dt) for x in xs]
    gb.gb_reduce_typed(d[0], d, op, 3)
    torch.cuda.synchronize()
    same(to_host(d[0], dt), O.reduce_typed(xs, dt, op, 3), dt, f"{dt} in place")


def test_f32_is_gb_reduce(gb):
    xs = W.normal_ranks(3, 10007, 2400)
    a = torch.empty(10007, device=DEV)
    b = torch.empty(10007, device=DEV)
    d = [torch.from_numpy(x).to(DEV) for x in xs]
    gb.gb_reduce_typed(a, d, gb.GB_OP_AVG, 3)
    gb.gb_reduce(b, d, gb.GB_OP_AVG, 3)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    same(a.cpu().numpy().view(np.uint32), O.reduce_typed(xs, "f32", 1, 3).view(np.uint32), "f32", "f32 avg")


@pytest.mark.parametrize("dt,op", [("f16", 0), ("bf16", 0), ("bf16", 1), ("f64", 0), ("i8", 0), ("u8", 2),
                                   ("i32", 0), ("i64", 3)])
def test_sweep_largest_size_whole(gb, dt, op):
    """Two ranks at the sweep's largest size (2^26 elements), the call the
    benchmark times, checked whole."""
    n = W.SWEEP_SIZES[-1]
    xs = inputs(dt, 2, n, 2500 + op)
    same(run(gb, xs, dt, op, 2), O.reduce_typed(xs, dt, op, 2), dt, f"{dt} op={op} n={n}")


def test_rejects_avg_on_integers_and_mixed_types(gb):
    x = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(gb.GbError, match="floating-point"):
        gb.gb_reduce_typed(x, [x], gb.GB_OP_AVG, 2)
    with pytest.raises(TypeError):
        gb.gb_reduce_typed(x, [x.view(torch.float32)], gb.GB_OP_SUM)


@pytest.mark.parametrize("dt", FLOATS + INTS)
@pytest.mark.parametrize("k", range(1, 9))
def test_every_rank_count(gb, dt, k):
    """Each rank count is its own kernel instantiation: SUM and MAX at a size
    with full workgroups and a ragged one."""
    n = 2 * 4096 + 3
    xs = inputs(dt, k, n, 2600 + k)
    for op in (0, 2):
        same(run(gb, xs, dt, op), O.reduce_typed(xs, dt, op), dt, f"{dt} op={op} k={k}")
