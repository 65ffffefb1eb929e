"""Seeded synthetic inputs for the tests and the benchmark.

This module draws random numbers and nothing else: it holds none of the
arithmetic under test, and it is the only code the GPU path's callers and the
oracle's callers share.  Every input is float32 unless typed_ranks draws it
in another element type.

Workloads (all seeds start at BASE_SEED; rank r uses BASE_SEED + r):
  two_rank_4mib      k=2, n=1,048,576, N(0,1).
  two_island_sweep   k=2, n=2^8 .. 2^26 (1 KiB .. 256 MiB per rank), N(0,1),
                     the same per-rank seeds at every size.  With another element
                     type: the same N(0,1) draws carried into that type
                     (typed_ranks).
  gradients_64mib    k=4, n=16,777,216, N(0, sigma=1e-3), then floor(n/100)
                     distinct positions drawn without replacement scaled by
                     100 (outliers).
  gradients_256mib   k=4, n=67,108,864, same distribution.
  ddp_1b_buckets     k=4, n=1,000,000,000, N(0, sigma=1e-3), no outliers,
                     25 MiB buckets of 6,553,600 values (152 full + one of
                     3,852,800); drawn on the GPU with torch's seeded device
                     generator (16 GB would take minutes on the host).
Normal draws are numpy's default_rng(seed).standard_normal(dtype=float32)
(or torch.randn for the device workload), scaled by a float32 multiply.
"""
import numpy as np

BASE_SEED = 0

TWO_RANK_N = 1 << 20
SWEEP_SIZES = [1 << p for p in range(8, 27)]  # elements: 1 KiB .. 256 MiB of fp32
GRAD64_N = 1 << 24
GRAD256_N = 1 << 26
DDP_N = 1_000_000_000
DDP_BUCKET = 25 * (1 << 20) // 4  # 25 MiB of fp32 = 6,553,600 values
SIGMA = np.float32(1e-3)
OUTLIER_SCALE = np.float32(100.0)


def normal(n, seed):
    """n float32 values N(0, 1) from the given seed."""
    return np.random.default_rng(seed).standard_normal(n, dtype=np.float32)


def normal_ranks(k, n, base_seed=BASE_SEED):
    return [normal(n, base_seed + r) for r in range(k)]


def gradients(n, seed):
    """N(0, sigma=1e-3) with floor(n/100) distinct positions scaled by 100."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32) * SIGMA
    idx = rng.choice(n, n // 100, replace=False)
    x[idx] *= OUTLIER_SCALE
    return x


def gradient_ranks(k, n, base_seed=BASE_SEED):
    return [gradients(n, base_seed + r) for r in range(k)]


def ddp_buckets(n=DDP_N, bucket=DDP_BUCKET):
    """(start, length) of every bucket of an n-value gradient buffer."""
    return [(s, min(bucket, n - s)) for s in range(0, n, bucket)]


def device_gradients(n, seed, device):
    """N(0, sigma=1e-3) float32 drawn on a torch device with a seeded generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    x.mul_(float(SIGMA))
    return x


def typed(n, dtype, seed):
    """n values of element type `dtype` ("f32", "f16", "bf16", "f64", "i8", "u8",
    "i32", "i64") from the given seed.  Floating types carry the N(0,1) draw:
    float16 by numpy's conversion, bfloat16 as the top 16 bits of the float32
    draw (uint16 codes, truncated: a draw, not a rounding under test), float64
    by widening.  Integer types are uniform over the type's whole range."""
    if dtype in ("f32", "f16", "bf16", "f64"):
        x = normal(n, seed)
        if dtype == "f32":
            return x
        if dtype == "f16":
            return x.astype(np.float16).view(np.uint16)
        if dtype == "bf16":
            return (x.view(np.uint32) >> 16).astype(np.uint16)
        return x.astype(np.float64)
    t = {"i8": np.int8, "u8": np.uint8, "i32": np.int32, "i64": np.int64}[dtype]
    info = np.iinfo(t)
    return np.random.default_rng(seed).integers(info.min, info.max, n, endpoint=True, dtype=t)


def typed_ranks(k, n, dtype, base_seed=BASE_SEED):
    return [typed(n, dtype, base_seed + r) for r in range(k)]


def device_gradients_typed(n, seed, device, dtype):
    """device_gradients carried into float16 (torch's conversion), bfloat16
    (the top 16 bits of each float32 draw: truncated, a draw and not a
    rounding under test) or float64 (widened)."""
    import torch

    x = device_gradients(n, seed, device)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.half()
    if dtype == "f64":
        return x.double()
    return (x.view(torch.int32) >> 16).to(torch.int16).view(torch.bfloat16)


def special_values():
    """float32 values where rounding and the format edges are decided."""
    u = np.array([
        0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x00800000,
        0x3F800000, 0xBF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
        0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFBFFFFF, 0x7FA00000,
        0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001,  # bf16 ties and near ties
        0x43E00000, 0x43E00001, 0x43E80000, 0x43F00000,  # 448, above, 464, 480
        0x3A800000, 0x3AC00000, 0x3B400000, 0x3C800000, 0x3C7FFFFF,  # E4M3 subnormal edges
    ], dtype=np.uint32)
    return u.view(np.float32)
