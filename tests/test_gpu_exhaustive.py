"""Exhaustive GPU parity of the two encoders against the CPU oracle.

bf16: every one of the 2^32 float32 bit patterns through gb_encode_bf16.
fp8: every float32 with |x| <= 448 (every non-NaN pattern up to 0x43E00000,
both signs) through gb_encode_fp8_e4m3_blockscaled, 255 per block with a 448
planted first so the block scale is 1 in both scale modes; every quotient
the encoder can form from a block with a normal scale lies in this range.

Each test covers one chunk of the patterns, so no single test runs long; the
oracle runs on the host's cores in parallel (its C code releases the GIL).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu, pytest.mark.exhaustive]

from oracle import oracle as O  # noqa: E402

DEV = "cuda:0"
THREADS = max(1, min(16, os.cpu_count() or 1))
BF16_CHUNK = 1 << 28
FP8_CHUNK_BLOCKS = 1 << 20          # blocks per test (255 patterns each)
FP8_LIMIT = 0x43E00000              # bits of 448.0
FP8_PER_SIGN = FP8_LIMIT + 1        # patterns 0 .. 0x43E00000
FP8_PATTERNS = 2 * FP8_PER_SIGN
FP8_TESTS = -(-FP8_PATTERNS // (255 * FP8_CHUNK_BLOCKS))


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def parallel(fn, arrays, parts):
    """Apply a per-array oracle function to `parts` slices concurrently."""
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        return list(ex.map(fn, np.array_split(arrays, parts)))


@pytest.mark.parametrize("chunk", range((1 << 32) // BF16_CHUNK))
def test_bf16_every_pattern(gb, chunk):
    base = chunk * BF16_CHUNK
    u = torch.arange(base, base + BF16_CHUNK, dtype=torch.int64, device=DEV)
    u = torch.where(u >= 1 << 31, u - (1 << 32), u)  # the same 32 bits as a signed int32
    x = u.to(torch.int32).view(torch.float32)
    codes = torch.empty(BF16_CHUNK, dtype=torch.uint16, device=DEV)
    gb.gb_encode_bf16(codes, x)
    got = codes.view(torch.int16).cpu().numpy().view(np.uint16)
    xh = np.arange(base, base + BF16_CHUNK, dtype=np.uint64).astype(np.uint32).view(np.float32)
    want = np.concatenate(parallel(O.encode_bf16, xh, 4 * THREADS))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, first patterns {[hex(base + int(b)) for b in bad[:4]]}"


def fp8_patterns(t):
    """Patterns t*255*B .. of the |x| <= 448 set: 0..LIMIT positive, then the
    same with the sign bit."""
    lo = t * 255 * FP8_CHUNK_BLOCKS
    hi = min(lo + 255 * FP8_CHUNK_BLOCKS, FP8_PATTERNS)
    i = np.arange(lo, hi, dtype=np.uint64)
    u = np.where(i < FP8_PER_SIGN, i, (i - FP8_PER_SIGN) | 0x80000000).astype(np.uint32)
    return u.view(np.float32)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("t", range(FP8_TESTS))
def test_fp8_every_value_up_to_448(gb, t, mode):
    if mode == 1 and t % 4 != 0:
        pytest.skip("the power-of-two mode repeats every fourth chunk: with 448 planted both "
                    "modes give the scale 1 and the same quotients")
    x = fp8_patterns(t)
    nb = -(-x.size // 255)
    blk = np.zeros((nb, 256), np.float32)
    blk[:, 0] = 448.0
    flat = np.zeros(nb * 255, np.float32)
    flat[:x.size] = x
    blk[:, 1:] = flat.reshape(nb, 255)
    buf = blk.reshape(-1)
    codes = torch.empty(buf.size, dtype=torch.uint8, device=DEV)
    scales = torch.empty(nb, dtype=torch.float32, device=DEV)
    gb.gb_encode_fp8_e4m3_blockscaled(codes, scales, torch.from_numpy(buf).to(DEV), mode)
    got_c = codes.cpu().numpy()
    got_s = scales.cpu().numpy()
    parts = parallel(lambda a: O.encode_fp8(a, mode), blk, 4 * THREADS)
    want_c = np.concatenate([p[0] for p in parts])
    want_s = np.concatenate([p[1] for p in parts])
    assert (want_s == 1.0).all()
    assert (got_s.view(np.uint32) == want_s.view(np.uint32)).all()
    bad = np.flatnonzero(got_c != want_c)
    assert bad.size == 0, f"{bad.size} mismatches, first values {buf[bad[:4]]}"
