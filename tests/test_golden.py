"""The README's worked example ("Simulation mode": four ranks in two islands,
10.0 on every rank) through every path of the oracle (CPU only)."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.golden import load_rank_example


def test_uncompressed_sum_gives_the_printed_value():
    xs, want = load_rank_example("simulate_two_islands.txt")
    assert (O.reduce_sum(xs) == want).all()
    # the leader arithmetic of reduce-bridge-broadcast: each island sums onto
    # its leader, then the leaders' island sums are added
    isl = [O.reduce_sum(xs[:2]), O.reduce_sum(xs[2:])]
    assert (O.reduce_sum(isl) == want).all()


def test_bf16_bridge_gives_the_printed_value():
    xs, want = load_rank_example("simulate_two_islands.txt")
    isl = [O.reduce_sum(xs[:2]), O.reduce_sum(xs[2:])]
    out = O.decode_accumulate([O.encode_bf16(s) for s in isl], None, O.CODEC_BF16)
    assert (out == want).all()


@pytest.mark.parametrize("mode", [O.SCALE_ABSMAX_DIV_448, O.SCALE_POW2])
def test_fp8_bridge_gives_the_printed_value(mode):
    xs, want = load_rank_example("simulate_two_islands.txt")
    for contributions in (xs, [O.reduce_sum(xs[:2]), O.reduce_sum(xs[2:])]):
        enc = [O.encode_fp8(x, mode) for x in contributions]
        out = O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8)
        assert (out == want).all()
        out2, _, _ = O.bucket_allreduce(contributions, 256, O.CODEC_FP8, mode)
        assert (out2 == want).all()
