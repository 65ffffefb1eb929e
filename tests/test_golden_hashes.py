"""The stored golden hashes (tests/golden/hashes.json, written by
tests/golden/make_hashes.py from the oracle alone) still match the oracle:
the cheap entries are recomputed here, CPU only."""
import hashlib
import json
import os

from oracle import oracle as O
import workloads as W

HASHES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hashes.json")))["outputs"]


def sha(a):
    return hashlib.sha256(a.tobytes()).hexdigest()


def test_two_rank_entries():
    xs = W.normal_ranks(2, W.TWO_RANK_N)
    s = O.reduce_sum(xs)
    c = O.encode_bf16(s)
    assert HASHES["two_rank_4mib/sum"] == sha(s)
    assert HASHES["two_rank_4mib/bf16_codes"] == sha(c)
    assert HASHES["two_rank_4mib/decoded"] == sha(O.decode_accumulate([c], None, O.CODEC_BF16))


def test_sweep_entries_up_to_a_mebivalue():
    for n in W.SWEEP_SIZES:
        if n <= 1 << 20:
            assert HASHES[f"two_island_sweep/sum/{n}"] == sha(O.reduce_sum(W.normal_ranks(2, n))), n


def test_every_workload_output_has_an_entry():
    keys = set(HASHES)
    assert {f"two_island_sweep/sum/{n}" for n in W.SWEEP_SIZES} <= keys
    for tag in ("absmax_div_448", "pow2"):
        for r in range(4):
            assert f"gradients_256mib/{tag}/fp8_codes/{r}" in keys
            assert f"gradients_256mib/{tag}/scales/{r}" in keys
    assert {f"gradients_64mib/bf16_codes/{r}" for r in range(4)} <= keys
