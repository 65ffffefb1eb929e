"""Writes tests/golden/hashes.json: SHA-256 of the oracle's whole outputs on
the host-drawn workloads at their full sizes.  Calls only the oracle
(oracle/) and the seeded input generators (workloads.py).

    python tests/golden/make_hashes.py      # about a minute on one core

Each entry names a workload, the output and its element type; the hash is of
the output's raw little-endian bytes.  The GPU test compares the library's
outputs in the benchmark's launch configuration with these, so whole outputs
are checked at sizes the oracle cannot redo inside a test.
"""
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hashes.json")


def sha(a):
    return hashlib.sha256(a.tobytes()).hexdigest()


def two_rank_4mib():
    xs = W.normal_ranks(2, W.TWO_RANK_N)
    s = O.reduce_sum(xs)
    c = O.encode_bf16(s)
    d = O.decode_accumulate([c], None, O.CODEC_BF16)
    return {"two_rank_4mib/sum": sha(s), "two_rank_4mib/bf16_codes": sha(c), "two_rank_4mib/decoded": sha(d)}


def two_island_sweep():
    h = {}
    for n in W.SWEEP_SIZES:
        h[f"two_island_sweep/sum/{n}"] = sha(O.reduce_sum(W.normal_ranks(2, n)))
    n = W.SWEEP_SIZES[-1]
    h[f"two_island_sweep/bf16_sum/{n}"] = sha(O.reduce_typed(W.typed_ranks(2, n, "bf16"), "bf16", O.OP_SUM))
    return h


def gradients_64mib():
    xs = W.gradient_ranks(4, W.GRAD64_N)
    codes = [O.encode_bf16(x) for x in xs]
    h = {f"gradients_64mib/bf16_codes/{r}": sha(c) for r, c in enumerate(codes)}
    h["gradients_64mib/decoded_sum"] = sha(O.decode_accumulate(codes, None, O.CODEC_BF16))
    return h


def gradients_256mib():
    xs = W.gradient_ranks(4, W.GRAD256_N)
    h = {}
    for mode, tag in ((O.SCALE_ABSMAX_DIV_448, "absmax_div_448"), (O.SCALE_POW2, "pow2")):
        enc = [O.encode_fp8(x, mode) for x in xs]
        for r, (c, s) in enumerate(enc):
            h[f"gradients_256mib/{tag}/fp8_codes/{r}"] = sha(c)
            h[f"gradients_256mib/{tag}/scales/{r}"] = sha(s)
        h[f"gradients_256mib/{tag}/decoded_sum"] = sha(
            O.decode_accumulate([c for c, _ in enc], [s for _, s in enc], O.CODEC_FP8))
    return h


BUILDERS = {"two_rank_4mib": two_rank_4mib, "two_island_sweep": two_island_sweep,
            "gradients_64mib": gradients_64mib, "gradients_256mib": gradients_256mib}


def main():
    hashes = {}
    for name, fn in BUILDERS.items():
        t0 = time.perf_counter()
        hashes.update(fn())
        print(f"{name}: {time.perf_counter() - t0:.1f} s", flush=True)
    with open(OUT, "w") as f:
        json.dump({"generated_by": "tests/golden/make_hashes.py (oracle and workloads.py only)",
                   "hash": "sha256 of the output's raw little-endian bytes", "outputs": hashes}, f, indent=1,
                  sort_keys=True)
        f.write("\n")
    print(f"wrote {len(hashes)} hashes to {OUT}")


if __name__ == "__main__":
    main()
