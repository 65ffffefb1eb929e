"""bench.py's host side, without a GPU: what it refuses, the split of a
workload into one GPU's share, and when it takes HBM traffic from the
committed rocprofv3 summaries."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


@pytest.mark.parametrize("workload", ["two_island_sweep", "two_rank_4mib", "staged_fp8_256mib"])
def test_shard_is_refused_where_it_does_not_apply(workload):
    r = run_bench("--workload", workload, "--shard", "8")
    assert r.returncode == 2
    assert "--shard" in r.stderr


def test_shard_zero_is_refused():
    r = run_bench("--shard", "0")
    assert r.returncode == 2


@pytest.mark.parametrize("g", [1, 2, 3, 7, 8, 16])
@pytest.mark.parametrize("length", [1, 255, 256, 257, 3_852_800, W.DDP_BUCKET, W.GRAD64_N, W.DDP_N])
def test_shard_len_is_the_first_of_g_aligned_ranges(length, g):
    s = bench.shard_len(length, g)
    # g ranges of s values each cover the buffer ...
    assert g * s >= length
    # ... each starts on a 256-value block boundary ...
    assert s % 256 == 0 or s == length
    # ... and s is the smallest such length
    assert s == length or (s - 256) * g < length


def test_ddp_share_of_eight_gpus():
    """Every bucket is cut on its own: 152 pieces of 819,200 values and the
    last bucket's piece, 125,000,192 values in all."""
    pieces = [bench.shard_len(l, 8) for _, l in W.ddp_buckets()]
    assert pieces[:-1] == [819_200] * 152
    assert pieces[-1] == 481_792
    assert sum(pieces) == 125_000_192
    # the library's uniform-bucket stream over the share has exactly these buckets
    assert [l for _, l in W.ddp_buckets(sum(pieces), 819_200)] == pieces


def test_profiled_traffic_requires_the_current_kernel_sources():
    """A committed summary's traffic is used only when the summary was taken
    on the kernel sources as they are now; a workload nobody profiled has
    none."""
    assert bench.profiled_traffic("fused_fp8_kernel<4,0>", "no_such_workload") is None
    lines = [ln for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")) for ln in open(path)
             if ln.startswith("traffic ")]
    assert lines, "no traffic lines in profiles/"
    current = bench.kernel_sources_sha256()
    for ln in lines:
        kv = dict(tok.split("=", 1) for tok in ln.split()[1:])
        got = bench.profiled_traffic(kv["kernel"], kv["workload"])
        if kv["kernels_sha256"] == current:
            assert got == int(float(kv["traffic_bytes"]))
            # counted HBM bytes within 5% of the algorithmic bytes: nothing re-read
            assert abs(got / float(kv["algorithmic_bytes"]) - 1) < 0.05, ln
        else:
            assert got is None


def test_memory_ceiling_never_takes_the_zero_data_contrast(monkeypatch, tmp_path):
    """The ceiling program reports a copy of a zero-filled buffer beside the
    copies of gradient-like data, as a contrast (HBM moves zeros faster).
    bench's best copy, the denominator of frac_of_copy_ceiling, must be one
    of the gradient-like copies even when the zero-data copy is faster."""
    res = {"copy_u1_4GiB": 6400.0, "copy_u1_fronts_4GiB": 6600.0, "read_u4_2percu_4GiB": 7500.0,
           "write_u1_4GiB": 6650.0, "zeros_copy_u1_4GiB": 6900.0, "fused_fp8_replica_4GiB": 5800.0}
    out = '{"median_gbs": %s, "launch_us": {"stream_1wg": 2.5}}' % str(res).replace("'", '"')

    class Done:
        returncode, stdout, stderr = 0, "gb_ceiling: buffers of 4 GiB\n" + out + "\n", ""

    exists = os.path.exists
    monkeypatch.setattr(os.path, "exists", lambda p: p.endswith("gb_ceiling") or exists(p))
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Done())
    got = bench.memory_ceiling()
    assert got["best_copy"] == "copy_u1_fronts_4GiB" and got["best_copy_gbs"] == 6600.0
    assert got["median_gbs"]["zeros_copy_u1_4GiB"] == 6900.0
