"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C ABI layer of libgbreduce (gb_api.cpp, built with g++ against the
host stand-ins of tests/sanitize/stub_hip.cpp, driven by
tests/sanitize/api_driver.c: validation, the refusal of overlapping buffers,
the launches a call plans, and a launch failure injected at every launch of
several multi-launch calls; then the GB_DEBUG and GB_TRACE hooks), and the
CPU oracle (gb_oracle.c, driven by
tests/sanitize/oracle_driver.c over ragged sizes and special values).  The
two are built and run apart.  Any sanitizer report aborts the program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
HIP_INCLUDE = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_layer_under_sanitizers(tmp_path):
    if not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not installed")
    cxx = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include")]
    api = tmp_path / "gb_api.o"
    stub = tmp_path / "stub_hip.o"
    drv = tmp_path / "api_driver.o"
    exe = tmp_path / "api_driver"
    run([*cxx, "-c", os.path.join(ROOT, "gradient_all_reduce_amd", "csrc", "gb_api.cpp"), "-o", str(api)])
    run([*cxx, "-c", os.path.join(HERE, "stub_hip.cpp"), "-o", str(stub)])
    run(["gcc", "-std=c11", *SAN, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "api_driver.c"),
         "-o", str(drv)])
    run(["g++", *SAN, str(api), str(stub), str(drv), "-o", str(exe)])
    env = {k: v for k, v in os.environ.items() if k not in ("GB_TRACE", "GB_DEBUG")}
    out = run([str(exe)], env=dict(env, ASAN_OPTIONS="detect_leaks=1"))
    assert "0 failed" in out.stdout, out.stdout + out.stderr
    assert "runtime error" not in out.stderr
    assert "gbreduce:" not in out.stderr  # no trace unless GB_TRACE is set

    # the per-call hooks: GB_DEBUG waits for the stream after each call that
    # enqueued work, GB_TRACE prints one line per call
    out = run([str(exe), "hooks"], env=dict(env, ASAN_OPTIONS="detect_leaks=1", GB_TRACE="1", GB_DEBUG="1"))
    assert "0 failed" in out.stdout, out.stdout + out.stderr
    assert "runtime error" not in out.stderr
    trace = [line for line in out.stderr.splitlines() if line.startswith("gbreduce: ")]
    assert len(trace) == 5, out.stderr
    assert trace[0].startswith("gbreduce: gb_reduce_sum k=1 n=10 stream=") and "-> GB_OK" in trace[0]
    assert "gb_bucket_allreduce_local k=1 n=1000 codec=2" in trace[1] and "-> GB_OK" in trace[1]
    assert "-> GB_ERR_HIP: gb_reduce_sum: GB_DEBUG: the stream reported HIP error" in trace[2]
    assert "-> GB_OK (stream under capture: not waited for)" in trace[3]
    assert "-> GB_ERR_INVALID_ARG: gb_reduce_sum: k = 0 is outside 1..16" in trace[4]


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-fno-fast-math", "-I", os.path.join(ROOT, "oracle"),
         os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "gb_oracle.c"), "-lm", "-o", str(exe)])
    out = run([str(exe)], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "0 failed" in out.stdout, out.stdout + out.stderr
    assert "runtime error" not in out.stderr
