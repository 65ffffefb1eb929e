"""The per-call hooks of libgbreduce on the GPU: GB_TRACE prints one line per
call, GB_DEBUG waits for the stream after a call that enqueued work and skips
the wait for a stream under graph capture.  Both are read once per process,
so the calls run in a child process started with them set; the child checks
its own results (the sum of two ranks against torch's, bit for bit) and the
parent checks the trace lines."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, torch
import gradient_all_reduce_amd as gb
n = 1000003
x = [torch.randn(n, device="cuda") for _ in range(2)]
out = torch.empty_like(x[0])
gb.gb_reduce_sum(out, x)
torch.cuda.synchronize()
assert torch.equal(out, x[0] + x[1]), "eager sum"
try:
    gb.gb_reduce_sum(out, [x[0]] * 17)
    raise AssertionError("k = 17 was accepted")
except gb.GbError as e:
    assert e.status == gb.GB_ERR_INVALID_ARG
g = torch.cuda.CUDAGraph()
out2 = torch.zeros_like(out)
with torch.cuda.graph(g):
    gb.gb_reduce_sum(out2, x)
g.replay()
torch.cuda.synchronize()
assert torch.equal(out2, out), "captured sum"
print("child ok", flush=True)
"""


def test_trace_and_debug_hooks():
    env = dict(os.environ, GB_TRACE="1", GB_DEBUG="1", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    print("[hooks] child with GB_TRACE=1 GB_DEBUG=1", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "child ok" in r.stdout
    trace = [line for line in r.stderr.splitlines() if line.startswith("gbreduce: ")]
    assert len(trace) == 3, r.stderr
    assert trace[0].startswith("gbreduce: gb_reduce_sum k=2 n=1000003 stream=") and "-> GB_OK (" in trace[0]
    assert "-> GB_ERR_INVALID_ARG: gb_reduce_sum: k = 17 is outside 1..16" in trace[1]
    assert "-> GB_OK (stream under capture: not waited for)" in trace[2]
