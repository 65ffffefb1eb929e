"""Build libgbreduce.so in-tree with hipcc for gfx950.

The library links the HIP runtime by its soname (libamdhip64.so.7); in a
process that has imported torch first, the dynamic loader reuses the runtime
torch already loaded, so both share one HIP runtime and one device context.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgbreduce.so")
# The kernels are split over several sources so that they compile in parallel.
SOURCES = ["gb_reduce.hip", "gb_codec_fp8.hip", "gb_codec_bf16.hip", "gb_ef.hip", "gb_noalloc.hip",
           "gb_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# The memory-ceiling measurement program bench.py runs (not part of the library).
CEILING_SRC = "gb_ceiling.hip"
CEILING = os.path.join(HERE, "gb_ceiling")

# -ffp-contract=off: no multiply-add fusion, so decode (multiply) and add
#   round separately as the arithmetic requires.
# packed fp32 ops disabled: the compiler may not pair fp32 adds and
#   multiplies into v_pk_* instructions.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE,
]


def build(verbose=False):
    """Compile every source (in parallel) and link the shared library; return
    its path."""
    def compile_one(src):
        obj = os.path.join(CSRC, src.rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    def compile_ceiling():
        tmp = CEILING + ".tmp"
        cmd = [HIPCC, *FLAGS, "-Wno-unused-function", "-x", "hip", os.path.join(CSRC, CEILING_SRC), "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, CEILING)

    jobs = max(1, min(len(SOURCES) + 1, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        ceiling = ex.submit(compile_ceiling)
        objs = list(ex.map(compile_one, SOURCES))
        ceiling.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
