"""The oracle and the HIP path share no code, and the product path never
reaches the oracle (CPU only, by reading the sources):

- nothing under oracle/ names the package, its sources or its header;
- no library source (the HIP kernels, the C ABI, the binding, the build)
  names the oracle;
- the only modules both sides' callers share are the seeded input
  generators (workloads.py), which hold none of the method's arithmetic:
  no rounding, encoding, scale or decode code;
- the product modules that may reach the oracle are the ones allowed to:
  tests, __graft_entry__.smoke() and bench.py's CPU baseline.
"""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gradient_all_reduce_amd")


def files(d, exts):
    for base, _, names in os.walk(d):
        for n in names:
            if n.endswith(exts):
                yield os.path.join(base, n)


def text(p):
    return open(p, encoding="utf-8").read()


def test_oracle_names_nothing_of_the_library():
    for p in files(os.path.join(ROOT, "oracle"), (".c", ".h", ".py")):
        t = text(p)
        for word in ("gradient_all_reduce_amd", "csrc", "gbreduce.h", "gb_device", "gb_internal", "libgbreduce"):
            assert word not in t, (p, word)
        assert not re.search(r'#\s*include\s*[<"]hip', t), p  # no HIP header in the C oracle


def test_library_sources_name_nothing_of_the_oracle():
    for p in files(PKG, (".hip", ".h", ".cpp", ".py")):
        assert not re.search(r"\boracle\b", text(p)), p
    assert not re.search(r"\boracle\b", text(os.path.join(ROOT, "include", "gbreduce.h")))


def test_shared_input_module_holds_no_arithmetic_of_the_method():
    """workloads.py defines only seeded generators (its edge values are input
    data) and performs no rounding, encoding, scaling or decoding step."""
    t = text(os.path.join(ROOT, "workloads.py"))
    defined = {n.name for n in ast.walk(ast.parse(t)) if isinstance(n, ast.FunctionDef)}
    assert defined <= {"normal", "normal_ranks", "gradients", "gradient_ranks", "ddp_buckets", "device_gradients",
                       "typed", "typed_ranks", "device_gradients_typed", "special_values"}, defined
    for pattern in (r"0x7[fF]{3}\b", r"/\s*448", r"448(\.0)?\s*\*", r"float8", r"\brint\(", r"nearbyint",
                    r"\bencode", r"\bdecode", r"absmax"):
        assert not re.search(pattern, t), pattern


def imports_oracle(path):
    tree = ast.parse(text(path))
    for node in ast.walk(tree):
        if isinstance(node, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in node.names):
            yield node
        if isinstance(node, ast.ImportFrom) and (node.module or "").split(".")[0] == "oracle":
            yield node


def enclosing_function(tree, node):
    for fn in ast.walk(tree):
        if isinstance(fn, (ast.FunctionDef, ast.AsyncFunctionDef)):
            if fn.lineno <= node.lineno <= max(getattr(fn, "end_lineno", fn.lineno), fn.lineno):
                yield fn.name


def test_only_the_allowed_callers_reach_the_oracle():
    allowed = {"__graft_entry__.py": {"smoke"}, "bench.py": {"cpu_units", "factory", "make", "compute", "check"}}
    product = [os.path.join(ROOT, n) for n in os.listdir(ROOT) if n.endswith(".py")] + list(files(PKG, (".py",)))
    for p in product:
        rel = os.path.relpath(p, ROOT)
        hits = list(imports_oracle(p))
        if not hits:
            continue
        assert rel in allowed, rel
        tree = ast.parse(text(p))
        for node in hits:
            names = set(enclosing_function(tree, node))
            assert names & allowed[rel], (rel, node.lineno, names)
