"""__graft_entry__.build() loads the build scripts without importing the
package: the package's __init__ binds every symbol of the library that is
about to be rebuilt, so a library built before a new entry point was added
would stop the build that adds it (CPU only, nothing compiled)."""
import subprocess
import sys
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_scripts_load_with_the_package_unimportable():
    code = (
        "import sys\n"
        "class Block:\n"
        "    def find_spec(self, name, path=None, target=None):\n"
        "        if name == 'gradient_all_reduce_amd' or name.startswith('gradient_all_reduce_amd.'):\n"
        "            raise ImportError('the package must not be imported to build it')\n"
        "sys.meta_path.insert(0, Block())\n"
        "import __graft_entry__ as g\n"
        "lib = g._load('gradient_all_reduce_amd/build.py', '_t_build')\n"
        "orc = g._load('oracle/build.py', '_t_oracle_build')\n"
        "assert callable(lib.build) and callable(orc.build)\n"
        "assert lib.LIB.endswith('libgbreduce.so')\n"
        "assert 'gradient_all_reduce_amd' not in sys.modules\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_the_binding_fails_loudly_without_the_library(tmp_path):
    """With libgbreduce.so absent the package refuses to import, naming the
    build step: there is no fallback to any other implementation."""
    import shutil
    pkg = tmp_path / "gradient_all_reduce_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "gradient_all_reduce_amd", "__init__.py"), pkg / "__init__.py")
    code = ("import sys\n"
            f"sys.path.insert(0, {str(tmp_path)!r})\n"
            "try:\n"
            "    import gradient_all_reduce_amd\n"
            "except ImportError as e:\n"
            "    assert 'not built' in str(e) and 'build.py' in str(e), e\n"
            "    print('refused')\n"
            "else:\n"
            "    raise SystemExit('imported without the library')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "refused" in r.stdout, r.stderr
