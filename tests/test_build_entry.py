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
