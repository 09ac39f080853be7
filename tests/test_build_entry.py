"""__graft_entry__.build() must work on a clean checkout, where libfa.so does
not exist yet: it loads the two build scripts by file path, without importing
the package (whose import needs the built library)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import sys
import __graft_entry__ as g
fa = g._load_script("exact_tiled_attention_27_amd/build.py", "_fa_build")
orc = g._load_script("oracle/build.py", "_oracle_build")
assert callable(fa.build) and callable(orc.build)
assert fa.LIB.endswith("libfa.so") and orc.LIB.endswith("liboracle.so")
assert "exact_tiled_attention_27_amd" not in sys.modules
assert "oracle" not in sys.modules
print("ok")
"""


def test_build_scripts_load_without_the_package():
    r = subprocess.run([sys.executable, "-c", PROBE], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("ok")
