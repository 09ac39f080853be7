"""Build libfa.so (the gfx950 attention library) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
    noise = ("unknown target feature", "packed-fp32-ops")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
