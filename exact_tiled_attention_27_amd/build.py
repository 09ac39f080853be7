"""Build libfa.so (the gfx950 attention library) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  The
sources compile to objects in parallel, then link into one shared library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
DEBUG_LIB = os.path.join(PKG, "libfa_debug.so")  # the same sources with event counters
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJDIR = os.path.join(ROOT, "_build")

FLAGS = ["--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]

# hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
_NOISE = ("unknown target feature", "packed-fp32-ops")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and not any(n in ln for n in _NOISE)]
    return res.returncode, msgs


def build(verbose: bool = False, extra=(), out: str = LIB, tag: str = "") -> str:
    """Compile every source (with `extra` flags) and link `out`."""
    os.makedirs(OBJDIR, exist_ok=True)
    objs, cmds = [], []
    for s in SOURCES:
        obj = os.path.join(OBJDIR, f"{os.path.splitext(s)[0]}{tag}.o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, msgs) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
    tmp = out + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> None:
    """libfa.so and the debug-counter build libfa_debug.so, side by side."""
    with ThreadPoolExecutor(max_workers=2) as ex:
        jobs = [ex.submit(build, verbose),
                ex.submit(build, verbose, ("-DFA_DEBUG_COUNTERS=1",), DEBUG_LIB, "_dbg")]
        for j in jobs:
            j.result()


if __name__ == "__main__":
    if len(sys.argv) > 1:
        print(build(verbose=True, extra=sys.argv[1:]))
    else:
        build_all(verbose=True)
