"""Binding of the debug-counter build libfa_debug.so (include/fa_debug.h).

The same forward entry points as the package (fa_fwd, fa_fwd_window), served
by libfa_debug.so, whose forward kernels count rescale decisions, rescales
taken and key tiles walked; fa_debug_counters() reads and clears the counts.
fa_debug_atomic_tiles() runs the backward's dQ atomic pattern alone.
For measurement only: the counters' atomics perturb timings.  Importing this
module fails if libfa_debug.so has not been built.
"""
import ctypes
import os

import torch  # noqa: F401  (one HIP runtime in the process, as in the package)

from . import _stream, _addr

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_debug.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")

COUNTERS = ("row_decisions", "row_rescales", "wave_rescales", "tiles", "masked_tiles",
            "workgroups")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.fa_fwd.restype = _i
_lib.fa_fwd_window.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.fa_fwd_window.restype = _i
_lib.fa_debug_counters.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), _i]
_lib.fa_debug_counters.restype = _i
_lib.fa_debug_atomic_tiles.argtypes = [_vp, _i, _i, _i, _vp]
_lib.fa_debug_atomic_tiles.restype = _i


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream=None) -> int:
    """fa_fwd of the debug build.  Status out."""
    return _lib.fa_fwd(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, Hq, Hkv, N, d,
                       float(scale), int(bool(causal)), _stream(stream, q, o))


def fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, window, stream=None) -> int:
    """fa_fwd_window of the debug build.  Status out."""
    return _lib.fa_fwd_window(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), B, Hq, Hkv, N,
                              d, float(scale), int(window), _stream(stream, q, o))


def fa_debug_atomic_tiles(buf, n_slots, tiles, blocks, stream=None) -> int:
    """fa_debug_atomic_tiles: the dQ atomic pattern alone.  Status out."""
    return _lib.fa_debug_atomic_tiles(_addr(buf), int(n_slots), int(tiles), int(blocks),
                                      _stream(stream, buf))


def fa_debug_counters() -> dict:
    """Counts since the last read (then cleared), by name."""
    buf = (ctypes.c_ulonglong * len(COUNTERS))()
    st = _lib.fa_debug_counters(buf, len(COUNTERS))
    if st:
        raise RuntimeError(f"fa_debug_counters: status {st}")
    return dict(zip(COUNTERS, (int(x) for x in buf)))
