"""fp64 CPU oracle for exact scaled-dot-product attention (forward + backward).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the GPU library or its Python binding.

The arithmetic lives in attn_oracle.c (plain C, double precision, sequential
sums); this module only marshals numpy arrays through ctypes.  Definitions
follow the FlashAttention-4 pages: the three per-tile phases in "The
Asymmetric Hardware Scaling Wall" (S = QK^T/sqrt(d), P = exp(S - m)/l,
O = PV) and the simulator's validation harness, which equates the tiled result
with softmax(QK^T * scale) V; the causal mask keeps key j for query i iff
j <= i (the simulator's in-tile causal mask), and a causal sliding window of
W keys (window=W > 0) keeps max(0, i - W + 1) <= j <= i.  With slopes (one
per query head, float64 [Hq]) every score gets the linear position bias
slopes[h] * (j - i) added after the scale (the ALiBi form of an additive score
modification).  The backward is the analytic gradient of that definition (the
pages give no backward formulas).

Inputs are bf16 bit patterns held in numpy uint16 arrays, laid out
[B, H, N, d].  Outputs are float64.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    c_int, c_float, c_i64 = ctypes.c_int, ctypes.c_float, ctypes.c_int64
    lib.oracle_fwd_rows.argtypes = [u16p, u16p, u16p, c_int, c_int, c_int, c_int, c_int,
                                    c_float, c_int, c_int, f64p, i64p, c_i64, f64p, f64p, c_int]
    lib.oracle_fwd_rows.restype = c_int
    lib.oracle_bwd_block.argtypes = [u16p, u16p, u16p, u16p, c_int, c_int, c_int, c_int, c_int,
                                     c_float, c_int, c_int, f64p, c_int, c_int, c_int, c_int,
                                     i64p, c_i64, f64p, f64p, f64p, f64p, f64p, f64p, f64p,
                                     ctypes.POINTER(c_int), c_int]
    lib.oracle_bwd_block.restype = c_int
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses: the cores this process may run on (capped by
    OMP_NUM_THREADS when that is set)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _u16(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold bf16 bit patterns as uint16, got {a.dtype}")
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _shape(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, N, d


def _slopes(slopes, Hq):
    if slopes is None:
        return None, None
    a = np.ascontiguousarray(slopes, dtype=np.float64)
    if a.shape != (Hq,):
        raise ValueError(f"slopes must have shape ({Hq},), got {a.shape}")
    return a, _ptr(a, ctypes.c_double)


def fwd(q, k, v, scale, causal, threads=None, window=0, slopes=None):
    """Exact attention forward.  Returns (O [B,Hq,N,d] f64, LSE [B,Hq,N] f64)."""
    B, Hq, N, d = q.shape
    o, lse = fwd_rows(q, k, v, scale, causal, np.arange(B * Hq * N), threads, window, slopes)
    return o.reshape(B, Hq, N, d), lse.reshape(B, Hq, N)


def fwd_rows(q, k, v, scale, causal, rows, threads=None, window=0, slopes=None):
    """Forward for selected query rows.  rows: flat indices (b*Hq + h)*N + i.
    Returns (O [n, d] f64, LSE [n] f64)."""
    lib = _load()
    q, k, v = _u16(q, "q"), _u16(k, "k"), _u16(v, "v")
    B, Hq, Hkv, N, d = _shape(q, k, v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, d), np.float64)
    lse = np.empty((rows.size,), np.float64)
    keep, sp = _slopes(slopes, Hq)
    st = lib.oracle_fwd_rows(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                             _ptr(v, ctypes.c_uint16), B, Hq, Hkv, N, d, float(scale),
                             int(bool(causal)), int(window), sp, _ptr(rows, ctypes.c_int64),
                             rows.size, _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                             threads or default_threads())
    if st:
        raise RuntimeError(f"oracle_fwd_rows failed with status {st}")
    return o, lse


def fwd_heads(q, k, v, scale, causal, heads, threads=None, window=0, slopes=None):
    """Forward for whole heads.  heads: flat indices b*Hq + h.
    Returns (O [n, N, d] f64, LSE [n, N] f64)."""
    N = q.shape[2]
    heads = np.asarray(heads, dtype=np.int64)
    rows = (heads[:, None] * N + np.arange(N, dtype=np.int64)[None, :]).reshape(-1)
    o, lse = fwd_rows(q, k, v, scale, causal, rows, threads, window, slopes)
    return o.reshape(heads.size, N, q.shape[3]), lse.reshape(heads.size, N)


def bwd_block(q, k, v, dout, scale, causal, groups, rows, keys, threads=None, window=0,
              slopes=None, stats=False):
    """Backward of the selected key/value groups (flat index b*Hkv + g),
    restricted to dQ (and O, LSE) for query rows rows[0] .. rows[1]-1 of each
    of the group's heads and dK, dV for keys keys[0] .. keys[1]-1.  Each
    entry equals the same slice of the whole backward, bit for bit.

    Returns dict with dq [G, Hq/Hkv, R, d], dk [G, K, d], dv [G, K, d],
    o [G, Hq/Hkv, R, d], lse [G, Hq/Hkv, R], all float64.  With stats=True
    also stat_rows (s0, s1), stat_lse and stat_D [G, Hq/Hkv, s1 - s0]: LSE_i
    and D_i = sum_c dO_ic O_ic of every row the block needed."""
    lib = _load()
    q, k, v, dout = _u16(q, "q"), _u16(k, "k"), _u16(v, "v"), _u16(dout, "dout")
    B, Hq, Hkv, N, d = _shape(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    r0, r1 = int(rows[0]), int(rows[1])
    k0, k1 = int(keys[0]), int(keys[1])
    groups = np.ascontiguousarray(groups, dtype=np.int64)
    G, grp, R, K = groups.size, Hq // Hkv, r1 - r0, k1 - k0
    out = {
        "dq": np.empty((G, grp, R, d), np.float64),
        "dk": np.empty((G, K, d), np.float64),
        "dv": np.empty((G, K, d), np.float64),
        "o": np.empty((G, grp, R, d), np.float64),
        "lse": np.empty((G, grp, R), np.float64),
    }
    keep, sp = _slopes(slopes, Hq)
    srange = np.zeros(2, np.int32)
    stat_lse = stat_D = None
    if stats:
        # the widest the stat rows can be; trimmed once the range is known
        stat_lse = np.empty((G, grp, N), np.float64)
        stat_D = np.empty((G, grp, N), np.float64)
    st = lib.oracle_bwd_block(
        _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
        _ptr(dout, ctypes.c_uint16), B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
        int(window), sp, r0, r1, k0, k1, _ptr(groups, ctypes.c_int64), G,
        _ptr(out["dq"], ctypes.c_double), _ptr(out["dk"], ctypes.c_double),
        _ptr(out["dv"], ctypes.c_double), _ptr(out["o"], ctypes.c_double),
        _ptr(out["lse"], ctypes.c_double),
        _ptr(stat_lse, ctypes.c_double) if stats else None,
        _ptr(stat_D, ctypes.c_double) if stats else None,
        _ptr(srange, ctypes.c_int), threads or default_threads())
    if st:
        raise RuntimeError(f"oracle_bwd_block failed with status {st}")
    if stats:
        s0, s1 = int(srange[0]), int(srange[1])
        ns = s1 - s0
        # the C side wrote [G, grp, ns] contiguously at the start of each buffer
        out["stat_rows"] = (s0, s1)
        out["stat_lse"] = stat_lse.reshape(-1)[:G * grp * ns].reshape(G, grp, ns).copy()
        out["stat_D"] = stat_D.reshape(-1)[:G * grp * ns].reshape(G, grp, ns).copy()
    return out


def bwd_groups(q, k, v, dout, scale, causal, groups, threads=None, window=0, slopes=None):
    """Backward for selected key/value groups (flat index b*Hkv + g).

    Returns dict with dq [G, Hq/Hkv, N, d], dk [G, N, d], dv [G, N, d],
    o [G, Hq/Hkv, N, d], lse [G, Hq/Hkv, N], all float64."""
    N = q.shape[2]
    return bwd_block(q, k, v, dout, scale, causal, groups, (0, N), (0, N), threads, window,
                     slopes)


def bwd_groups_tail(q, k, v, dout, scale, row0, groups, threads=None, window=0, slopes=None):
    """Causal backward restricted to rows and keys row0 .. N-1 of the selected
    groups (a key there only receives gradient from later rows, whose forward
    statistics still run over all their keys).

    Returns dict with dq [G, Hq/Hkv, N-row0, d], dk [G, N-row0, d],
    dv [G, N-row0, d], o [G, Hq/Hkv, N-row0, d], lse [G, Hq/Hkv, N-row0]."""
    N = q.shape[2]
    return bwd_block(q, k, v, dout, scale, True, groups, (row0, N), (row0, N), threads, window,
                     slopes)


def bwd_groups_head(q, k, v, dout, scale, causal, n0, groups, threads=None, window=0,
                    slopes=None, stats=False):
    """Backward restricted to rows and keys 0 .. n0-1 of the selected groups:
    the first keys, whose gradients sum over every later row (the forward
    statistics of all those rows are computed).

    Returns dict with dq [G, Hq/Hkv, n0, d], dk [G, n0, d], dv [G, n0, d],
    o [G, Hq/Hkv, n0, d], lse [G, Hq/Hkv, n0]."""
    return bwd_block(q, k, v, dout, scale, causal, groups, (0, n0), (0, n0), threads, window,
                     slopes, stats)


def bwd(q, k, v, dout, scale, causal, threads=None, window=0, slopes=None):
    """Whole backward.  Returns dict dq [B,Hq,N,d], dk/dv [B,Hkv,N,d], o, lse."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    r = bwd_groups(q, k, v, dout, scale, causal, np.arange(B * Hkv), threads, window, slopes)
    return {
        "dq": r["dq"].reshape(B, Hq, N, d),
        "dk": r["dk"].reshape(B, Hkv, N, d),
        "dv": r["dv"].reshape(B, Hkv, N, d),
        "o": r["o"].reshape(B, Hq, N, d),
        "lse": r["lse"].reshape(B, Hq, N),
    }
