"""Representation floor of the backward's bf16 operands (test infrastructure).

The kernels round P (for dV = P^T dO) and dS (for dK = dS^T Q and dQ = dS K)
to bf16 before the matrix products, as the FlashAttention-4 pages' kernels do
for their tensor-core operands.  This module computes, in float64 with numpy
and independently of the oracle's code, what that rounding alone costs:
P and dS exact, then rounded to bf16 (round to nearest even), every other
step exact.  The largest deviation from the exact gradients is the floor no
bf16-operand kernel can beat; where it exceeds the parity bar, the bar for
that output is the floor with a 25% margin.
"""
import math

import numpy as np

from synth import bf16_bits_to_f32, f32_to_bf16_bits


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _bf16(x):
    return _f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def backward_emulation(q, k, v, dout, scale, causal, window=0, round_operands=True, slopes=None):
    """dQ, dK, dV (float64) with P and dS rounded to bf16 when round_operands.
    slopes: per-query-head linear position bias slopes[h] * (j - i), or None."""
    qf, kf, vf, df = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, N, d = qf.shape
    Hkv = kf.shape[1]
    grp = Hq // Hkv
    sc = float(np.float32(scale))
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    keep = np.ones((N, N), bool)
    if causal:
        keep &= j <= i
        if window > 0:
            keep &= j > i - window
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            s = sc * qf[b, h] @ kf[b, g].T
            if slopes is not None:
                s = s + slopes[h] * (j - i)
            s = np.where(keep, s, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            o = p @ vf[b, g]
            D = (df[b, h] * o).sum(1, keepdims=True)
            ds = p * (df[b, h] @ vf[b, g].T - D)
            if round_operands:
                p, ds = _bf16(p), _bf16(ds)
            dv[b, g] += p.T @ df[b, h]
            dk[b, g] += sc * ds.T @ qf[b, h]
            dq[b, h] = sc * ds @ kf[b, g]
    return {"dq": dq, "dk": dk, "dv": dv}


def backward_bars(q, k, v, dout, scale, causal, ref, window=0, max_abs=1e-2, slopes=None):
    """Max-abs bar per gradient: max_abs, or 1.25 x the bf16-operand floor
    (deviation of the emulation from the exact `ref`) where that is larger."""
    emu = backward_emulation(q, k, v, dout, scale, causal, window, slopes=slopes)
    bars, floors = {}, {}
    for name in ("dq", "dk", "dv"):
        floors[name] = float(np.abs(emu[name] - ref[name]).max())
        bars[name] = max(max_abs, 1.25 * floors[name])
    return bars, floors
