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


def head_block_floor(q, k, v, dout, scale, causal, groups, n0, ref, chunk=4096):
    """bf16-operand floor of the head block of a backward: dQ for rows
    0 .. n0-1 and dK, dV for keys 0 .. n0-1 of the listed key/value groups.

    `ref` is the oracle's head block with stats=True: its exact dq, dk, dv
    and the per-row LSE_i and D_i of rows s0 .. s1-1 (every row that sees
    one of the block's keys).  P_ij = exp(s_ij - LSE_i) and
    dS_ij = P_ij (dP_ij - D_i) are formed here in float64 (numpy, rows in
    chunks), rounded to bf16, and summed as the kernels' products use them:
    dV_j = sum bf16(P_ij) dO_i, dK_j = scale sum bf16(dS_ij) q_i,
    dQ_i = scale sum_j bf16(dS_ij) k_j.  Returns ({name: emulated}, {name:
    floor = max |emulated - exact|})."""
    qf, kf, vf, df = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, N, d = qf.shape
    Hkv = kf.shape[1]
    grp = Hq // Hkv
    sc = float(np.float32(scale))
    s0, s1 = ref["stat_rows"]
    assert s0 == 0, "head block: the statistics start at row 0"
    G = len(groups)
    emu = {"dq": np.zeros((G, grp, n0, d)), "dk": np.zeros((G, n0, d)),
           "dv": np.zeros((G, n0, d))}

    def p_ds(b, g, h, t, hl, r0, r1, k1):
        """P and dS of rows r0 .. r1-1 against keys 0 .. k1-1 (float64)."""
        i = np.arange(r0, r1)[:, None]
        jj = np.arange(k1)[None, :]
        s = sc * qf[b, h, r0:r1] @ kf[b, g, :k1].T
        keep = (jj <= i) if causal else np.ones((r1 - r0, k1), bool)
        lse = ref["stat_lse"][t, hl, r0 - s0:r1 - s0, None]
        D = ref["stat_D"][t, hl, r0 - s0:r1 - s0, None]
        p = np.where(keep, np.exp(s - lse), 0.0)
        return p, p * (df[b, h, r0:r1] @ vf[b, g, :k1].T - D)

    for t, gflat in enumerate(groups):
        b, g = divmod(int(gflat), Hkv)
        for hl in range(grp):
            h = g * grp + hl
            # dK, dV of keys 0 .. n0-1: every row that sees them
            for c0 in range(s0, s1, chunk):
                c1 = min(s1, c0 + chunk)
                p, ds = p_ds(b, g, h, t, hl, c0, c1, n0)
                emu["dv"][t] += _bf16(p).T @ df[b, h, c0:c1]
                emu["dk"][t] += sc * _bf16(ds).T @ qf[b, h, c0:c1]
            # dQ of rows 0 .. n0-1: all of their keys
            _, ds = p_ds(b, g, h, t, hl, 0, n0, n0 if causal else N)
            emu["dq"][t, hl] = sc * _bf16(ds) @ kf[b, g, :ds.shape[1]]
    floors = {n: float(np.abs(emu[n] - ref[n]).max()) for n in emu}
    return emu, floors
