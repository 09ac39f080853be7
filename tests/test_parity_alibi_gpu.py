"""GPU parity of the linear position bias entry points (fa_fwd_alibi,
fa_bwd_alibi) against the fp64 oracle with the same slopes, through the C ABI.

Same guard zones and NaN poisoning as the plain parity tests.  O and LSE
keep the plain bars.  The ragged backward sweep runs end to end: fa_fwd_alibi
then fa_bwd_alibi on the forward's own O and LSE.  Gradients are held to the
floor-aware max-abs bar of the plain tests, max(1e-2, 1.25 x the floor of
rounding exactly P and dS to bf16; tests/bf16_floor.py, which takes the
bias), and the plain mean-abs bar.  A strong bias makes the softmax nearly
one-hot, so dS is a small difference P (dP - D) and the bf16 operands alone
move dK and dQ by about 1e-2.  The bias backward takes D_i = sum_j P_ij dP_ij
from its own recomputed P (not sum_c dO_ic O_ic from the forward's O, whose
P V product weighs V with bf16 P): with dO . O in a one-hot row, the forward's
rounding of the dominant P entered every dS of the row undamped and put dK
and dQ at up to 2.4 x the floor.  A second sweep feeds the oracle's O and LSE
(rounded to fp32) instead, isolating the backward.
Slopes: per query head from U[-0.6, 0.9) (negative slopes favour distant
keys) for the ragged sweeps, causal and not; the geometric ALiBi sequence
2^(-8 (h + 1) / Hq) for the long causal case.
"""
import math

import numpy as np
import pytest

import oracle
from synth import random_bf16
from bf16_floor import backward_bars
from test_parity_gpu import (MEAN_ABS, MEAN_ABS_FEW_TERMS, Guarded, check_ordered_counters,
                             compare, compare_lse, dev, note)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_27_amd as m
    return m


def sweep_slopes(Hq, seed):
    return np.random.default_rng(seed).uniform(-0.6, 0.9, Hq)


def alibi_slopes(Hq):
    return np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)])


def dev_slopes(a):
    # fp32 on the device; the oracle gets the same fp32 values widened
    a32 = np.asarray(a, np.float32)
    return torch.from_numpy(a32.copy()).cuda(), a32.astype(np.float64)


def gpu_fwd_alibi(fa, q, k, v, slopes_t, scale, causal):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o, lse = Guarded((B, Hq, N, d)), Guarded((B, Hq, N))
    st = fa.fa_fwd_alibi(dev(q), dev(k), dev(v), o.t, lse.t, slopes_t, B, Hq, Hkv, N, d, scale,
                         causal)
    assert st == 0, fa.fa_status_string(st)
    return o.result("o"), lse.result("lse")


def gpu_bwd_alibi(fa, q, k, v, dout, o, lse, slopes_t, scale, causal, mode):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = Guarded((B, Hq, N, d)), Guarded((B, Hkv, N, d)), Guarded((B, Hkv, N, d))
    need = fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, mode)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    st = fa.fa_bwd_alibi(dev(q), dev(k), dev(v), torch.from_numpy(o).cuda(),
                         torch.from_numpy(lse).cuda(), dev(dout), dq.t, dk.t, dv.t, slopes_t,
                         B, Hq, Hkv, N, d, scale, causal, mode, ws, need)
    assert st == 0, fa.fa_status_string(st)
    if mode == fa.BWD_ORDERED:
        check_ordered_counters(fa, ws, B, Hq, Hkv, N, d, causal, 0)
    return dq.result("dq"), dk.result("dk"), dv.result("dv")


FWD_SWEEP = [(n, d, c) for n in (1, 3, 64, 127, 129, 300, 600) for d in (64, 128)
             for c in (False, True)]


@pytest.mark.parametrize("N,d,causal", FWD_SWEEP)
def test_alibi_fwd_small(fa, N, d, causal):
    B, Hq, Hkv = 2, 4, 2
    note(f"alibi fwd B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = (random_bf16((B, Hq, N, d), 3 * N), random_bf16((B, Hkv, N, d), 3 * N + 1),
               random_bf16((B, Hkv, N, d), 3 * N + 2))
    st, a = dev_slopes(sweep_slopes(Hq, N))
    scale = 1 / math.sqrt(d)
    o, lse = gpu_fwd_alibi(fa, q, k, v, st, scale, causal)
    o_ref, lse_ref = oracle.fwd(q, k, v, scale, causal, slopes=a)
    compare("o", o, o_ref)
    compare_lse(lse, lse_ref)


BWD_SWEEP = [(n, d, c) for n in (1, 3, 64, 129, 300, 600) for d in (64, 128) for c in (False, True)]


def check_alibi_grads(got, ref, bars, floors, mean_bar):
    for name, g in zip(("dq", "dk", "dv"), got):
        err = np.abs(g.astype(np.float64) - ref[name])
        mx, mean = float(err.max()), float(err.mean())
        note(f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e} (bf16-operand floor "
             f"{floors[name]:.3e}, bar {bars[name]:.3e}; flat 1e-2 bar "
             f"{'met' if mx <= 1e-2 else 'MISSED'})")
        assert mx <= bars[name] and mean <= mean_bar, name


def alibi_bwd_case(N, d, causal):
    B, Hq, Hkv = 2, 4, 2
    q, k, v, do = (random_bf16((B, Hq, N, d), 5 * N), random_bf16((B, Hkv, N, d), 5 * N + 1),
                   random_bf16((B, Hkv, N, d), 5 * N + 2), random_bf16((B, Hq, N, d), 5 * N + 3))
    return q, k, v, do, sweep_slopes(Hq, N + 7), 1 / math.sqrt(d)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("N,d,causal", BWD_SWEEP)
def test_alibi_bwd_small(fa, N, d, causal, mode):
    """End to end: fa_fwd_alibi, then fa_bwd_alibi on its O and LSE."""
    q, k, v, do, slopes, scale = alibi_bwd_case(N, d, causal)
    note(f"alibi fwd+bwd N={N} d={d} causal={causal} mode={mode}")
    st, a = dev_slopes(slopes)
    o, lse = gpu_fwd_alibi(fa, q, k, v, st, scale, causal)
    got = gpu_bwd_alibi(fa, q, k, v, do, o, lse, st, scale, causal, mode)
    ref = oracle.bwd(q, k, v, do, scale, causal, slopes=a)
    bars, floors = backward_bars(q, k, v, do, scale, causal, ref, slopes=a)
    check_alibi_grads(got, ref, bars, floors, MEAN_ABS_FEW_TERMS if N < 64 else MEAN_ABS)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("N,d,causal", BWD_SWEEP)
def test_alibi_bwd_small_isolated(fa, N, d, causal, mode):
    """The backward alone: fa_bwd_alibi on the oracle's O and LSE (fp32)."""
    q, k, v, do, slopes, scale = alibi_bwd_case(N, d, causal)
    note(f"alibi bwd (oracle O, LSE) N={N} d={d} causal={causal} mode={mode}")
    st, a = dev_slopes(slopes)
    ref = oracle.bwd(q, k, v, do, scale, causal, slopes=a)
    o32, lse32 = ref["o"].astype(np.float32), ref["lse"].astype(np.float32)
    got = gpu_bwd_alibi(fa, q, k, v, do, o32, lse32, st, scale, causal, mode)
    bars, floors = backward_bars(q, k, v, do, scale, causal, ref, slopes=a)
    check_alibi_grads(got, ref, bars, floors, MEAN_ABS_FEW_TERMS if N < 64 else MEAN_ABS)


def test_alibi_long_causal(fa):
    """B1 Hq8 Hkv2 N8192 d128, causal, geometric slopes: every element of the
    forward; the backward on the head block (rows and keys 0 .. 255, whose
    gradients sum over every later row) and the causal tail block (rows and
    keys N-256 .. N-1) of both KV groups, in every dQ mode, end to end."""
    B, Hq, Hkv, N, d = 1, 8, 2, 8192, 128
    note(f"alibi long B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal")
    q, k, v, do = (random_bf16((B, Hq, N, d), 71), random_bf16((B, Hkv, N, d), 72),
                   random_bf16((B, Hkv, N, d), 73), random_bf16((B, Hq, N, d), 74))
    st, a = dev_slopes(alibi_slopes(Hq))
    scale = 1 / math.sqrt(d)
    o, lse = gpu_fwd_alibi(fa, q, k, v, st, scale, True)
    o_ref, lse_ref = oracle.fwd(q, k, v, scale, True, slopes=a)
    compare("o", o, o_ref)
    compare_lse(lse, lse_ref)
    row0 = N - 256
    groups = np.arange(B * Hkv)
    tail = oracle.bwd_groups_tail(q, k, v, do, scale, row0, groups, slopes=a)
    head = oracle.bwd_groups_head(q, k, v, do, scale, True, 256, groups, slopes=a)
    grp = Hq // Hkv
    for mode in (0, 1, 2, 3):
        note(f"  dQ mode {mode}")
        dq, dk, dv = gpu_bwd_alibi(fa, q, k, v, do, o, lse, st, scale, True, mode)
        dq, dk, dv = dq.reshape(Hkv, grp, N, d), dk.reshape(Hkv, N, d), dv.reshape(Hkv, N, d)
        compare("dq (tail)", dq[:, :, row0:], tail["dq"])
        compare("dk (tail)", dk[:, row0:], tail["dk"])
        compare("dv (tail)", dv[:, row0:], tail["dv"])
        compare("dq (head)", dq[:, :, :256], head["dq"])
        compare("dk (head)", dk[:, :256], head["dk"])
        compare("dv (head)", dv[:, :256], head["dv"])


def test_alibi_zero_slopes_match_plain_kernels(fa):
    """Zero slopes add exactly zero to every raw score: forward outputs bit
    for bit equal to fa_fwd.  The bias backward forms D_i from its own P and
    dP instead of dO . O, so its dQ and dK equal fa_bwd's up to rounding (dV
    bit for bit) and both match the oracle, under the floor-aware max-abs
    bar: on this causal GQA input rounding P alone moves dV by about 1e-2."""
    B, Hq, Hkv, N, d = 1, 4, 2, 777, 128
    note(f"alibi zero slopes B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}")
    q, k, v, do = (random_bf16((B, Hq, N, d), 81), random_bf16((B, Hkv, N, d), 82),
                   random_bf16((B, Hkv, N, d), 83), random_bf16((B, Hq, N, d), 84))
    st, _ = dev_slopes(np.zeros(Hq))
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        o_b, lse_b = gpu_fwd_alibi(fa, q, k, v, st, scale, causal)
        o_p, lse_p = fa.attention_fwd(dev(q), dev(k), dev(v), scale=scale, causal=causal)
        assert np.array_equal(o_b, o_p.cpu().numpy()) and np.array_equal(lse_b, lse_p.cpu().numpy())
        g_b = gpu_bwd_alibi(fa, q, k, v, do, o_b, lse_b, st, scale, causal, 1)
        g_p = fa.attention_bwd(dev(q), dev(k), dev(v), torch.from_numpy(o_b).cuda(),
                               torch.from_numpy(lse_b).cuda(), dev(do), scale=scale,
                               causal=causal, deterministic=True)
        ref = oracle.bwd(q, k, v, do, scale, causal)
        bars, floors = backward_bars(q, k, v, do, scale, causal, ref)
        note(f"  bf16-operand floors {floors}")
        for name, x, y in zip(("dq", "dk", "dv"), g_b, g_p):
            compare(name + " (bias path)", x, ref[name], max_bar=bars[name])
            compare(name + " (plain path)", y.cpu().numpy(), ref[name], max_bar=bars[name])
            if name == "dv":  # dV does not involve D: same kernels, same bits
                assert np.array_equal(x, y.cpu().numpy())
