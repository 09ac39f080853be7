"""GPU parity of the linear position bias entry points (fa_fwd_alibi,
fa_bwd_alibi) against the fp64 oracle with the same slopes, through the C ABI.

Same guard zones and NaN poisoning as the plain parity tests.  O and LSE
keep the plain bars.  The ragged backward sweep isolates the backward: it
feeds the oracle's own O and LSE (rounded to fp32) to fa_bwd_alibi, so the
expected result is exactly the oracle's gradients, and holds them to the
floor-aware max-abs bar of the plain tests, max(1e-2, 1.25 x the floor of
rounding exactly P and dS to bf16; tests/bf16_floor.py, which takes the
bias), and the plain mean-abs bar.  A strong bias makes the softmax nearly
one-hot, so dS is a small difference P (dP - D) and the bf16 operands alone
move dK and dQ by about 1e-2; the backward kernels then sit at that floor.
End to end (the kernel's own O, whose bf16-weighted P V product enters
D = rowsum(dO * O)), such rows measured 1.27-1.45 x the floor; the long causal
case below runs end to end with the geometric slopes and the plain bars.
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


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,d,causal", BWD_SWEEP)
def test_alibi_bwd_small(fa, N, d, causal, mode):
    B, Hq, Hkv = 2, 4, 2
    note(f"alibi bwd B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} mode={mode}")
    q, k, v, do = (random_bf16((B, Hq, N, d), 5 * N), random_bf16((B, Hkv, N, d), 5 * N + 1),
                   random_bf16((B, Hkv, N, d), 5 * N + 2), random_bf16((B, Hq, N, d), 5 * N + 3))
    st, a = dev_slopes(sweep_slopes(Hq, N + 7))
    scale = 1 / math.sqrt(d)
    ref = oracle.bwd(q, k, v, do, scale, causal, slopes=a)
    o32, lse32 = ref["o"].astype(np.float32), ref["lse"].astype(np.float32)
    dq, dk, dv = gpu_bwd_alibi(fa, q, k, v, do, o32, lse32, st, scale, causal, mode)
    mean_bar = MEAN_ABS_FEW_TERMS if N < 64 else MEAN_ABS
    bars, floors = backward_bars(q, k, v, do, scale, causal, ref, slopes=a)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        err = np.abs(got.astype(np.float64) - ref[name])
        mx, mean = float(err.max()), float(err.mean())
        note(f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e} (bf16-operand floor "
             f"{floors[name]:.3e}, bar {bars[name]:.3e})")
        assert mx <= bars[name] and mean <= mean_bar, name


def test_alibi_long_causal(fa):
    """B1 Hq8 Hkv2 N8192 d128, causal, geometric slopes: forward on sampled
    rows (tile edges and random rows), backward on the causal tail block of
    both KV groups (rows and keys N-256 .. N-1, exact there) in every dQ mode."""
    B, Hq, Hkv, N, d = 1, 8, 2, 8192, 128
    note(f"alibi long B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal")
    q, k, v, do = (random_bf16((B, Hq, N, d), 71), random_bf16((B, Hkv, N, d), 72),
                   random_bf16((B, Hkv, N, d), 73), random_bf16((B, Hq, N, d), 74))
    st, a = dev_slopes(alibi_slopes(Hq))
    scale = 1 / math.sqrt(d)
    o, lse = gpu_fwd_alibi(fa, q, k, v, st, scale, True)
    rng = np.random.default_rng(75)
    edges = [0, 1, 63, 64, 255, 256, 4095, 4096, N - 1]
    rows = np.unique(np.concatenate([
        [(h * N + i) for h in range(Hq) for i in edges], rng.integers(0, Hq * N, 200)]))
    o_ref, lse_ref = oracle.fwd_rows(q, k, v, scale, True, rows, slopes=a)
    compare("o (sampled rows)", o.reshape(-1, d)[rows], o_ref)
    compare_lse(lse.reshape(-1)[rows], lse_ref)
    row0 = N - 256
    ref = oracle.bwd_groups_tail(q, k, v, do, scale, row0, np.arange(B * Hkv), slopes=a)
    grp = Hq // Hkv
    for mode in (0, 1, 2):
        note(f"  dQ mode {mode}")
        dq, dk, dv = gpu_bwd_alibi(fa, q, k, v, do, o, lse, st, scale, True, mode)
        compare("dq (tail)", dq.reshape(Hkv, grp, N, d)[:, :, row0:], ref["dq"])
        compare("dk (tail)", dk.reshape(Hkv, N, d)[:, row0:], ref["dk"])
        compare("dv (tail)", dv.reshape(Hkv, N, d)[:, row0:], ref["dv"])


def test_alibi_zero_slopes_equal_plain_kernels(fa):
    """Zero slopes add exactly zero to every raw score: outputs bit for bit
    equal to fa_fwd / fa_bwd (deterministic mode)."""
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
        for x, y in zip(g_b, g_p):
            assert np.array_equal(x, y.cpu().numpy())
