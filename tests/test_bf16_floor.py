"""The bf16-operand floor emulation (tests/bf16_floor.py), pinned on the CPU:
without rounding it reproduces the oracle's gradients, and on the causal GQA
input of the smoke check the rounding of P alone already moves dV by more than
the 1e-2 bar (the case the floor-aware bar exists for)."""
import math

import numpy as np
import pytest

import oracle
from bf16_floor import backward_bars, backward_emulation
from synth import random_bf16


def test_unrounded_emulation_is_the_oracle():
    B, Hq, Hkv, N, d = 1, 4, 2, 37, 32
    q, k, v = random_bf16((B, Hq, N, d), 51), random_bf16((B, Hkv, N, d), 52), random_bf16((B, Hkv, N, d), 53)
    do = random_bf16((B, Hq, N, d), 54)
    for causal, window in ((False, 0), (True, 0), (True, 9)):
        ref = oracle.bwd(q, k, v, do, 0.2, causal, window=window)
        emu = backward_emulation(q, k, v, do, 0.2, causal, window, round_operands=False)
        for name in ("dq", "dk", "dv"):
            np.testing.assert_allclose(emu[name], ref[name], rtol=1e-10, atol=1e-12)


def test_floor_exceeds_bar_on_the_smoke_input():
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v = random_bf16((B, Hq, N, d), 1), random_bf16((B, Hkv, N, d), 2), random_bf16((B, Hkv, N, d), 3)
    do = random_bf16((B, Hq, N, d), 4)
    ref = oracle.bwd(q, k, v, do, scale, True)
    bars, floors = backward_bars(q, k, v, do, scale, True, ref)
    assert floors["dv"] > 1e-2 and bars["dv"] == 1.25 * floors["dv"]
    assert floors["dk"] < 1e-2 and bars["dk"] == 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_emulation_with_bias_equals_oracle_without_rounding(causal):
    """The floor's emulation with the linear position bias, rounding off,
    reproduces the oracle's biased gradients (numpy vs the C oracle)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 40, 16
    q, k, v, do = (random_bf16((B, Hq, N, d), 31), random_bf16((B, Hkv, N, d), 32),
                   random_bf16((B, Hkv, N, d), 33), random_bf16((B, Hq, N, d), 34))
    a = np.array([0.5, -0.4, 0.1, 0.9])
    ref = oracle.bwd(q, k, v, do, 0.25, causal, slopes=a)
    emu = backward_emulation(q, k, v, do, 0.25, causal, round_operands=False, slopes=a)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(emu[name], ref[name], rtol=1e-9, atol=1e-11)


def test_head_block_floor_without_rounding_is_the_oracle(monkeypatch):
    """The head-block emulation with the bf16 rounding switched off equals the
    oracle's head block (its P, dS and sums are the same mathematics in
    numpy), causal and not, GQA 2:1; with rounding its floor is nonzero."""
    import bf16_floor
    B, Hq, Hkv, N, d, n0 = 1, 4, 2, 150, 16, 40
    q, k, v = random_bf16((B, Hq, N, d), 31), random_bf16((B, Hkv, N, d), 32), random_bf16((B, Hkv, N, d), 33)
    do = random_bf16((B, Hq, N, d), 34)
    for causal in (True, False):
        ref = oracle.bwd_groups_head(q, k, v, do, 0.25, causal, n0, [0, 1], stats=True)
        _, floors = bf16_floor.head_block_floor(q, k, v, do, 0.25, causal, [0, 1], n0, ref,
                                                chunk=64)
        assert all(f > 1e-5 for f in floors.values()), floors
        monkeypatch.setattr(bf16_floor, "_bf16", lambda x: np.asarray(x, np.float64))
        emu, floors = bf16_floor.head_block_floor(q, k, v, do, 0.25, causal, [0, 1], n0, ref,
                                                  chunk=64)
        monkeypatch.undo()
        assert all(f < 1e-12 for f in floors.values()), floors
