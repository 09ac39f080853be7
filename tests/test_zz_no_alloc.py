"""fa_bwd_noalloc (the backward whose workspace lives in the library's static
device array) against fa_bwd with a caller workspace, through the C ABI, on
two calls in a row, the second with a smaller input.  The reproducible dQ
modes must give the same bits as fa_bwd (same kernels, same workspace
layout); the atomic mode the same dK and dV bits and dQ within 1e-5.  Both
calls are also held to the oracle's bars (max-abs floor-aware, as for every
causal GQA input where rounding P to bf16 alone nears 1e-2)."""
import math

import numpy as np
import pytest

import oracle
from bf16_floor import backward_bars
from synth import random_bf16
from test_parity_gpu import MEAN_ABS, Guarded, compare, dev, gpu_bwd, gpu_fwd, note

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_27_amd as m
    return m


def noalloc_bwd(fa, q, k, v, dout, o, lse, scale, causal, mode):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = Guarded((B, Hq, N, d)), Guarded((B, Hkv, N, d)), Guarded((B, Hkv, N, d))
    st = fa.fa_bwd_noalloc(dev(q), dev(k), dev(v), torch.from_numpy(o).cuda(),
                           torch.from_numpy(lse).cuda(), dev(dout), dq.t, dk.t, dv.t, B, Hq, Hkv,
                           N, d, scale, causal, mode)
    assert st == 0, fa.fa_status_string(st)
    return dq.result("dq"), dk.result("dk"), dv.result("dv")


# First a larger call, then a smaller one: the second reuses the array the
# first left behind (its D, LSE2 and, ordered mode, counters are rewritten).
SHAPES = [(2, 4, 2, 1000, 128, True, 11), (1, 2, 1, 300, 64, False, 12)]


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_noalloc_matches_workspace_call(fa, mode):
    for B, Hq, Hkv, N, d, causal, seed in SHAPES:
        note(f"noalloc mode={mode} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
        q, k, v = (random_bf16((B, Hq, N, d), seed), random_bf16((B, Hkv, N, d), seed + 1),
                   random_bf16((B, Hkv, N, d), seed + 2))
        dout = random_bf16((B, Hq, N, d), seed + 3)
        scale = 1 / math.sqrt(d)
        o, lse = gpu_fwd(fa, q, k, v, scale, causal)
        got = noalloc_bwd(fa, q, k, v, dout, o, lse, scale, causal, mode)
        want = gpu_bwd(fa, q, k, v, dout, o, lse, scale, causal, mode)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            if mode in (0, 3) and name == "dq":
                assert float(np.abs(a - b).max()) <= 1e-5, name
            else:
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
        ref = oracle.bwd(q, k, v, dout, scale, causal)
        bars, _ = backward_bars(q, k, v, dout, scale, causal, ref)
        for name, a in zip(("dq", "dk", "dv"), got):
            compare(name, a, ref[name], MEAN_ABS, max_bar=bars[name])

