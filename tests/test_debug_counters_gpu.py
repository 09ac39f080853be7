"""The debug-counter build (libfa_debug.so): its forward gives the same bits
as libfa.so, and its counts of rescale decisions, rescales taken, key tiles
walked and masked tiles equal the counts derived by hand for the planted-jump
input (scores 0 before key 160, `jump` from key 160 on; N = 320, two heads,
64-key tiles, 256-row query tiles)."""
import math

import numpy as np
import pytest

from test_parity_gpu import Guarded, dev, gpu_fwd, note, planted_jump_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_27_amd as m
    return m


@pytest.fixture(scope="module")
def dbg(fa):
    from exact_tiled_attention_27_amd import debug
    return debug


def expected(N, H, causal, jump, tau=8.0):
    """Hand count: every row walks its workgroup's key tiles; a decision is
    each tile after the row's first (here tile 0 for every row, since key 0
    is valid for all of them), masked tiles included; the reference moves
    once, at the tile holding key 160, for rows that see key 160, when the
    jump exceeds tau."""
    tiles = masked = decisions = rescales = wgs = 0
    for q0 in range(0, N, 256):
        wgs += 1
        rows = range(q0, min(q0 + 256, N))
        n_tiles = math.ceil(min(q0 + 256, N) / 64) if causal else math.ceil(N / 64)
        n_full = min(n_tiles, min(N // 64, (q0 + 1) // 64)) if causal else N // 64
        tiles += n_tiles
        masked += sum(1 for t in range(n_tiles) if t >= n_full)
        for i in rows:
            decisions += n_tiles - 1
            sees_jump = (i >= 160) if causal else True
            rescales += int(sees_jump and jump > tau)
    return {"row_decisions": H * decisions, "row_rescales": H * rescales, "tiles": H * tiles,
            "masked_tiles": H * masked, "workgroups": H * wgs}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jump", [7.875, 8.125, 40.0])
def test_counters_on_planted_jump(fa, dbg, causal, jump):
    q, k, v, scale = planted_jump_inputs(jump)
    B, H, N, d = q.shape
    note(f"debug counters: jump {jump} causal={causal}")
    dbg.fa_debug_counters()  # clear
    o, lse = Guarded((B, H, N, d)), Guarded((B, H, N))
    st = dbg.fa_fwd(dev(q), dev(k), dev(v), o.t, lse.t, B, H, H, N, d, scale, causal)
    assert st == 0, fa.fa_status_string(st)
    got_o = o.result("o")
    c = dbg.fa_debug_counters()
    note(f"  counters {c}")
    want = expected(N, H, causal, jump)
    for key, val in want.items():
        assert c[key] == val, (key, c[key], val)
    assert (c["wave_rescales"] == 0) == (c["row_rescales"] == 0)
    assert c["wave_rescales"] <= c["row_rescales"]
    # The counters do not change the arithmetic: same bits as libfa.so.
    ref_o, _ = gpu_fwd(fa, q, k, v, scale, causal)
    assert np.array_equal(got_o.view(np.uint32), ref_o.view(np.uint32))


@pytest.mark.parametrize("name", ["fwd_causal_rowscale_n8192", "fwd_n4096"])
def test_rescale_rate_on_workloads(fa, dbg, name):
    """How often the reference maximum moves after a row's first tile, on the
    row-scaled causal workload (each query row scaled by its own factor, so
    the running maximum jumps mid-row) and on the iid non-causal one.  The
    counts are printed for the record; the test checks that rescales happen
    on the row-scaled workload, and rarely."""
    from synth import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    x = make_inputs(w)
    o, lse = Guarded((w.B, w.Hq, w.N, w.d)), Guarded((w.B, w.Hq, w.N))
    dbg.fa_debug_counters()
    st = dbg.fa_fwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), o.t, lse.t, w.B, w.Hq, w.Hkv, w.N,
                    w.d, w.scale, w.causal)
    assert st == 0, fa.fa_status_string(st)
    o.result("o")
    c = dbg.fa_debug_counters()
    wave_decisions = c["row_decisions"] / 32.0
    note(f"rescale rate {name}: {c}; rows moved per decision "
         f"{c['row_rescales'] / c['row_decisions']:.4%}, waves rescaling per wave-tile "
         f"{c['wave_rescales'] / wave_decisions:.4%}, masked tiles "
         f"{c['masked_tiles'] / c['tiles']:.2%} of {c['tiles']}")
    assert c["workgroups"] == w.B * w.Hq * math.ceil(w.N / 256)
    if w.row_scale:
        assert 0 < c["row_rescales"] < 0.05 * c["row_decisions"]


def test_dq_atomic_pattern_rate(fa, dbg):
    """The backward's dQ atomic pattern alone (fa_debug_atomic_tiles): every
    add lands exactly once (the buffer sums to the count of adds), and the
    device's rate for it is printed: the atomic dK/dV kernel's adds per
    second are compared against it in the design notes."""
    n_slots, tiles = 4096, 64
    buf = torch.zeros(n_slots * 64 * 128, dtype=torch.float32, device="cuda")
    for blocks in (1024, 4096):
        buf.zero_()
        st = dbg.fa_debug_atomic_tiles(buf, n_slots, tiles, blocks)
        assert st == 0
        torch.cuda.synchronize()
        total = float(buf.double().sum())
        assert total == blocks * tiles * 64 * 128
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            assert dbg.fa_debug_atomic_tiles(buf, n_slots, tiles, blocks) == 0
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        lanes = blocks * tiles * 64 * 128
        note(f"dQ atomic pattern: {blocks} workgroups x {tiles} tiles: {ms:.3f} ms, "
             f"{lanes / ms / 1e6:.1f} G fp32 adds/s, {lanes / 16 / ms / 1e6:.2f} G 64-byte "
             f"requests/s")
