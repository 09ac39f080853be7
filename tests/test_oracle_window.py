"""Pins for the oracle's causal sliding window (no GPU).

A window of W keys keeps key j for query i iff i - W < j <= i.  Pinned to:
  * brute force in pure Python over the banded key set;
  * torch's scaled_dot_product_attention with an explicit boolean band mask,
    its logsumexp and its float64 autograd (independent library routines);
  * closed forms: W = 1 gives O_i = V_i and LSE_i = s_ii; W >= N is plain
    causal, bit for bit;
  * locality: changing key i - W leaves row i untouched, changing key
    i - W + 1 does not;
  * central finite differences of the gradients on a bf16-exact grid, and the
    exact identities sum_j dK_j = 0, sum_j dV_j = sum_i dO_i.
A wrong window edge (off by one on either side), a window applied to keys
after the query, or a gradient pass that ignores the window fails one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def band(N, W):
    """Boolean [N, N], True where query i may see key j (i - W < j <= i)."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    return (j <= i) & (j > i - W)


def brute_fwd_window(q, k, v, scale, W):
    qf, kf, vf = f64(q), f64(k), f64(v)
    B, Hq, N, d = qf.shape
    grp = Hq // kf.shape[1]
    o = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    sc = float(np.float32(scale))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for i in range(N):
                keys = [j for j in range(N) if i - W < j <= i]
                s = [sc * math.fsum(qf[b, h, i, c] * kf[b, g, j, c] for c in range(d)) for j in keys]
                m = max(s)
                p = [math.exp(x - m) for x in s]
                l = math.fsum(p)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(p[t] * vf[b, g, j, c] for t, j in enumerate(keys)) / l
                lse[b, h, i] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("W", [1, 2, 3, 5])
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 1, 1, 6, 3), (1, 2, 1, 9, 4), (2, 2, 2, 7, 5)])
def test_window_brute_force(B, Hq, Hkv, N, d, W):
    q, k, v = random_bf16((B, Hq, N, d), 201), random_bf16((B, Hkv, N, d), 202), random_bf16((B, Hkv, N, d), 203)
    o, lse = oracle.fwd(q, k, v, 0.4, True, window=W)
    o_ref, lse_ref = brute_fwd_window(q, k, v, 0.4, W)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-13)


def torch_window(q, k, v, scale, W, dout=None):
    qt, kt, vt = (torch.from_numpy(f64(x)).requires_grad_() for x in (q, k, v))
    grp = qt.shape[1] // kt.shape[1]
    N = qt.shape[2]
    mask = torch.from_numpy(band(N, W))
    sc = float(np.float32(scale))
    ke, ve = kt.repeat_interleave(grp, 1), vt.repeat_interleave(grp, 1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, ke, ve, attn_mask=mask, scale=sc)
    s = (qt @ ke.transpose(-1, -2)) * sc
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    grads = None
    if dout is not None:
        o.backward(torch.from_numpy(f64(dout)))
        grads = (qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy())
    return o.detach().numpy(), lse.detach().numpy(), grads


@pytest.mark.parametrize("W", [1, 7, 16, 63])
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 2, 2, 64, 32), (2, 4, 1, 37, 16)])
def test_window_vs_torch(B, Hq, Hkv, N, d, W):
    q, k, v = random_bf16((B, Hq, N, d), 211), random_bf16((B, Hkv, N, d), 212), random_bf16((B, Hkv, N, d), 213)
    dout = random_bf16((B, Hq, N, d), 214)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.fwd(q, k, v, scale, True, window=W)
    o_ref, lse_ref, (dq, dk, dv) = torch_window(q, k, v, scale, W, dout)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-11, atol=1e-12)
    r = oracle.bwd(q, k, v, dout, scale, True, window=W)
    np.testing.assert_allclose(r["dq"], dq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dk"], dk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dv"], dv, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(r["o"], o)
    rows = np.array([0, 5, N - 1, N + 3, 2 * N - 1])
    o_rows, lse_rows = oracle.fwd_rows(q, k, v, scale, True, rows, window=W)
    np.testing.assert_array_equal(o_rows, o.reshape(-1, d)[rows])
    np.testing.assert_array_equal(lse_rows, lse.reshape(-1)[rows])


def test_window_one_and_wide():
    B, Hq, Hkv, N, d = 1, 2, 1, 20, 8
    q, k, v = random_bf16((B, Hq, N, d), 221), random_bf16((B, Hkv, N, d), 222), random_bf16((B, Hkv, N, d), 223)
    o, lse = oracle.fwd(q, k, v, 0.5, True, window=1)
    np.testing.assert_array_equal(o, np.repeat(f64(v), 2, axis=1))
    s_ii = 0.5 * np.einsum("bhnc,bhnc->bhn", f64(q), np.repeat(f64(k), 2, axis=1))
    np.testing.assert_allclose(lse, s_ii, rtol=1e-15, atol=1e-15)
    oc, lc = oracle.fwd(q, k, v, 0.5, True)
    for W in (N, N + 1, 1000):
        ow, lw = oracle.fwd(q, k, v, 0.5, True, window=W)
        np.testing.assert_array_equal(ow, oc)
        np.testing.assert_array_equal(lw, lc)
    dout = random_bf16((B, Hq, N, d), 224)
    rc = oracle.bwd(q, k, v, dout, 0.5, True)
    rw = oracle.bwd(q, k, v, dout, 0.5, True, window=N)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(rw[name], rc[name])


def test_window_locality():
    B, Hq, Hkv, N, d, W = 1, 1, 1, 16, 4, 5
    q, k, v = random_bf16((B, Hq, N, d), 231), random_bf16((B, Hkv, N, d), 232), random_bf16((B, Hkv, N, d), 233)
    i = 11
    o, lse = oracle.fwd(q, k, v, 0.7, True, window=W)
    for j, same in ((i - W, True), (i - W + 1, False), (i, False), (i + 1, True)):
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, j] = random_bf16((d,), 234 + j)
        v2[0, 0, j] = random_bf16((d,), 334 + j)
        o2, l2 = oracle.fwd(q, k2, v2, 0.7, True, window=W)
        assert np.array_equal(o2[0, 0, i], o[0, 0, i]) == same, j
        assert (l2[0, 0, i] == lse[0, 0, i]) == same, j


def test_window_requires_causal():
    q = random_bf16((1, 1, 4, 4), 241)
    with pytest.raises(RuntimeError):
        oracle.fwd(q, q, q, 0.5, False, window=2)


def _grid(shape, rng):
    return (rng.integers(-32, 33, size=shape) / 32.0).astype(np.float32)


@pytest.mark.parametrize("W", [2, 4])
def test_window_finite_differences(W):
    """L = sum(dO * O), Richardson-extrapolated central differences (step
    2^-7, exact in bf16) against sum(grad * direction) for Q, K, V."""
    B, Hq, Hkv, N, d = 1, 2, 1, 9, 4
    rng = np.random.default_rng(251 + W)
    base = {"q": _grid((B, Hq, N, d), rng), "k": _grid((B, Hkv, N, d), rng), "v": _grid((B, Hkv, N, d), rng)}
    dout = f32_to_bf16_bits(_grid((B, Hq, N, d), rng))
    bits = {n: f32_to_bf16_bits(x) for n, x in base.items()}
    grads = oracle.bwd(bits["q"], bits["k"], bits["v"], dout, 0.5, True, window=W)

    def loss(arrs):
        o, _ = oracle.fwd(f32_to_bf16_bits(arrs["q"]), f32_to_bf16_bits(arrs["k"]),
                          f32_to_bf16_bits(arrs["v"]), 0.5, True, window=W)
        return float(np.sum(f64(dout) * o))

    eps = 2.0 ** -7
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        direction = rng.integers(-1, 2, size=base[name].shape).astype(np.float32)

        def central(step):
            plus, minus = dict(base), dict(base)
            plus[name] = base[name] + np.float32(step) * direction
            minus[name] = base[name] - np.float32(step) * direction
            return (loss(plus) - loss(minus)) / (2 * step)

        fd = (4 * central(eps) - central(2 * eps)) / 3
        assert fd == pytest.approx(float(np.sum(grads[gname] * direction)), rel=2e-6, abs=1e-8), name


def test_window_gradient_identities():
    B, Hq, Hkv, N, d, W = 2, 4, 2, 21, 8, 6
    q, k, v = random_bf16((B, Hq, N, d), 261), random_bf16((B, Hkv, N, d), 262), random_bf16((B, Hkv, N, d), 263)
    dout = random_bf16((B, Hq, N, d), 264)
    r = oracle.bwd(q, k, v, dout, 0.35, True, window=W)
    np.testing.assert_allclose(r["dk"].sum(2), 0.0, atol=1e-13)
    want = f64(dout).reshape(B, Hkv, Hq // Hkv, N, d).sum((2, 3))
    np.testing.assert_allclose(r["dv"].sum(2), want, rtol=1e-12, atol=1e-12)
    # the causal tail block with a window matches the full backward
    full = oracle.bwd_groups(q, k, v, dout, 0.35, True, [1, 2], window=W)
    tail = oracle.bwd_groups_tail(q, k, v, dout, 0.35, 13, [1, 2], window=W)
    for name in ("dq", "o"):
        np.testing.assert_array_equal(tail[name], full[name][:, :, 13:])
    for name in ("dk", "dv"):
        np.testing.assert_array_equal(tail[name], full[name][:, 13:])
