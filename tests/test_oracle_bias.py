"""Pins for the oracle's linear position bias (no GPU).

With one slope a_h per query head, score s_ij = scale * q_i . k_j + a_h (j - i)
(the ALiBi form of an additive score modification).  Pinned to:
  * brute force in pure Python (math.exp / math.fsum), causal, non-causal,
    GQA, with a sliding window;
  * torch's scaled_dot_product_attention with the bias as an explicit float
    mask, its logsumexp, and float64 autograd for the gradients;
  * closed forms: with Q = 0 the causal LSE is a geometric series,
    LSE_i = ln((1 - e^{-a (i+1)}) / (1 - e^{-a}));
  * a = 0 equals the plain oracle bit for bit; a large slope concentrates
    causal row i on key i (a sign error would concentrate it on key 0);
  * row-shift invariance: the -a i part is a per-row constant, so O does not
    change and LSE moves by exactly that constant when it is dropped.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_bits_to_f32, random_bf16


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def brute_fwd_bias(q, k, v, scale, causal, slopes, window=0):
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
                keys = [j for j in range(N)
                        if (not causal or j <= i) and (window <= 0 or j > i - window)]
                s = [sc * math.fsum(qf[b, h, i, c] * kf[b, g, j, c] for c in range(d))
                     + slopes[h] * (j - i) for j in keys]
                m = max(s)
                p = [math.exp(x - m) for x in s]
                l = math.fsum(p)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(p[t] * vf[b, g, j, c] for t, j in enumerate(keys)) / l
                lse[b, h, i] = m + math.log(l)
    return o, lse


def slopes_for(Hq, seed):
    return np.random.default_rng(seed).uniform(-0.6, 0.9, Hq)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 1, 1, 6, 3), (1, 2, 1, 9, 4), (2, 4, 2, 7, 5)])
def test_bias_forward_brute_force(B, Hq, Hkv, N, d, causal, window):
    q, k, v = (random_bf16((B, Hq, N, d), 1), random_bf16((B, Hkv, N, d), 2),
               random_bf16((B, Hkv, N, d), 3))
    a = slopes_for(Hq, 4)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.fwd(q, k, v, scale, causal, window=window, slopes=a)
    ob, lseb = brute_fwd_bias(q, k, v, scale, causal, a, window)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-13)


def torch_ref(q, k, v, do, scale, causal, slopes):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    qt = torch.tensor(f64(q), requires_grad=True)
    kt = torch.tensor(f64(k), requires_grad=True)
    vt = torch.tensor(f64(v), requires_grad=True)
    kr = kt.repeat_interleave(Hq // Hkv, dim=1)
    vr = vt.repeat_interleave(Hq // Hkv, dim=1)
    i = torch.arange(N, dtype=torch.float64)[:, None]
    j = torch.arange(N, dtype=torch.float64)[None, :]
    bias = torch.tensor(slopes, dtype=torch.float64)[:, None, None] * (j - i)  # [Hq, N, N]
    if causal:
        bias = bias.masked_fill(j > i, float("-inf"))
    sc = float(np.float32(scale))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, attn_mask=bias[None], scale=sc)
    lse = torch.logsumexp(sc * qt @ kr.transpose(-1, -2) + bias[None], dim=-1)
    o.backward(torch.tensor(f64(do)))
    return o.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 2, 2, 33, 8), (2, 4, 2, 40, 16)])
def test_bias_matches_torch_sdpa_and_autograd(B, Hq, Hkv, N, d, causal):
    q, k, v, do = (random_bf16((B, Hq, N, d), 5), random_bf16((B, Hkv, N, d), 6),
                   random_bf16((B, Hkv, N, d), 7), random_bf16((B, Hq, N, d), 8))
    a = slopes_for(Hq, 9)
    scale = 1 / math.sqrt(d)
    o_t, lse_t, dq_t, dk_t, dv_t = torch_ref(q, k, v, do, scale, causal, a)
    o, lse = oracle.fwd(q, k, v, scale, causal, slopes=a)
    np.testing.assert_allclose(o, o_t, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=1e-10, atol=1e-12)
    r = oracle.bwd(q, k, v, do, scale, causal, slopes=a)
    np.testing.assert_allclose(r["o"], o_t, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dq"], dq_t, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r["dk"], dk_t, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r["dv"], dv_t, rtol=1e-9, atol=1e-11)


def test_bias_closed_form_zero_queries():
    B, Hq, Hkv, N, d = 1, 3, 1, 50, 4
    q = np.zeros((B, Hq, N, d), np.uint16)  # bf16 +0
    k, v = random_bf16((B, Hkv, N, d), 10), random_bf16((B, Hkv, N, d), 11)
    a = np.array([0.25, 1.5, 3.0])
    o, lse = oracle.fwd(q, k, v, 0.125, True, slopes=a)
    vf = f64(v)[0, 0]
    for h in range(Hq):
        for i in range(N):
            want = math.log((1 - math.exp(-a[h] * (i + 1))) / (1 - math.exp(-a[h])))
            assert abs(lse[0, h, i] - want) < 1e-12
            w = np.exp(a[h] * (np.arange(i + 1) - i))
            np.testing.assert_allclose(o[0, h, i], (w[:, None] * vf[:i + 1]).sum(0) / w.sum(),
                                       rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_slopes_equal_plain_oracle_bitwise(causal):
    B, Hq, Hkv, N, d = 2, 4, 2, 37, 16
    q, k, v, do = (random_bf16((B, Hq, N, d), 12), random_bf16((B, Hkv, N, d), 13),
                   random_bf16((B, Hkv, N, d), 14), random_bf16((B, Hq, N, d), 15))
    zero = np.zeros(Hq)
    o0, l0 = oracle.fwd(q, k, v, 0.25, causal)
    o1, l1 = oracle.fwd(q, k, v, 0.25, causal, slopes=zero)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    r0 = oracle.bwd(q, k, v, do, 0.25, causal)
    r1 = oracle.bwd(q, k, v, do, 0.25, causal, slopes=zero)
    for name in ("dq", "dk", "dv", "o", "lse"):
        assert np.array_equal(r0[name], r1[name]), name


def test_large_slope_concentrates_on_the_diagonal():
    B, Hq, Hkv, N, d = 1, 1, 1, 30, 8
    q, k, v = (random_bf16((B, Hq, N, d), 16), random_bf16((B, Hkv, N, d), 17),
               random_bf16((B, Hkv, N, d), 18))
    o, _ = oracle.fwd(q, k, v, 0.01, True, slopes=np.array([60.0]))
    np.testing.assert_allclose(o[0, 0], f64(v)[0, 0], rtol=0, atol=1e-20)


def test_row_constant_part_of_the_bias():
    """a (j - i) = a j - a i: dropping the per-row constant -a i leaves O and
    moves LSE by a i.  Checked by comparing slopes a against the same bias
    built from keys alone on a non-causal problem, via the brute force."""
    B, Hq, Hkv, N, d = 1, 2, 2, 8, 4
    q, k, v = (random_bf16((B, Hq, N, d), 19), random_bf16((B, Hkv, N, d), 20),
               random_bf16((B, Hkv, N, d), 21))
    a = np.array([0.7, -0.3])
    o, lse = oracle.fwd(q, k, v, 0.5, False, slopes=a)
    qf, kf, vf = f64(q), f64(k), f64(v)
    sc = float(np.float32(0.5))
    for h in range(Hq):
        s = sc * qf[0, h] @ kf[0, h].T + a[h] * np.arange(N)[None, :]  # keys-only bias
        m = s.max(1, keepdims=True)
        p = np.exp(s - m)
        np.testing.assert_allclose(o[0, h], (p @ vf[0, h]) / p.sum(1, keepdims=True),
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], (m[:, 0] + np.log(p.sum(1))) - a[h] * np.arange(N),
                                   rtol=1e-12, atol=1e-12)
