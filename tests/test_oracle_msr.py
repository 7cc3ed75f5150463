"""Pins of the oracle's gated multi-scale retention layer ("Retentive Network" paper
summary, Sec. 2.2 "Gated Multi-Scale Retention"):

    MSR(X) = (swish(X W_G) (.) GroupNorm_h(Concat_h Retention(X, gamma_h))) W_O

Weights are stored [out, in].  Pins: gamma = 0 reduces retention to
o_n = (q_n . k_n) v_n, which gives a closed form computed here with numpy
matmuls; a zero gate gives zero output; GroupNorm makes the output invariant to
scaling W_Q (up to eps); the token-sampled path equals the full path.
"""
import numpy as np

import oracle
from workloads import multiscale_gamma, rotation_theta

B, L, DM, H, DK, DV = 2, 37, 32, 2, 8, 16


def _w(seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, L, DM))
    w_q = r.standard_normal((H * DK, DM)) * 0.2
    w_k = r.standard_normal((H * DK, DM)) * 0.2
    w_v = r.standard_normal((H * DV, DM)) * 0.2
    w_g = r.standard_normal((H * DV, DM)) * 0.2
    w_o = r.standard_normal((DM, H * DV)) * 0.2
    return x, w_q, w_k, w_v, w_g, w_o


def _rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


def test_gamma0_closed_form():
    x, w_q, w_k, w_v, w_g, w_o = _w(1)
    eps = 1e-5
    th = rotation_theta(DK).double().numpy()
    y = oracle.msr_layer(x, w_q, w_k, w_v, w_g, w_o, H, DK, DV, np.zeros(H), th, pos0=9, gn_eps=eps)
    X = x.reshape(B * L, DM)
    q = (X @ w_q.T).reshape(-1, H, DK)
    k = (X @ w_k.T).reshape(-1, H, DK)
    v = (X @ w_v.T).reshape(-1, H, DV)
    a = (q * k).sum(-1, keepdims=True)                       # q_n . k_n, rotation cancels
    mu = v.mean(-1, keepdims=True)
    var = v.var(-1, keepdims=True)
    gn = a * (v - mu) / np.sqrt(a * a * var + eps)            # GroupNorm of a * v
    gx = X @ w_g.T
    gate = gx / (1.0 + np.exp(-gx))
    expect = ((gate * gn.reshape(-1, H * DV)) @ w_o.T).reshape(B, L, DM)
    assert _rel(y, expect) < 1e-11


def test_zero_gate_gives_zero():
    x, w_q, w_k, w_v, w_g, w_o = _w(2)
    g = multiscale_gamma(H).double().numpy()
    y = oracle.msr_layer(x, w_q, w_k, w_v, np.zeros_like(w_g), w_o, H, DK, DV, g)
    assert np.all(y == 0.0)


def test_scale_invariance_of_wq():
    x, w_q, w_k, w_v, w_g, w_o = _w(3)
    g = multiscale_gamma(H).double().numpy()
    th = rotation_theta(DK).double().numpy()
    y1 = oracle.msr_layer(x, w_q, w_k, w_v, w_g, w_o, H, DK, DV, g, th, gn_eps=1e-8)
    y2 = oracle.msr_layer(x, 3.0 * w_q, w_k, w_v, w_g, w_o, H, DK, DV, g, th, gn_eps=1e-8)
    assert _rel(y2, y1) < 1e-6


def test_sampled_tokens_equal_full():
    x, w_q, w_k, w_v, w_g, w_o = _w(4)
    g = multiscale_gamma(H).double().numpy()
    th = rotation_theta(DK).double().numpy()
    y = oracle.msr_layer(x, w_q, w_k, w_v, w_g, w_o, H, DK, DV, g, th, pos0=4, gn_eps=1e-5)
    toks = [(1, 36), (0, 0), (1, 5), (0, 20)]
    ys = oracle.msr_layer(x, w_q, w_k, w_v, w_g, w_o, H, DK, DV, g, th, pos0=4, gn_eps=1e-5, tokens=toks)
    assert _rel(ys, np.stack([y[b, l] for b, l in toks])) < 1e-12
