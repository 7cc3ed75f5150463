"""Pins of the oracle's block wrapper pieces (the pre-LN residual block and FFN of
the "Retentive Network" paper summary): LayerNorm and gelu against library
routines and their defining properties, and the block's reductions when the
layer's or the FFN's output weights vanish."""
import numpy as np
import torch

import oracle


def _r(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_layernorm_properties_and_library():
    x = _r((7, 33), 1) * 3 + 2
    y = oracle.layernorm(x, 1e-5)
    var = x.var(-1)
    assert np.allclose(y.mean(-1), 0.0, atol=1e-13)
    assert np.allclose((y ** 2).mean(-1), var / (var + 1e-5), rtol=1e-12)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (33,), eps=1e-5).numpy()
    assert np.abs(y - ref).max() < 1e-12


def test_gelu_library_and_values():
    x = np.linspace(-6, 6, 241)
    y = oracle.gelu(x)
    ref = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    assert np.abs(y - ref).max() < 1e-14
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    # gelu(x) - gelu(-x) = x (Phi(x) + Phi(-x) = 1)
    assert np.allclose(y - y[::-1], x, atol=1e-14)


def _weights(dm, H, dk, dv, dff, seed):
    return [_r((H * dk, dm), seed, 0.05), _r((H * dk, dm), seed + 1, 0.05), _r((H * dv, dm), seed + 2, 0.05),
            _r((H * dv, dm), seed + 3, 0.05), _r((dm, H * dv), seed + 4, 0.05), _r((dff, dm), seed + 5, 0.05),
            _r((dm, dff), seed + 6, 0.05)]


def test_block_reductions():
    """W_O = 0 and W_2 = 0 give the identity; W_2 = 0 leaves X + MSR(LN(X)); the
    sampled-row form equals the full form."""
    B, L, dm, H, dk, dv, dff = 2, 11, 16, 2, 4, 8, 24
    x = _r((B, L, dm), 5)
    w = _weights(dm, H, dk, dv, dff, 10)
    g, th = [0.9, 0.7], np.array([0.5, 0.05])
    z4, z6 = np.zeros_like(w[4]), np.zeros_like(w[6])
    same = oracle.retnet_block(x, *w[:4], z4, w[5], z6, H, dk, dv, g, th)
    assert np.abs(same - x).max() == 0.0
    y = oracle.retnet_block(x, *w[:6], z6, H, dk, dv, g, th)
    ref = x + oracle.msr_layer(oracle.layernorm(x, 1e-5), *w[:5], H, dk, dv, g, th)
    assert np.abs(y - ref).max() < 1e-12
    full = oracle.retnet_block(x, *w, H, dk, dv, g, th, pos0=3)
    toks = [(0, 0), (1, 10), (0, 5)]
    part = oracle.retnet_block(x, *w, H, dk, dv, g, th, pos0=3, tokens=toks)
    assert np.abs(part - np.stack([full[b, l] for b, l in toks])).max() < 1e-12
