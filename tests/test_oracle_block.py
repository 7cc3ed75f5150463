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


def _perm(n, seed):
    p = np.random.default_rng(seed).permutation(n)
    assert np.any(p[p] != np.arange(n)), "want a permutation that is not its own inverse"
    return p


def _ffn_pin_error(block_fn):
    """Largest deviation of block_fn's FFN branch from a closed form.

    The block equations give out = Y + FFN(LN(Y)), FFN(Z) = gelu(Z W_1) W_2, with
    Y = MSR(LN(X)) + X.  Y is taken from the same block with W_2 = 0 (that
    reduction is pinned above).  W_1 [d_ffn, d_model] and W_2 [d_model, d_ffn]
    (stored [out, in]) are scaled selection matrices, d_ffn = 2 d_model:
      row j < d_model of W_1 is c1 e_{pi1(j)}, row d_model + j is c2 e_{pi2(j)},
      row i of W_2 is d1 e_{s1(i)} + d2 e_{d_model + s2(i)},
    so FFN(Z)[:, i] = d1 gelu(c1 Z[:, pi1(s1(i))]) + d2 gelu(c2 Z[:, pi2(s2(i))])
    by indexing alone.  LN and gelu come from torch (library routines)."""
    B, L, dm, H, dk, dv = 2, 9, 16, 2, 4, 8
    x = _r((B, L, dm), 21) * 1.5 + 0.3
    w = _weights(dm, H, dk, dv, 2 * dm, 30)[:5]
    w[4] = w[4] * 40.0  # a large W_O, so Y is far from X
    g, th = [0.9, 0.6], np.array([0.3, 0.02])
    pi1, pi2, s1, s2 = _perm(dm, 1), _perm(dm, 2), _perm(dm, 3), _perm(dm, 4)
    c1, c2, d1, d2 = 1.7, -0.6, 2.5, 0.75
    w1 = np.zeros((2 * dm, dm))
    w1[np.arange(dm), pi1] = c1
    w1[dm + np.arange(dm), pi2] = c2
    w2 = np.zeros((dm, 2 * dm))
    w2[np.arange(dm), s1] = d1
    w2[np.arange(dm), dm + s2] = d2
    y = block_fn(x, *w, w1, np.zeros_like(w2), H, dk, dv, g, th, pos0=2)
    out = block_fn(x, *w, w1, w2, H, dk, dv, g, th, pos0=2)
    if np.abs(y - x).max() < 1.0:  # the W_2 = 0 reduction must leave Y = MSR(LN(X)) + X, far from X here
        return float("inf")
    ln = torch.nn.functional.layer_norm(torch.from_numpy(y), (dm,), eps=1e-5)
    gelu = torch.nn.functional.gelu
    expect = y + (d1 * gelu(c1 * ln[..., pi1[s1]]) + d2 * gelu(c2 * ln[..., pi2[s2]])).numpy()
    return float(np.abs(out - expect).max())


def test_block_ffn_branch_closed_form():
    assert _ffn_pin_error(oracle.retnet_block) < 1e-12


def _mutant(kind):
    """The block with one plausible composition mistake in the FFN branch."""
    def block(x, w_q, w_k, w_v, w_g, w_o, w_1, w_2, H, dk, dv, gamma, theta=None, pos0=0, gn_eps=1e-5,
              ln_eps=1e-5):
        x = oracle.as_f64(x)
        B, L, dm = x.shape
        y = (oracle.msr_layer(oracle.layernorm(x, ln_eps), w_q, w_k, w_v, w_g, w_o, H, dk, dv, gamma, theta, pos0,
                              gn_eps) + x).reshape(B * L, dm)
        x2 = x.reshape(B * L, dm)
        src = {"ln_of_x": oracle.layernorm(x2, ln_eps), "no_ln": y}.get(kind, oracle.layernorm(y, ln_eps))
        if kind == "gelu_after_w2":
            f = oracle.gelu(oracle.matmul_nt(oracle.matmul_nt(src, w_1), w_2))
        elif kind == "transposed_w1":
            f = oracle.matmul_nt(oracle.gelu(src @ w_1[:dm, :dm]), w_2[:, :dm])
        else:
            f = oracle.matmul_nt(oracle.gelu(oracle.matmul_nt(src, w_1)), w_2)
        base = x2 if kind == "residual_x" else y
        return (base + f).reshape(B, L, dm)
    return block


def test_block_ffn_pin_rejects_composition_mistakes():
    """The pin above fails each plausible mistake and passes the correct composition
    written the same way (so the mutants differ from it only in the mistake)."""
    assert _ffn_pin_error(_mutant("correct")) < 1e-12
    for kind in ("ln_of_x", "gelu_after_w2", "residual_x", "no_ln", "transposed_w1"):
        assert _ffn_pin_error(_mutant(kind)) > 1e-3, kind
