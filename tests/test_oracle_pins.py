"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

No pin re-types an oracle formula: each one compares the oracle with a closed
form, a special case that reduces to a textbook computation (done here with
plain numpy matrix algebra), brute force, an invariant, a hand-written fixture
(tests/golden/) or a library routine.  Sources are cited by page title and
section:

* "Retentive Network" paper summary (blog.csdn.net), Sec. 2.1 "Retention"
  (parallel (1), recurrent (2), chunkwise (3) representations) and Sec. 2.2
  "Gated Multi-Scale Retention".
* "RetNet dual-mode hands-on manual", Sec. 1 (decay matrix) and Sec. 3.1
  (the recurrent form unrolls to the parallel form).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import CHUNKWISE_32K, PARALLEL_2K, TINY, multiscale_gamma, rotation_theta

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load_txt(name):
    return np.loadtxt(os.path.join(GOLD, name), comments="#")


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, H, L, dk, dv, seed=0):
    return _rand((B, H, L, dk), seed), _rand((B, H, L, dk), seed + 1), _rand((B, H, L, dv), seed + 2)


def _gam(H):
    return multiscale_gamma(H).double().numpy()


def _th(dk):
    return rotation_theta(dk).double().numpy()


# ---------------------------------------------------------------- fixtures
def test_gamma_fixture_matches_workload_generator():
    """gamma_h = 1 - 2^(-5-h) (Sec. 2.2), hand-written fixture vs the workload generator."""
    g = _load_txt("msr_gamma_h8.txt")
    assert np.array_equal(multiscale_gamma(8).double().numpy(), g)


def test_theta_values():
    th = rotation_theta(16).double().numpy()
    assert th[0] == 1.0
    assert np.allclose(th, 10000.0 ** (-2.0 * np.arange(8) / 16), rtol=1e-7)


# ---------------------------------------------------------------- P3: decay mask
@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunk2", "chunk3"])
def test_mask_extraction_fixture(form):
    """theta = 0, q_n = k_m = e_0, v_m = e_m: o[n][m] = D[n][m].  Compared with the
    hand-written gamma = 0.5 fixture (lower-triangular, D_nn = 1, geometric)."""
    D = _load_txt("decay_mask_gamma0.5_L5.txt")
    L = 5
    q = np.zeros((1, 1, L, 2)); q[..., 0] = 1.0
    k = q.copy()
    v = np.eye(L)[None, None]
    g = np.array([0.5])
    if form == "parallel":
        o = oracle.parallel(q, k, v, g)
    elif form == "recurrent":
        o, _ = oracle.recurrent(q, k, v, g)
    else:
        o, _ = oracle.chunkwise(q, k, v, g, int(form[-1]))
    assert np.array_equal(o[0, 0], D)


def test_mask_structure_and_rotation_phase():
    """Same probe with rotation on: o[n][m] = gamma^(n-m) cos((n-m) theta_0)."""
    L, gm = 64, 1 - 2 ** -5
    q = np.zeros((1, 1, L, 16)); q[..., 0] = 1.0
    v = np.eye(L)[None, None]
    th = _th(16)
    o = oracle.parallel(q, q.copy(), v, np.array([gm]), th, pos0=7)[0, 0]
    n, m = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    expect = np.where(n >= m, gm ** (n - m) * np.cos((n - m) * th[0]), 0.0)
    assert _rel(o, expect) < 1e-12
    # structure: strictly upper triangle zero, unit diagonal when theta = 0
    o0 = oracle.parallel(q, q.copy(), v, np.array([gm]))[0, 0]
    assert np.all(np.triu(o0, 1) == 0.0)
    assert np.all(np.diag(o0) == 1.0)
    assert np.allclose(o0[1:, :-1][np.tril_indices(L - 1)] / o0[:-1, :-1][np.tril_indices(L - 1)], gm,
                       rtol=1e-13)


# ---------------------------------------------------------------- P1, P2, P5: three forms agree
def test_tiny_workload_three_forms_agree():
    """Tiny workload (B1 H2 L64 dk=dv=16, chunk 16): parallel = recurrent = chunkwise."""
    q, k, v = TINY.qkv()
    g, th = TINY.gamma(), TINY.theta()
    op = oracle.parallel(q, k, v, g, th)
    orr, sr = oracle.recurrent(q, k, v, g, th)
    oc, sc = oracle.chunkwise(q, k, v, g, 16, th)
    assert _rel(orr, op) < 1e-12
    assert _rel(oc, op) < 1e-12
    assert _rel(sc, sr) < 1e-12


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 23, 64, 100])
def test_chunk_size_independence(chunk):
    """Outputs and final state do not depend on the chunk size, including chunk sizes
    that leave a short last chunk; chunk = 1 is the recurrent form, chunk >= L the
    parallel form."""
    q, k, v = _qkv(2, 3, 64, 8, 12, seed=3)
    g, th = _gam(3), _th(8)
    s0 = _rand((2, 3, 8, 12), 9)
    op = oracle.parallel(q, k, v, g, th, pos0=5)
    oc, sc = oracle.chunkwise(q, k, v, g, chunk, th, pos0=5)
    orr, sr = oracle.recurrent(q, k, v, g, th, pos0=5)
    assert _rel(oc, op) < 1e-12 and _rel(orr, op) < 1e-12
    assert _rel(sc, sr) < 1e-12
    oc2, sc2 = oracle.chunkwise(q, k, v, g, chunk, th, pos0=5, s_in=s0)
    orr2, sr2 = oracle.recurrent(q, k, v, g, th, pos0=5, s_in=s0)
    assert _rel(oc2, orr2) < 1e-12 and _rel(sc2, sr2) < 1e-12


# ---------------------------------------------------------------- P4: linear attention
def test_gamma1_theta0_is_causal_linear_attention():
    """gamma = 1, no rotation: o_n = sum_{m<=n} (q_n . k_m) v_m, i.e. causal
    unnormalised linear attention, computed here as tril(Q K^T) V with numpy."""
    q, k, v = _qkv(1, 2, 40, 6, 5, seed=11)
    g = np.ones(2)
    expect = np.tril(q @ np.swapaxes(k, -1, -2)) @ v
    for o in (oracle.parallel(q, k, v, g), oracle.recurrent(q, k, v, g)[0],
              oracle.chunkwise(q, k, v, g, 7)[0]):
        assert _rel(o, expect) < 1e-12
    # brute force, pure python, on a few rows
    for n in (0, 17, 39):
        bf = sum(float(np.dot(q[0, 1, n], k[0, 1, m])) * v[0, 1, m] for m in range(n + 1))
        assert np.allclose(oracle.parallel(q, k, v, g)[0, 1, n], bf, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- P6: closed form
@pytest.mark.parametrize("use_theta", [False, True])
def test_constant_inputs_closed_form(use_theta):
    """q_n = k_m = u, v = 1:  o_n[j] = sum_i |z_i|^2 Re[(1 - w_i^(n+1)) / (1 - w_i)],
    z_i = u_{2i} + i u_{2i+1}, w_i = gamma e^{i theta_i} (geometric series)."""
    L, dk, dv = 300, 8, 3
    u = _rand(dk, 21)
    q = np.broadcast_to(u, (1, 1, L, dk)).copy()
    v = np.ones((1, 1, L, dv))
    gm = 0.99
    th = _th(dk) if use_theta else np.zeros(dk // 2)
    z2 = u[0::2] ** 2 + u[1::2] ** 2
    w = gm * np.exp(1j * th)
    n = np.arange(L)[:, None]
    expect = (z2 * np.real((1 - w ** (n + 1)) / (1 - w))).sum(-1)
    for o in (oracle.parallel(q, q.copy(), v, np.array([gm]), th if use_theta else None, pos0=123),
              oracle.chunkwise(q, q.copy(), v, np.array([gm]), 64, th if use_theta else None,
                               pos0=123)[0]):
        assert _rel(o[0, 0, :, 0], expect) < 1e-11
        assert np.all(o[0, 0, :, 1] == o[0, 0, :, 0])


# ---------------------------------------------------------------- P7: translation invariance
@pytest.mark.parametrize("delta", [1, 100000])
def test_translation_invariance(delta):
    q, k, v = _qkv(1, 2, 48, 16, 8, seed=31)
    g, th = _gam(2), _th(16)
    a = oracle.parallel(q, k, v, g, th, pos0=0)
    b = oracle.parallel(q, k, v, g, th, pos0=delta)
    assert _rel(b, a) < 1e-10


# ---------------------------------------------------------------- P8: pairing permutation
def test_pairing_permutation_equivalence():
    """Interleaved pairs (2i, 2i+1) and the 'halves' pairing (i, i + dk/2) give the same
    result after one fixed permutation of the dk axis of Q and K."""
    q, k, v = _qkv(1, 2, 32, 16, 4, seed=41)
    g, th = _gam(2), _th(16)
    perm = np.empty(16, dtype=int)
    perm[0::2] = np.arange(8)
    perm[1::2] = np.arange(8) + 8
    # halves layout: x_h[i] = real part, x_h[i+8] = imag part
    qh = np.empty_like(q); kh = np.empty_like(k)
    qh[..., perm] = q; kh[..., perm] = k
    # rotate halves by explicit formula (textbook rotary form) and take real dot product
    pos = np.arange(32)[:, None]
    c, s = np.cos(pos * th), np.sin(pos * th)

    def rot_halves(x):
        re, im = x[..., :8], x[..., 8:]
        return np.concatenate([re * c - im * s, re * s + im * c], -1)

    qr, kr = rot_halves(qh), rot_halves(kh)
    n, m = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
    out = []
    for h in range(2):
        D = np.where(n >= m, g[h] ** np.maximum(n - m, 0), 0.0)
        out.append(((qr[0, h] @ kr[0, h].T) * D) @ v[0, h])
    assert _rel(oracle.parallel(q, k, v, g, th)[0], np.stack(out)) < 1e-12


# ---------------------------------------------------------------- P9: gamma = 0
def test_gamma0_is_diagonal():
    q, k, v = _qkv(1, 1, 20, 8, 6, seed=51)
    expect = np.einsum("bhnd,bhnd->bhn", q, k)[..., None] * v
    for th in (None, _th(8)):
        o = oracle.parallel(q, k, v, np.zeros(1), th, pos0=99)
        assert _rel(o, expect) < 1e-12
        assert _rel(oracle.chunkwise(q, k, v, np.zeros(1), 6, th, pos0=99)[0], expect) < 1e-12
        assert _rel(oracle.recurrent(q, k, v, np.zeros(1), th, pos0=99)[0], expect) < 1e-12


# ---------------------------------------------------------------- P10: algebra
def test_linearity_scaling_heads_causality_L1():
    q, k, v = _qkv(1, 3, 24, 8, 6, seed=61)
    g, th = _gam(3), _th(8)
    o = oracle.parallel(q, k, v, g, th)
    v2 = _rand(v.shape, 62)
    assert _rel(oracle.parallel(q, k, v + 2.5 * v2, g, th), o + 2.5 * oracle.parallel(q, k, v2, g, th)) < 1e-12
    assert _rel(oracle.parallel(2 * q, 3 * k, -0.5 * v, g, th), -3.0 * o) < 1e-12
    perm = [2, 0, 1]
    op = oracle.parallel(q[:, perm], k[:, perm], v[:, perm], g[perm], th)
    assert _rel(op, o[:, perm]) < 1e-12
    # causality: changing token p changes no output before p
    p = 10
    q3, k3, v3 = q.copy(), k.copy(), v.copy()
    q3[:, :, p] += 1.0; k3[:, :, p] -= 2.0; v3[:, :, p] *= 3.0
    o3 = oracle.parallel(q3, k3, v3, g, th)
    assert np.array_equal(o3[:, :, :p], o[:, :, :p])
    assert not np.allclose(o3[:, :, p], o[:, :, p])
    # L = 1: o = (q . k) v (rotation at one position cancels)
    o1 = oracle.parallel(q[:, :, :1], k[:, :, :1], v[:, :, :1], g, th, pos0=77)
    assert _rel(o1, (q[:, :, :1] * k[:, :, :1]).sum(-1, keepdims=True) * v[:, :, :1]) < 1e-12


# ---------------------------------------------------------------- P11: state composition
def test_state_composition():
    q, k, v = _qkv(2, 2, 70, 8, 10, seed=71)
    g, th = _gam(2), _th(8)
    o, s = oracle.chunkwise(q, k, v, g, 16, th, pos0=3)
    L1 = 29
    o1, s1 = oracle.chunkwise(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], g, 16, th, pos0=3)
    o2, s2 = oracle.chunkwise(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], g, 16, th, pos0=3 + L1, s_in=s1)
    assert _rel(np.concatenate([o1, o2], 2), o) < 1e-12
    assert _rel(s2, s) < 1e-12
    # decode steps after a prefill state = one long run
    st = s1
    outs = []
    for t in range(L1, 70):
        ot, st = oracle.recurrent(q[:, :, t:t + 1], k[:, :, t:t + 1], v[:, :, t:t + 1], g, th,
                                  pos0=3 + t, s_in=st)
        outs.append(ot)
    assert _rel(np.concatenate(outs, 2), o[:, :, L1:]) < 1e-12
    assert _rel(st, s) < 1e-12


# ---------------------------------------------------------------- P15: complex transcription
def test_complex_transcription_agrees():
    q, k, v = _qkv(1, 2, 40, 16, 6, seed=81)
    g, th = _gam(2), _th(16)
    assert _rel(oracle.parallel(q, k, v, g, th, pos0=11),
                oracle.parallel_complex(q, k, v, g, th, pos0=11)) < 1e-12


def test_rotation_is_orthogonal_and_relative():
    x = _rand((3, 50, 16), 91)
    th = _th(16)
    xr = oracle.rotate(x, th, pos0=1000)
    assert np.allclose(np.linalg.norm(xr, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # (R_p a) . (R_p b) = a . b
    y = _rand((3, 50, 16), 92)
    assert np.allclose((xr * oracle.rotate(y, th, pos0=1000)).sum(-1), (x * y).sum(-1), rtol=1e-11,
                       atol=1e-12)


# ---------------------------------------------------------------- spot-check helpers
def test_rows_and_state_entries_match_full_forms():
    q, k, v = _qkv(2, 3, 40, 8, 6, seed=101)
    g, th = _gam(3), _th(8)
    s0 = _rand((2, 3, 8, 6), 102)
    o, s = oracle.recurrent(q, k, v, g, th, pos0=17, s_in=s0)
    idx = [(0, 0, 0), (1, 2, 39), (0, 1, 20), (1, 0, 5)]
    r = oracle.rows(q, k, v, g, idx, th, pos0=17, s_in=s0)
    assert _rel(r, np.stack([o[b, h, n] for b, h, n in idx])) < 1e-12
    sidx = [(0, 0, 0, 0), (1, 2, 7, 5), (0, 1, 3, 2)]
    se = oracle.state_entries(k, v, g, sidx, th, pos0=17, s_in=s0)
    assert _rel(se, np.array([s[b, h, a, c] for b, h, a, c in sidx])) < 1e-12


# ---------------------------------------------------------------- P12: GroupNorm
def test_groupnorm_properties_and_library():
    """Per-(token, head) GroupNorm: mean 0 and mean square var/(var+eps) per row, and
    equal to torch's group_norm with one group per head and no affine."""
    B, H, L, dv, eps = 2, 3, 5, 16, 1e-2
    o = _rand((B, H, L, dv), 111) * 0.2
    y = oracle.groupnorm(o, eps)
    var = o.var(-1)
    assert np.allclose(y.mean(-1), 0.0, atol=1e-14)
    assert np.allclose((y ** 2).mean(-1), var / (var + eps), rtol=1e-12)
    t = torch.from_numpy(np.ascontiguousarray(o.transpose(0, 2, 1, 3).reshape(B * L, H * dv)))
    ref = torch.nn.functional.group_norm(t, H, eps=eps).numpy().reshape(B, L, H, dv).transpose(0, 2, 1, 3)
    assert _rel(y, ref) < 1e-12


def test_matmul_and_swish_library():
    x, w = _rand((7, 13), 121), _rand((5, 13), 122)
    assert _rel(oracle.matmul_nt(x, w), x @ w.T) < 1e-13
    z = _rand(100, 123) * 4
    assert _rel(oracle.swish(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy()) < 1e-14
    assert oracle.swish(np.zeros(3)).tolist() == [0.0, 0.0, 0.0]


def test_parallel_and_recurrent_agree_at_the_parallel_workload():
    """The parallel workload's reference is the literal double sum; the recurrent
    form (an independent algorithm) must give the same outputs on four (b, h)
    slices of its seeded inputs at full length ("Retentive Network" paper summary,
    Sec. 2.1 (1) and (2))."""
    wl = PARALLEL_2K
    q, k, v = wl.qkv()
    g, th = wl.gamma(), wl.theta()
    pick = [(0, 0), (3, 2), (5, 5), (7, 7)]
    sel = lambda t: torch.stack([t[b, h] for b, h in pick])[None]
    gs = [float(g[h]) for _, h in pick]
    par = oracle.parallel(sel(q), sel(k), sel(v), gs, th)
    rec, _ = oracle.recurrent(sel(q), sel(k), sel(v), gs, th)
    err = np.abs(par - rec).max() / np.abs(par).max()
    assert err < 1e-11, err


def test_recurrent_and_parallel_agree_at_the_chunkwise_workload():
    """The long-context workload's reference is the recurrent form; the literal
    double sum must agree with it on the first 4096 tokens of the fastest- and
    slowest-decaying heads of its seeded inputs (Sec. 2.1 (1) and (2))."""
    wl = CHUNKWISE_32K
    q, k, v = wl.qkv()
    g, th = wl.gamma(), wl.theta()
    hs, n = [0, wl.H - 1], 4096
    sel = lambda t: t[:, hs, :n].contiguous()
    gs = [float(g[h]) for h in hs]
    par = oracle.parallel(sel(q), sel(k), sel(v), gs, th)
    rec, _ = oracle.recurrent(sel(q), sel(k), sel(v), gs, th)
    err = np.abs(par - rec).max() / np.abs(par).max()
    assert err < 1e-11, err
