"""Pins of the oracle's gradients of retention (no GroupNorm): central differences
of the forward oracle, the degree-one homogeneity identities, a closed form at
gamma = 0, and agreement of the sampled-row function with the full one.  Forward
definition: "Retentive Network" paper summary, Sec. 2.1 (scalar-gamma form)."""
import numpy as np
import pytest

import oracle


def _inputs(B, H, L, dk, dv, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal(s) for s in ((B, H, L, dk), (B, H, L, dk), (B, H, L, dv), (B, H, L, dv))]


THETA = np.array([0.7, 0.11, 0.013])
GAMMA = np.array([0.9, 0.55])


@pytest.mark.parametrize("pos0", [0, 9])
def test_gradients_match_central_differences(pos0):
    """Every entry of dq, dk and dv equals the central difference of
    sum(o * dO) computed with the forward oracle (the loss is quadratic in
    (q, k) jointly and linear in each, so the difference quotient is exact up to
    rounding)."""
    B, H, L, dk, dv = 1, 2, 7, 6, 3
    q, k, v, do = _inputs(B, H, L, dk, dv, 1)
    dq, dkk, dvv = oracle.backward(q, k, v, do, GAMMA, THETA, pos0)

    def loss(q_, k_, v_):
        return float((oracle.parallel(q_, k_, v_, GAMMA, THETA, pos0) * do).sum())
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dkk), ("v", v, dvv)):
        fd = np.empty_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.abs(fd - grad).max() / np.abs(grad).max()
        assert err < 1e-7, f"d{name}: {err:.2e}"


def test_homogeneity_identities():
    """o is linear in v, in q and in k separately (rotation is linear), so
    sum(dv*v) = sum(dq*q) = sum(dk*k) = sum(dO*o)."""
    q, k, v, do = _inputs(2, 2, 33, 6, 5, 2)
    dq, dkk, dvv = oracle.backward(q, k, v, do, GAMMA, THETA, 4)
    ref = float((oracle.parallel(q, k, v, GAMMA, THETA, 4) * do).sum())
    for x, gx in ((q, dq), (k, dkk), (v, dvv)):
        assert abs(float((x * gx).sum()) - ref) <= 1e-11 * max(1.0, abs(ref))


def test_gamma0_closed_form():
    """gamma = 0 keeps only n = m: dv_n = (q~_n . k~_n) dO_n and, with no rotation,
    dq_n = (dO_n . v_n) k_n, dk_n = (dO_n . v_n) q_n."""
    q, k, v, do = _inputs(1, 1, 9, 4, 3, 3)
    dq, dkk, dvv = oracle.backward(q, k, v, do, [0.0])
    s = (q * k).sum(-1, keepdims=True)
    t = (do * v).sum(-1, keepdims=True)
    assert np.allclose(dvv, s * do, rtol=1e-13, atol=1e-13)
    assert np.allclose(dq, t * k, rtol=1e-13, atol=1e-13)
    assert np.allclose(dkk, t * q, rtol=1e-13, atol=1e-13)


def test_rows_match_full():
    B, H, L, dk, dv = 2, 2, 21, 6, 5
    q, k, v, do = _inputs(B, H, L, dk, dv, 4)
    full = dict(zip("qkv", oracle.backward(q, k, v, do, GAMMA, THETA, 2)))
    idx = [(0, 0, 0), (1, 1, L - 1), (0, 1, 10), (1, 0, 5)]
    for w in "qkv":
        got = oracle.backward_rows(q, k, v, do, GAMMA, w, idx, THETA, 2)
        ref = np.stack([full[w][b, h, n] for b, h, n in idx])
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), w


@pytest.mark.parametrize("L,pos0,rot", [(1, 0, True), (29, 7, True), (40, 0, False)])
def test_recurrent_adjoint_matches_double_sum(L, pos0, rot):
    """The adjoint of the recurrent form (forward sweep of the state for dq, reverse
    sweep for dk and dv) and the double sum over n >= m are two independent
    derivations of the same gradients; they agree to rounding, including a head
    with gamma = 0 (only n = m) and one with gamma = 1 (no decay)."""
    B, H, dk, dv = 2, 3, 6, 5
    q, k, v, do = _inputs(B, H, L, dk, dv, 10 + L)
    g = np.array([0.0, 1.0, 0.83])
    th = THETA if rot else None
    ref = oracle.backward(q, k, v, do, g, th, pos0)
    got = oracle.backward_recurrent(q, k, v, do, g, th, pos0)
    for name, a, b in zip("qkv", got, ref):
        err = np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)
        assert err < 1e-12, f"d{name}: {err:.2e}"
