"""fp64 CPU oracle for multi-scale retention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.

Every function takes numpy arrays or torch tensors (any float dtype; they are
upcast exactly to fp64) and returns fp64 numpy arrays.  The arithmetic lives in
``oracle.c`` (plain loops) and, for the multi-scale retention layer, in plain
numpy glue below.  Pages followed (cited by title and section):

* "Retentive Network: A Successor to Transformer for Large Language Models"
  (paper summary on blog.csdn.net), Sec. 2.1 "Retention" -- the
  scalar-gamma form and its parallel (1), recurrent (2) and chunkwise (3)
  representations; Sec. 2.2 "Gated Multi-Scale Retention".
* "RetNet dual-mode hands-on manual" (lanjinlin.com.cn), Sec. 1 (decay
  matrix D) and Sec. 3.1 (parallel/recurrent equivalence).

All functions are pinned by ``tests/test_oracle_pins.py`` and
``tests/test_oracle_msr.py``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_L = ctypes.POINTER(ctypes.c_long)
_l = ctypes.c_long
_ll = ctypes.c_longlong


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sigs = {
        "orc_rotate": [_D, _D, _l, _l, _l, _D, _ll],
        "orc_parallel": [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _ll],
        "orc_parallel_complex": [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _ll],
        "orc_recurrent": [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _ll, _D, _D],
        "orc_chunkwise": [_D, _D, _D, _D, _l, _l, _l, _l, _l, _l, _D, _D, _ll, _D, _D],
        "orc_rows": [_D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _ll, _D, _L, _l, _D],
        "orc_state_entries": [_D, _D, _l, _l, _l, _l, _l, _D, _D, _ll, _D, _L, _l, _D],
        "orc_groupnorm": [_D, _l, _l, ctypes.c_double],
        "orc_matmul_nt": [_D, _D, _D, _l, _l, _l],
        "orc_swish": [_D, _l],
        "orc_layernorm": [_D, _l, _l, ctypes.c_double],
        "orc_gelu": [_D, _l],
        "orc_backward": [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _ll, _D, _D, _D],
        "orc_backward_recurrent": [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _ll, _D, _D, _D],
        "orc_backward_rows": [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _ll, ctypes.c_int, _L, _l, _D],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    _lib = lib
    return lib


def as_f64(x):
    """Exact upcast of a numpy array / torch tensor to a C-contiguous fp64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (bf16 has no numpy dtype: go via fp32, exact)
        import torch
        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def _theta(theta):
    return None if theta is None else as_f64(theta)


def _dims(q, v):
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert v.shape[:3] == (B, H, L)
    return B, H, L, dk, dv


def rotate(x, theta, pos0=0):
    """xPOS rotation of x [..., L, dk] at positions pos0 + n."""
    x = as_f64(x)
    out = np.empty_like(x)
    L, dk = x.shape[-2], x.shape[-1]
    BH = int(np.prod(x.shape[:-2])) if x.ndim > 2 else 1
    th = _theta(theta)
    _load().orc_rotate(_p(x), _p(out), BH, L, dk, _p(th), pos0)
    return out


def parallel(q, k, v, gamma, theta=None, pos0=0):
    """Parallel form (Q K^T (.) D) V as the literal double sum."""
    q, k, v, g = as_f64(q), as_f64(k), as_f64(v), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    o = np.empty((B, H, L, dv))
    _load().orc_parallel(_p(q), _p(k), _p(v), _p(o), B, H, L, dk, dv, _p(g), _p(_theta(theta)), pos0)
    return o


def parallel_complex(q, k, v, gamma, theta=None, pos0=0):
    """Complex-number transcription of the conjugate-transpose form (pins rotate)."""
    q, k, v, g = as_f64(q), as_f64(k), as_f64(v), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    o = np.empty((B, H, L, dv))
    _load().orc_parallel_complex(_p(q), _p(k), _p(v), _p(o), B, H, L, dk, dv, _p(g),
                                 _p(_theta(theta)), pos0)
    return o


def recurrent(q, k, v, gamma, theta=None, pos0=0, s_in=None):
    """Recurrent form; returns (o, final state)."""
    q, k, v, g = as_f64(q), as_f64(k), as_f64(v), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    o = np.empty((B, H, L, dv))
    s_out = np.empty((B, H, dk, dv))
    s_in = as_f64(s_in)
    _load().orc_recurrent(_p(q), _p(k), _p(v), _p(o), B, H, L, dk, dv, _p(g), _p(_theta(theta)),
                          pos0, _p(s_in), _p(s_out))
    return o, s_out


def chunkwise(q, k, v, gamma, chunk, theta=None, pos0=0, s_in=None):
    """Chunkwise recurrent form with chunk size `chunk` (last chunk may be short)."""
    q, k, v, g = as_f64(q), as_f64(k), as_f64(v), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    assert chunk >= 1
    o = np.empty((B, H, L, dv))
    s_out = np.empty((B, H, dk, dv))
    s_in = as_f64(s_in)
    _load().orc_chunkwise(_p(q), _p(k), _p(v), _p(o), B, H, L, dk, dv, chunk, _p(g),
                          _p(_theta(theta)), pos0, _p(s_in), _p(s_out))
    return o, s_out


def rows(q, k, v, gamma, idx, theta=None, pos0=0, s_in=None):
    """Output rows o[b, h, n, :] for each (b, h, n) in idx, by the defining sum."""
    q, k, v, g = as_f64(q), as_f64(k), as_f64(v), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 3))
    out = np.empty((ix.shape[0], dv))
    s_in = as_f64(s_in)
    _load().orc_rows(_p(q), _p(k), _p(v), B, H, L, dk, dv, _p(g), _p(_theta(theta)), pos0,
                     _p(s_in), ix.ctypes.data_as(_L), ix.shape[0], _p(out))
    return out


def state_entries(k, v, gamma, idx, theta=None, pos0=0, s_in=None):
    """Final-state entries S[b, h, a, c] for each (b, h, a, c) in idx."""
    k, v, g = as_f64(k), as_f64(v), as_f64(gamma)
    B, H, L, dk, dv = _dims(k, v)
    ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 4))
    out = np.empty(ix.shape[0])
    s_in = as_f64(s_in)
    _load().orc_state_entries(_p(k), _p(v), B, H, L, dk, dv, _p(g), _p(_theta(theta)), pos0,
                              _p(s_in), ix.ctypes.data_as(_L), ix.shape[0], _p(out))
    return out


def backward(q, k, v, do, gamma, theta=None, pos0=0):
    """Gradients (dq, dk, dv) of the defining sum (no GroupNorm) for output gradient do."""
    q, k, v, do, g = as_f64(q), as_f64(k), as_f64(v), as_f64(do), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    dq, dkk, dvv = np.empty((B, H, L, dk)), np.empty((B, H, L, dk)), np.empty((B, H, L, dv))
    _load().orc_backward(_p(q), _p(k), _p(v), _p(do), B, H, L, dk, dv, _p(g), _p(_theta(theta)), pos0,
                         _p(dq), _p(dkk), _p(dvv))
    return dq, dkk, dvv


def backward_recurrent(q, k, v, do, gamma, theta=None, pos0=0):
    """The same gradients by the adjoint of the recurrent form (O(L dk dv) per
    (b, h)): a forward sweep of the state for dq, a reverse sweep for dk and dv."""
    q, k, v, do, g = as_f64(q), as_f64(k), as_f64(v), as_f64(do), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    dq, dkk, dvv = np.empty((B, H, L, dk)), np.empty((B, H, L, dk)), np.empty((B, H, L, dv))
    _load().orc_backward_recurrent(_p(q), _p(k), _p(v), _p(do), B, H, L, dk, dv, _p(g), _p(_theta(theta)), pos0,
                                   _p(dq), _p(dkk), _p(dvv))
    return dq, dkk, dvv


def backward_rows(q, k, v, do, gamma, which, idx, theta=None, pos0=0):
    """Rows of one gradient ('q', 'k' or 'v') at each (b, h, n) in idx."""
    q, k, v, do, g = as_f64(q), as_f64(k), as_f64(v), as_f64(do), as_f64(gamma)
    B, H, L, dk, dv = _dims(q, v)
    w = {"q": 0, "k": 1, "v": 2}[which]
    ix = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 3))
    out = np.empty((ix.shape[0], dv if w == 2 else dk))
    _load().orc_backward_rows(_p(q), _p(k), _p(v), _p(do), B, H, L, dk, dv, _p(g), _p(_theta(theta)), pos0,
                              w, ix.ctypes.data_as(_L), ix.shape[0], _p(out))
    return out


def groupnorm(x, eps):
    """Per-(token, head) GroupNorm over the last axis, no affine."""
    x = as_f64(x).copy()
    dv = x.shape[-1]
    _load().orc_groupnorm(_p(x), x.size // dv, dv, float(eps))
    return x


def matmul_nt(x, w):
    """x [M, K] times w^T, w stored [N, K]."""
    x, w = as_f64(x), as_f64(w)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    y = np.empty((M, N))
    _load().orc_matmul_nt(_p(x), _p(w), _p(y), M, N, K)
    return y


def swish(x):
    x = as_f64(x).copy()
    _load().orc_swish(_p(x), x.size)
    return x


def layernorm(x, eps):
    """Per-row LayerNorm over the last axis, no affine."""
    x = as_f64(x).copy()
    _load().orc_layernorm(_p(x), x.size // x.shape[-1], x.shape[-1], float(eps))
    return x


def gelu(x):
    """Exact gelu, x * Phi(x)."""
    x = as_f64(x).copy()
    _load().orc_gelu(_p(x), x.size)
    return x


def retnet_block(x, w_q, w_k, w_v, w_g, w_o, w_1, w_2, H, dk, dv, gamma, theta=None, pos0=0, gn_eps=1e-5,
                 ln_eps=1e-5, tokens=None):
    """The pre-LN residual block around the gated layer (P2, block equations):
        Y = MSR(LN(X)) + X,   X' = FFN(LN(Y)) + Y,   FFN(Z) = gelu(Z W_1) W_2
    with weights stored [out, in] (w_1 [d_ffn, d_model], w_2 [d_model, d_ffn]).
    Returns [B, L, d_model], or only the rows in `tokens` ((b, l) pairs): every
    step after the layer acts on one row at a time."""
    x = as_f64(x)
    B, L, dm = x.shape
    h1 = layernorm(x, ln_eps)
    if tokens is None:
        y = msr_layer(h1, w_q, w_k, w_v, w_g, w_o, H, dk, dv, gamma, theta, pos0, gn_eps) + x
        y = y.reshape(B * L, dm)
    else:
        toks = [tuple(t) for t in tokens]
        y = msr_layer(h1, w_q, w_k, w_v, w_g, w_o, H, dk, dv, gamma, theta, pos0, gn_eps, tokens=toks)
        y = y + np.stack([x[b, l] for b, l in toks])
    f = matmul_nt(gelu(matmul_nt(layernorm(y, ln_eps), w_1)), w_2)
    out = y + f
    return out.reshape(B, L, dm) if tokens is None else out


def msr_layer(x, w_q, w_k, w_v, w_g, w_o, H, dk, dv, gamma, theta=None, pos0=0, gn_eps=1e-5,
              tokens=None):
    """Gated multi-scale retention layer (P2 Sec. 2.2):
        Q = X W_Q, K = X W_K, V = X W_V  (head h = column block h)
        head_h = Retention(X, gamma_h)
        Y = GroupNorm_h(Concat(heads));   MSR(X) = (swish(X W_G) (.) Y) W_O
    Weights are stored transposed, [out, in] (row j holds output column j).
    x: [B, L, d_model].  Returns [B, L, d_model], or -- if `tokens` (a list of
    (b, l)) is given -- only those rows, computed one by one from the defining
    sum (K and V of the batches involved are projected in full)."""
    x = as_f64(x)
    B, L, dm = x.shape
    g = as_f64(gamma)
    if tokens is None:
        X = x.reshape(B * L, dm)
        q = matmul_nt(X, w_q).reshape(B, L, H, dk).transpose(0, 2, 1, 3)
        k = matmul_nt(X, w_k).reshape(B, L, H, dk).transpose(0, 2, 1, 3)
        v = matmul_nt(X, w_v).reshape(B, L, H, dv).transpose(0, 2, 1, 3)
        gate = swish(matmul_nt(X, w_g))                         # [B*L, H*dv]
        o, _ = recurrent(q, k, v, g, theta, pos0)                # [B, H, L, dv]
        y = groupnorm(o, gn_eps).transpose(0, 2, 1, 3).reshape(B * L, H * dv)
        z = gate * y
        return matmul_nt(z, w_o).reshape(B, L, -1)
    out = []
    toks = [tuple(t) for t in tokens]
    for b in sorted({t[0] for t in toks}):
        X = x[b]
        k = matmul_nt(X, w_k).reshape(L, H, dk).transpose(1, 0, 2)[None]
        v = matmul_nt(X, w_v).reshape(L, H, dv).transpose(1, 0, 2)[None]
        ls = [t[1] for t in toks if t[0] == b]
        Xs = X[ls]
        qs = matmul_nt(Xs, w_q).reshape(len(ls), H, dk)
        gate = swish(matmul_nt(Xs, w_g))                         # [n, H*dv]
        # place the selected query rows into a full-size q so rows() sees positions
        q = np.zeros((1, H, L, dk))
        for i, l in enumerate(ls):
            q[0, :, l, :] = qs[i]
        idx = [(0, h, l) for l in ls for h in range(H)]
        o = rows(q, k, v, g, idx, theta, pos0).reshape(len(ls), H, dv)
        y = groupnorm(o, gn_eps).reshape(len(ls), H * dv)
        z = gate * y
        yo = matmul_nt(z, w_o)
        for i, l in enumerate(ls):
            out.append(((b, l), yo[i]))
    order = {t: i for i, t in enumerate(toks)}
    res = np.empty((len(toks), out[0][1].shape[0]))
    for t, row in out:
        res[order[t]] = row
    return res
