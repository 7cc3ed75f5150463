"""GPU parity of the chunkwise backward (gradients of retention with respect to q,
k and v; "Retentive Network" paper summary, Sec. 2.1) against the fp64 oracle:
fp32 on the vector path, bf16 on the MFMA kernels, ragged lengths and chunks, and
sampled rows at the long-context workload size."""
import numpy as np
import pytest
import torch

import oracle
import retentive_network_scale_amd as rn
from tests import _tol
from workloads import CHUNKWISE_32K, multiscale_gamma, randn, rotation_theta

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, H, L, dk, dv, seed, dtype):
    s = dk ** -0.5
    return (randn((B, H, L, dk), seed, s, dtype), randn((B, H, L, dk), seed + 1, s, dtype),
            randn((B, H, L, dv), seed + 2, 1.0, dtype), randn((B, H, L, dv), seed + 3, 1.0, dtype))


@pytest.mark.parametrize("L,chunk,pos0,rot", [(64, 16, 0, True), (77, 16, 5, True), (50, 64, 0, False)])
def test_backward_fp32(L, chunk, pos0, rot):
    B, H, dk, dv = 2, 2, 16, 24
    q, k, v, do = _inputs(B, H, L, dk, dv, 1100 + L, torch.float32)
    g, th = multiscale_gamma(H), (rotation_theta(dk) if rot else None)
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, chunk, th, pos0=pos0)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, do, g, th, pos0)
    for name, a, b in zip("qkv", got, ref):
        _tol.assert_fp32(a, b, slice_dims=2, what=f"d{name}")


@pytest.mark.parametrize("dk,dv,L,chunk,rot,pos0", [(128, 256, 300, 64, True, 3), (128, 256, 513, 256, True, 3),
                                                     (64, 128, 200, 100, True, 3), (128, 128, 260, 128, True, 3),
                                                     (64, 128, 130, 64, False, 0),
                                                     (128, 256, 200, 64, True, 100000)])
def test_backward_bf16(dk, dv, L, chunk, rot, pos0):
    """bf16 inputs on the MFMA kernels, which rotate on load (value rows at their
    own positions, reversed queries and keys by -theta): with and without
    rotation, and at a large starting position."""
    B, H = 1, 4
    q, k, v, do = _inputs(B, H, L, dk, dv, 1200 + dk + L, torch.bfloat16)
    g, th = multiscale_gamma(H), (rotation_theta(dk) if rot else None)
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, chunk, th, pos0=pos0,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, do, g, th, pos0)
    for name, a, b in zip("qkv", got, ref):
        _tol.assert_bf16(a, b, slice_dims=2, what=f"d{name}")


def test_backward_32k_sampled_rows():
    """The long-context workload (B1 H8 L32768 dk128 dv256, chunk 256) with a seeded
    output gradient: sampled rows of dq, dk and dv against the oracle's sums.  The
    sampled rows are compared as one set, normalised as a (b, h) slice is: a row
    whose sum has a single term (dv of the last token is (q~ . k~) dO) carries the
    relative rounding error of one bf16 score, which alone can exceed the bar when
    that score is small."""
    wl = CHUNKWISE_32K
    q, k, v = wl.qkv()
    do = randn((wl.B, wl.H, wl.L, wl.dv), 3009, 1.0, torch.bfloat16)
    g, th = wl.gamma(), wl.theta()
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, wl.chunk, th)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    idx = [(0, 0, 0), (0, 7, wl.L - 1), (0, 3, 255), (0, 3, 256), (0, 5, 16384)]
    idx += [(0, int(rng.integers(wl.H)), int(rng.integers(wl.L))) for _ in range(5)]
    qn, kn, vn, don = (oracle.as_f64(t) for t in (q, k, v, do))
    for name, t in zip("qkv", got):
        ref = oracle.backward_rows(qn, kn, vn, don, g, name, idx, th)
        gotr = np.stack([t[b, h, n].float().cpu().numpy() for b, h, n in idx])
        _tol.assert_bf16(gotr, ref, slice_dims=0, what=f"d{name} sampled rows")
