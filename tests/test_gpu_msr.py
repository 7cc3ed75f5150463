"""GPU parity of the gated multi-scale retention layer (C ABI msr_layer_fwd) against
the fp64 oracle ("Retentive Network" paper summary, Sec. 2.2): projections, xPOS,
per-head gamma, chunkwise retention, GroupNorm, swish gate, output projection.
Ragged token counts (B*L not a multiple of the 128-row GEMM tile, L not a
multiple of the chunk) are included."""
import numpy as np
import pytest
import torch

import oracle
import retentive_network_scale_amd as rn
from tests import _tol
from workloads import MSRWorkload, multiscale_gamma, randn, rotation_theta

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, L, dm, H, dk, dv, seed, w_std=0.05):
    bf = torch.bfloat16
    x = randn((B, L, dm), seed, 1.0, bf)
    w = [randn((H * dk, dm), seed + 3, w_std, bf), randn((H * dk, dm), seed + 4, w_std, bf),
         randn((H * dv, dm), seed + 5, w_std, bf), randn((H * dv, dm), seed + 6, w_std, bf),
         randn((dm, H * dv), seed + 7, w_std, bf)]
    return x, w


@pytest.mark.parametrize("B,L,dm,H,dk,dv,chunk", [
    (2, 300, 256, 2, 64, 128, 64),
    (1, 257, 256, 2, 128, 256, 100),
    (1, 200, 512, 2, 256, 512, 128),
])
def test_msr_layer_small(B, L, dm, H, dk, dv, chunk):
    x, (wq, wk, wv, wg, wo) = _inputs(B, L, dm, H, dk, dv, 600 + dk)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    ref = oracle.msr_layer(x, wq, wk, wv, wg, wo, H, dk, dv, g, th, pos0=3, gn_eps=1e-5)
    y = rn.msr_layer_fwd(*[t.to(DEV) for t in (x, wq, wk, wv, wg, wo)], H, dk, dv, chunk, g, th, pos0=3,
                         gn_eps=1e-5)
    torch.cuda.synchronize()
    _tol.assert_bf16(y, ref, slice_dims=0, what="msr layer")
    _tol.assert_bf16(y, ref, slice_dims=1, what="msr layer per batch")


def test_msr_zero_gate():
    """W_G = 0 gives swish(0) = 0 and an all-zero output."""
    B, L, dm, H, dk, dv = 1, 130, 256, 2, 64, 128
    x, (wq, wk, wv, wg, wo) = _inputs(B, L, dm, H, dk, dv, 700)
    g = multiscale_gamma(H)
    y = rn.msr_layer_fwd(*[t.to(DEV) for t in (x, wq, wk, wv, torch.zeros_like(wg), wo)], H, dk, dv, 64, g)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0


def test_msr_full_size_sampled():
    """The MSR layer workload (X [4,4096,2048], 8 heads, dk 256, dv 512, chunk 512) at full size;
    sampled output rows checked against the oracle, which computes each from the
    defining sums (only the tokens up to the latest sampled one are needed: the
    layer is causal)."""
    wl = MSRWorkload()
    x, wq, wk, wv, wg, wo = wl.inputs()
    g, th = wl.gamma(), wl.theta()
    dev = [t.to(DEV) for t in (x, wq, wk, wv, wg, wo)]
    y = rn.msr_layer_fwd(*dev, wl.H, wl.dk, wl.dv, wl.chunk, g, th, pos0=0, gn_eps=wl.gn_eps)
    torch.cuda.synchronize()
    yc = y.float().cpu().numpy()
    samples = {0: [0, 1, 511, 512, 1023], 3: [7, 600]}
    for b, ls in samples.items():
        lmax = max(ls) + 1
        ref = oracle.msr_layer(x[b:b + 1, :lmax], wq, wk, wv, wg, wo, wl.H, wl.dk, wl.dv, g, th, pos0=0,
                               gn_eps=wl.gn_eps, tokens=[(0, l) for l in ls])
        got = np.stack([yc[b, l] for l in ls])
        _tol.assert_bf16(got, ref, slice_dims=0, what=f"msr full-size batch {b}")
