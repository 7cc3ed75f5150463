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
                                                     (128, 256, 200, 64, True, 100000),
                                                     (128, 256, 389, 128, True, 5), (128, 256, 1100, 256, False, 0)])
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


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128), (128, 256)])
@pytest.mark.parametrize("chunk", [192, 256])
def test_backward_chunks_split_inside_segments(dk, dv, chunk):
    """A caller's chunk that is a multiple of 64 is walked in 64-token chunks inside
    the caller's segments; the dk sum then reads the dv sum's segment states.
    Two sequences, three heads, a ragged length spanning several segments, bf16
    with rotation, against the oracle's gradients."""
    B, H, L = 2, 3, 450
    q, k, v, do = _inputs(B, H, L, dk, dv, 1500 + dk + dv + chunk, torch.bfloat16)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, chunk, th, pos0=9,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, do, g, th, 9)
    for name, a, b in zip("qkv", got, ref):
        _tol.assert_bf16(a, b, slice_dims=2, what=f"d{name} dk={dk} dv={dv} chunk={chunk}")


def test_backward_32k_sampled_rows():
    """The long-context workload (B1 H8 L32768 dk128 dv256, chunk 256) with a seeded
    output gradient: ten sampled rows of dq, dk and dv in each of three heads (the
    fastest and slowest decay and one between) against the oracle's sums, compared
    per head -- the rows of one head form one slice of the tolerance metric."""
    wl = CHUNKWISE_32K
    q, k, v = wl.qkv()
    do = randn((wl.B, wl.H, wl.L, wl.dv), 3009, 1.0, torch.bfloat16)
    g, th = wl.gamma(), wl.theta()
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, wl.chunk, th)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    heads, per = (0, 3, 7), 10
    fixed = [0, 255, 256, 16384, wl.L - 1]
    idx = [(0, h, n) for h in heads for n in fixed + [int(x) for x in rng.integers(wl.L, size=per - len(fixed))]]
    qn, kn, vn, don = (oracle.as_f64(t) for t in (q, k, v, do))
    for name, t in zip("qkv", got):
        ref = oracle.backward_rows(qn, kn, vn, don, g, name, idx, th).reshape(len(heads), per, -1)
        gotr = np.stack([t[b, h, n].float().cpu().numpy() for b, h, n in idx]).reshape(len(heads), per, -1)
        _tol.assert_bf16(gotr, ref, slice_dims=1, what=f"d{name} sampled rows, per head")


@pytest.mark.parametrize("dk,dv,B,H,L,chunk,rot,pos0", [(128, 256, 1, 4, 513, 256, True, 3),
                                                         (128, 256, 2, 8, 2000, 192, True, 7),
                                                         (128, 256, 4, 8, 4000, 128, True, 0),
                                                         (64, 128, 2, 8, 1500, 128, False, 0),
                                                         (128, 128, 1, 4, 700, 64, True, 11)])
def test_backward_with_forward_states(dk, dv, B, H, L, chunk, rot, pos0):
    """The backward that reuses the forward call's segment states for the dq sum
    (retention_chunkwise_bwd_saved): the forward runs first on the same inputs and
    its workspace is handed over.  Gradients against the oracle, and against the
    self-contained backward.  Shapes give one and several segments per head, a
    ragged last chunk, several chunks per segment and a chunk split into 64-token
    pieces inside segments.  The reference is the oracle's recurrent adjoint."""
    q, k, v, do = _inputs(B, H, L, dk, dv, 1300 + dk + L, torch.bfloat16)
    g, th = multiscale_gamma(H), (rotation_theta(dk) if rot else None)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    fws = torch.empty(rn.retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk), dtype=torch.uint8, device=DEV)
    rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=pos0, workspace=fws)
    got = rn.retention_chunkwise_bwd(qd, kd, vd, dod, g, chunk, th, pos0=pos0, out_dtype=torch.float32,
                                     fwd_workspace=fws)
    own = rn.retention_chunkwise_bwd(qd, kd, vd, dod, g, chunk, th, pos0=pos0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward_recurrent(q, k, v, do, g, th, pos0)
    for name, a, b, c in zip("qkv", got, ref, own):
        _tol.assert_bf16(a, b, slice_dims=2, what=f"d{name} with forward states")
        _tol.assert_bf16(a, c.double().cpu().numpy(), slice_dims=2, what=f"d{name} vs own states")


def test_backward_32k_with_forward_states_sampled_rows():
    """The long-context workload's backward with the forward's states: ten sampled
    rows of dq (the sum that reads them) in each of three heads, per head."""
    wl = CHUNKWISE_32K
    q, k, v = wl.qkv()
    do = randn((wl.B, wl.H, wl.L, wl.dv), 3009, 1.0, torch.bfloat16)
    g, th = wl.gamma(), wl.theta()
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    fws = torch.empty(rn.retention_chunkwise_workspace_bytes(wl.B, wl.H, wl.L, wl.dk, wl.dv, wl.chunk),
                      dtype=torch.uint8, device=DEV)
    rn.retention_chunkwise(qd, kd, vd, g, wl.chunk, th, workspace=fws)
    got = rn.retention_chunkwise_bwd(qd, kd, vd, dod, g, wl.chunk, th, fwd_workspace=fws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    heads, per = (0, 3, 7), 10
    fixed = [0, 1023, 1024, 20000, wl.L - 1]
    idx = [(0, h, n) for h in heads for n in fixed + [int(x) for x in rng.integers(wl.L, size=per - len(fixed))]]
    qn, kn, vn, don = (oracle.as_f64(t) for t in (q, k, v, do))
    ref = oracle.backward_rows(qn, kn, vn, don, g, "q", idx, th).reshape(len(heads), per, -1)
    gotr = np.stack([got[0][b, h, n].float().cpu().numpy() for b, h, n in idx]).reshape(len(heads), per, -1)
    _tol.assert_bf16(gotr, ref, slice_dims=1, what="dq sampled rows with forward states, per head")
