"""GPU parity of the bf16 MFMA retention kernels against the fp64 oracle (C ABI).

Shapes span several 64-token tiles with ragged tails, every supported head-size
pair, rotation on/off, GroupNorm on/off, fp32 and bf16 outputs, chunk sizes that
do and do not divide L, several chunks per segment (state carried inside a
workgroup) and several segments (state carried by the scan), incoming state and
aliased state_in/state_out.  bf16 bar: rel-L2 <= 2e-2, unit-normalised max-abs
<= 5e-2, per (b, h) slice.
"""
import numpy as np
import pytest
import torch

import oracle
import retentive_network_scale_amd as rn
from tests import _tol
from workloads import multiscale_gamma, randn, rotation_theta

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAIRS = [(64, 128), (128, 128), (128, 256), (256, 128), (256, 256), (256, 512)]


def _qkv(B, H, L, dk, dv, seed):
    s = 1.0 / np.sqrt(dk)
    return (randn((B, H, L, dk), seed, s, torch.bfloat16), randn((B, H, L, dk), seed + 1, s, torch.bfloat16),
            randn((B, H, L, dv), seed + 2, 1.0, torch.bfloat16))


def _gpu(*ts):
    return [t.to(DEV) for t in ts]


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("rot,gn,odt", [(True, None, torch.bfloat16), (False, 1e-5, torch.float32),
                                        (True, 1e-5, torch.bfloat16)])
def test_parallel_mfma(dk, dv, rot, gn, odt):
    B, H, L = 2, 3, 200
    q, k, v = _qkv(B, H, L, dk, dv, 100 + dk + dv)
    g = multiscale_gamma(H)
    th = rotation_theta(dk) if rot else None
    ref = oracle.parallel(q, k, v, g, th, pos0=37)
    if gn is not None:
        ref = oracle.groupnorm(ref, gn)
    o = rn.retention_parallel(*_gpu(q, k, v), g, th, pos0=37, gn_eps=gn, out_dtype=odt)
    torch.cuda.synchronize()
    assert o.dtype == odt
    _tol.assert_bf16(o, ref, what=f"parallel dk={dk} dv={dv} rot={rot} gn={gn}")


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("L,chunk", [(300, 64), (300, 100), (130, 256)])
def test_chunkwise_mfma(dk, dv, L, chunk):
    B, H = 1, 2
    q, k, v = _qkv(B, H, L, dk, dv, 200 + dk + dv + chunk)
    s0 = randn((B, H, dk, dv), 7, 0.5)
    g = torch.tensor([0.97, 0.5], dtype=torch.float32)
    th = rotation_theta(dk)
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=11, s_in=s0)
    qd, kd, vd, sd = _gpu(q, k, v, s0)
    o, s = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=11, state_in=sd, state_out=True,
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    _tol.assert_bf16(o, ref_o, what=f"chunkwise dk={dk} dv={dv} L={L} chunk={chunk}")
    _tol.assert_bf16(s, ref_s, what="final state")


@pytest.mark.parametrize("dk,dv,chunk,rot,gn,odt", [
    (128, 256, 256, True, None, torch.bfloat16), (128, 256, 192, False, 1e-5, torch.bfloat16),
    (128, 256, 256, False, 1e-5, torch.float32), (128, 128, 256, True, None, torch.float32),
    (64, 128, 192, True, None, torch.bfloat16), (128, 256, 160, True, None, torch.bfloat16)])
def test_chunkwise_three_and_four_block_chunks(dk, dv, chunk, rot, gn, odt):
    """Chunks of three or four 64-token blocks (the chunk's first V block stays in
    LDS beside its keys): segments of two chunks, a ragged last chunk (4000 tokens),
    an incoming state, GroupNorm without rotation (the partial sums share the score
    tile), bf16 (staged) and fp32 outputs."""
    B, H, L = 4, 8, 4000
    q, k, v = _qkv(B, H, L, dk, dv, 500 + dk + dv + chunk)
    s0 = randn((B, H, dk, dv), 9, 0.3)
    g = multiscale_gamma(H)
    th = rotation_theta(dk) if rot else None
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=3, s_in=s0)
    if gn is not None:
        ref_o = oracle.groupnorm(ref_o, gn)
    qd, kd, vd, sd = _gpu(q, k, v, s0)
    o, s = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=3, state_in=sd, state_out=True, gn_eps=gn,
                                  out_dtype=odt)
    torch.cuda.synchronize()
    _tol.assert_bf16(o, ref_o, what=f"chunkwise dk={dk} dv={dv} chunk={chunk} rot={rot} gn={gn}")
    _tol.assert_bf16(s, ref_s, what="final state")


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 256), (256, 512)])
def test_chunkwise_segments_and_carry(dk, dv):
    """B*H = 32 units so that every head gets several segments of several chunks
    (state carried in registers inside a segment and by the scan across them);
    GroupNorm on; state_out aliases state_in."""
    B, H, L, chunk = 4, 8, 1100, 64
    q, k, v = _qkv(B, H, L, dk, dv, 300 + dk)
    s0 = randn((B, H, dk, dv), 8, 0.3)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=5, s_in=s0)
    ref_gn = oracle.groupnorm(ref_o, 1e-5)
    qd, kd, vd, sd = _gpu(q, k, v, s0)
    o, s = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=5, state_in=sd, state_out=sd, gn_eps=1e-5)
    torch.cuda.synchronize()
    _tol.assert_bf16(o, ref_gn, what="chunkwise+GN")
    _tol.assert_bf16(sd, ref_s, what="aliased final state")


def test_chunk_size_independence_gpu():
    """Outputs and the final state agree across chunk sizes (and with the parallel kernel)."""
    B, H, L, dk, dv = 1, 4, 512, 128, 256
    q, k, v = _qkv(B, H, L, dk, dv, 400)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    qd, kd, vd = _gpu(q, k, v)
    ref = oracle.recurrent(q, k, v, g, th)[0]
    par = rn.retention_parallel(qd, kd, vd, g, th, out_dtype=torch.float32)
    _tol.assert_bf16(par, ref, what="parallel")
    states = []
    for chunk in (64, 128, 256, 512, 1000):
        o, s = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, state_out=True, out_dtype=torch.float32)
        _tol.assert_bf16(o, ref, what=f"chunk {chunk}")
        states.append(s)
    torch.cuda.synchronize()
    for s in states[1:]:
        _tol.assert_bf16(s, states[0], what="state vs chunk 64")


def test_mask_extraction_mfma():
    """theta = 0, q = k = e_0, v_m = e_m (exact in bf16): o[n][m] = D[n][m] up to the
    bf16 rounding of the decayed scores."""
    L, dk, dv = 128, 64, 128
    q = torch.zeros((1, 1, L, dk), dtype=torch.bfloat16); q[..., 0] = 1.0
    v = torch.zeros((1, 1, L, dv), dtype=torch.bfloat16)
    v[0, 0, torch.arange(L), torch.arange(L)] = 1.0
    gm = 1 - 2 ** -5
    o = rn.retention_parallel(*_gpu(q, q.clone(), v), [gm], out_dtype=torch.float32)
    oc, _ = rn.retention_chunkwise(*_gpu(q, q.clone(), v), [gm], 64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    n, m = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    D = np.where(n >= m, gm ** np.maximum(n - m, 0), 0.0)
    for out in (o, oc):
        got = out[0, 0].double().cpu().numpy()
        assert np.all(got[n < m] == 0.0)
        assert np.all(got[n == m] == 1.0)
        assert np.abs(got - D).max() <= 2 ** -8


def test_gamma_edges_mfma():
    """gamma = 0 (identity decay) and gamma = 1 (causal linear attention) through the MFMA path."""
    B, H, L, dk, dv = 1, 2, 150, 64, 128
    q, k, v = _qkv(B, H, L, dk, dv, 500)
    g = torch.tensor([0.0, 1.0])
    ref = oracle.parallel(q, k, v, g)
    qd, kd, vd = _gpu(q, k, v)
    _tol.assert_bf16(rn.retention_parallel(qd, kd, vd, g, out_dtype=torch.float32), ref, what="parallel")
    o, _ = rn.retention_chunkwise(qd, kd, vd, g, 64, out_dtype=torch.float32)
    _tol.assert_bf16(o, ref, what="chunkwise")


def test_chunkwise_gn_rot_graph_replay():
    """The chunkwise path for large states with GroupNorm and rotation runs its
    hi+lo first query blocks on a second stream forked from the caller's and
    joined back.  Captured in a graph and replayed with new inputs, eager work
    and synchronisations between replays: every replay equals the eager call on
    the same inputs, bit for bit."""
    B, H, L, dk, dv, chunk = 2, 2, 320, 256, 512, 128
    g, th = multiscale_gamma(H), rotation_theta(dk)
    inputs = [_gpu(*_qkv(B, H, L, dk, dv, 700 + 10 * i)) for i in range(3)]
    wsb = rn.retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    eager = [rn.retention_chunkwise(q, k, v, g, chunk, th, gn_eps=1e-5, workspace=ws)[0] for q, k, v in inputs]
    qs, ks, vs = (torch.empty_like(t) for t in inputs[0])
    out = torch.empty((B, H, L, dv), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        rn.retention_chunkwise(qs, ks, vs, g, chunk, th, gn_eps=1e-5, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rn.retention_chunkwise(qs, ks, vs, g, chunk, th, gn_eps=1e-5, out=out, workspace=ws)
    torch.cuda.synchronize()
    for i, (q, k, v) in enumerate(inputs):
        qs.copy_(q)
        ks.copy_(k)
        vs.copy_(v)
        _ = (q.float() * 2).sum()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[i]), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("dk,dv,L,chunk", [(256, 512, 300, 4096), (128, 256, 200, 2 ** 31 - 1)])
def test_chunk_longer_than_sequence(dk, dv, L, chunk):
    """A chunk longer than the sequence is one chunk (the parallel form): the
    (256, 512) pair takes the query-block path, (128, 256) the segment path."""
    B, H = 1, 2
    q, k, v = _qkv(B, H, L, dk, dv, 400 + dk)
    g, th = torch.tensor([0.97, 0.6], dtype=torch.float32), rotation_theta(dk)
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=3)
    o, s = rn.retention_chunkwise(*_gpu(q, k, v), g, chunk, th, pos0=3, state_out=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _tol.assert_bf16(o, ref_o, what=f"chunk {chunk} > L={L}")
    _tol.assert_bf16(s, ref_s, what="final state")


@pytest.mark.parametrize("form", ["parallel", "chunkwise", "step"])
def test_rotation_at_the_position_cap(form):
    """The last positions a call may use (pos0 + L = 2^31): the rotation angle
    p theta_i is reduced in fp64 before the fp32 sine and cosine, so outputs keep
    the bf16 bar there (the pages' e^{i n theta} at n near 2^31)."""
    dk, dv, H = 128, 256, 2
    L = 1 if form == "step" else 150
    pos0 = 2 ** 31 - L
    q, k, v = _qkv(1, H, L, dk, dv, 500)
    g, th = torch.tensor([0.9, 0.5], dtype=torch.float32), rotation_theta(dk)
    s0 = randn((1, H, dk, dv), 501, 0.3)
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=pos0, s_in=s0)
    if form == "parallel":
        ref_o, _ = oracle.recurrent(q, k, v, g, th, pos0=pos0)
        o = rn.retention_parallel(*_gpu(q, k, v), g, th, pos0=pos0, out_dtype=torch.float32)
    elif form == "chunkwise":
        o, s = rn.retention_chunkwise(*_gpu(q, k, v, ), g, 64, th, pos0=pos0, state_in=s0.to(DEV), state_out=True,
                                      out_dtype=torch.float32)
    else:
        s = s0.to(DEV)
        pos = torch.full((1,), pos0, dtype=torch.int32, device=DEV)
        o = rn.retention_recurrent_step(*_gpu(q[:, :, 0], k[:, :, 0], v[:, :, 0]), s, pos, g, th,
                                        out_dtype=torch.float32)[:, :, None]
    torch.cuda.synchronize()
    _tol.assert_bf16(o, ref_o, what=f"{form} at positions {pos0}..{pos0 + L - 1}")
    if form != "parallel":
        _tol.assert_bf16(s, ref_s, what="state")
