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


def test_msr_layer_graph_replay():
    """The whole layer (hipBLASLt GEMMs, the chunkwise passes, the query-block
    kernel's first blocks on a second stream forked from the caller's and joined
    back) captured in a graph and replayed with new inputs, with eager work and
    synchronisations between replays: every replay equals the eager call on the
    same inputs, bit for bit."""
    B, L, dm, H, dk, dv, chunk = 1, 256, 512, 2, 256, 512, 128
    g, th = multiscale_gamma(H), rotation_theta(dk)
    _, w = _inputs(B, L, dm, H, dk, dv, 640)
    wd = [t.to(DEV) for t in w]
    xs_in = [randn((B, L, dm), 650 + i, 1.0, torch.bfloat16).to(DEV) for i in range(3)]
    ws = torch.empty(rn.msr_layer_fwd_workspace_bytes(B, L, dm, H, dk, dv, chunk), dtype=torch.uint8, device=DEV)
    eager = [rn.msr_layer_fwd(x, *wd, H, dk, dv, chunk, g, th, workspace=ws).clone() for x in xs_in]
    xs = torch.empty_like(xs_in[0])
    out = torch.empty_like(xs_in[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream (library plans are built here)
        rn.msr_layer_fwd(xs, *wd, H, dk, dv, chunk, g, th, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rn.msr_layer_fwd(xs, *wd, H, dk, dv, chunk, g, th, out=out, workspace=ws)
    torch.cuda.synchronize()
    for i, x in enumerate(xs_in):
        xs.copy_(x)
        _ = (x.float() * 2).sum()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[i]), f"replay {i} differs from the eager call"


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


def _step_weights(dm, H, dk, dv, seed, w_std=0.05):
    bf = torch.bfloat16
    return [randn((H * dk, dm), seed + 3, w_std, bf), randn((H * dk, dm), seed + 4, w_std, bf),
            randn((H * dv, dm), seed + 5, w_std, bf), randn((H * dv, dm), seed + 6, w_std, bf),
            randn((dm, H * dv), seed + 7, w_std, bf)]


@pytest.mark.parametrize("B,T,dm,H,dk,dv", [(3, 24, 256, 2, 64, 128), (2, 10, 512, 2, 256, 512)])
def test_msr_step_matches_layer(B, T, dm, H, dk, dv):
    """Decode steps from a zero state reproduce the layer's outputs token by token
    (the recurrent representation of the same layer), with a different starting
    position per sequence."""
    x = randn((B, T, dm), 800 + dk, 1.0, torch.bfloat16)
    w = _step_weights(dm, H, dk, dv, 800 + dk)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    starts = [0, 5, 11][:B]
    wd = [t.to(DEV) for t in w]
    state = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=DEV)
    pos = torch.tensor(starts, dtype=torch.int32, device=DEV)
    ys = []
    for t in range(T):
        ys.append(rn.msr_layer_step(x[:, t].contiguous().to(DEV), *wd, state, pos, H, dk, dv, g, th, gn_eps=1e-5))
    got = torch.stack(ys, 1)
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == [s + T for s in starts]
    for b in range(B):
        ref = oracle.msr_layer(x[b:b + 1], *w, H, dk, dv, g, th, pos0=starts[b], gn_eps=1e-5)
        _tol.assert_bf16(got[b:b + 1], ref, slice_dims=0, what=f"msr step b={b}")


def test_msr_step_many_sequences():
    """70 sequences per step: the step's GEMMs take one full 64-row tile and a
    ragged one of 6 rows; 3 steps from a zero state against the oracle layer."""
    B, T, dm, H, dk, dv = 70, 3, 256, 2, 64, 128
    x = randn((B, T, dm), 870, 1.0, torch.bfloat16)
    w = _step_weights(dm, H, dk, dv, 870)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    wd = [t.to(DEV) for t in w]
    state = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    got = torch.stack([rn.msr_layer_step(x[:, t].contiguous().to(DEV), *wd, state, pos, H, dk, dv, g, th,
                                         gn_eps=1e-5) for t in range(T)], 1)
    torch.cuda.synchronize()
    ref = oracle.msr_layer(x, *w, H, dk, dv, g, th, pos0=0, gn_eps=1e-5)
    _tol.assert_bf16(got[:64], ref[:64], slice_dims=0, what="msr step, first 64-row tile")
    _tol.assert_bf16(got[64:], ref[64:], slice_dims=0, what="msr step, ragged 6-row tile")


def test_msr_step_graph_replay():
    """One step captured as a graph (positions advanced on the device) and replayed
    once per token, with host copies and synchronisations between replays: every
    replay equals the eager step."""
    B, T, dm, H, dk, dv = 4, 12, 256, 2, 64, 128
    x = randn((B, T, dm), 900, 1.0, torch.bfloat16).to(DEV)
    wd = [t.to(DEV) for t in _step_weights(dm, H, dk, dv, 900)]
    g, th = multiscale_gamma(H), rotation_theta(dk)
    # eager reference
    s_e = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=DEV)
    p_e = torch.zeros(B, dtype=torch.int32, device=DEV)
    eager = [rn.msr_layer_step(x[:, t].contiguous(), *wd, s_e, p_e, H, dk, dv, g, th) for t in range(T)]
    # captured step on static buffers
    xs = torch.empty((B, dm), dtype=torch.bfloat16, device=DEV)
    ys = torch.empty((B, dm), dtype=torch.bfloat16, device=DEV)
    s_g = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=DEV)
    p_g = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = torch.empty(rn.msr_layer_step_workspace_bytes(B, dm, H, dk, dv), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream (library plans are built here)
        xs.copy_(x[:, 0])
        rn.msr_layer_step(xs, *wd, s_g, p_g, H, dk, dv, g, th, out=ys, workspace=ws, advance_pos=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    s_g.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rn.msr_layer_step(xs, *wd, s_g, p_g, H, dk, dv, g, th, out=ys, workspace=ws, advance_pos=True)
    torch.cuda.synchronize()
    s_g.zero_()
    p_g.zero_()
    torch.cuda.synchronize()
    for t in range(T):
        xs.copy_(x[:, t])
        graph.replay()
        torch.cuda.synchronize()
        _tol.assert_bf16(ys, eager[t], slice_dims=0, what=f"replay {t}")
    assert p_g.cpu().tolist() == [T] * B
    _tol.assert_bf16(s_g, s_e, slice_dims=0, what="state after replays")


def test_msr_step_full_layer_dims():
    """The layer workload's dimensions (d_model 2048, 8 heads, dk 256, dv 512), 4
    sequences, 6 steps from a zero state, against the oracle layer."""
    wl = MSRWorkload()
    B, T = 4, 6
    x, wq, wk, wv, wg, wo = wl.inputs()
    x = x[:, :T].contiguous()
    g, th = wl.gamma(), wl.theta()
    wd = [t.to(DEV) for t in (wq, wk, wv, wg, wo)]
    state = torch.zeros((B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    got = torch.stack([rn.msr_layer_step(x[:, t].contiguous().to(DEV), *wd, state, pos, wl.H, wl.dk, wl.dv, g, th,
                                         gn_eps=wl.gn_eps) for t in range(T)], 1)
    torch.cuda.synchronize()
    ref = oracle.msr_layer(x, wq, wk, wv, wg, wo, wl.H, wl.dk, wl.dv, g, th, pos0=0, gn_eps=wl.gn_eps)
    _tol.assert_bf16(got, ref, slice_dims=0, what="msr step, layer dims")


def test_msr_step_decode_batch_fused():
    """The decode benchmark's step: 64 sequences at the layer workload's
    dimensions with the four projection weights back to back (one fused GEMM of
    12288 columns over d_model 2048, then the output GEMM over H dv = 4096), 2
    steps from a zero state against the oracle layer, every sequence."""
    wl = MSRWorkload()
    B, T = 64, 2
    _, wq, wk, wv, wg, wo = wl.inputs()
    x = randn((B, T, wl.d_model), 5100, 1.0, torch.bfloat16)
    g, th = wl.gamma(), wl.theta()
    cat = torch.cat([wq, wk, wv, wg], 0).to(DEV)
    fq, fk, fv, fg = torch.split(cat, [wl.H * wl.dk, wl.H * wl.dk, wl.H * wl.dv, wl.H * wl.dv], 0)
    state = torch.zeros((B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    got = torch.stack([rn.msr_layer_step(x[:, t].contiguous().to(DEV), fq, fk, fv, fg, wo.to(DEV), state, pos, wl.H,
                                         wl.dk, wl.dv, g, th, gn_eps=wl.gn_eps) for t in range(T)], 1)
    torch.cuda.synchronize()
    ref = oracle.msr_layer(x, wq, wk, wv, wg, wo, wl.H, wl.dk, wl.dv, g, th, pos0=0, gn_eps=wl.gn_eps)
    _tol.assert_bf16(got, ref, slice_dims=0, what="msr decode batch, fused weights")


def test_msr_fused_weights_match_separate():
    """Weights stored back to back (one fused projection matrix) take the
    single-GEMM path; layer and step outputs match the separate-weight path and
    the oracle."""
    B, L, dm, H, dk, dv = 2, 96, 256, 2, 64, 128
    x, (wq, wk, wv, wg, wo) = _inputs(B, L, dm, H, dk, dv, 950)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    cat = torch.cat([wq, wk, wv, wg], 0).to(DEV)
    fq, fk, fv, fg = torch.split(cat, [H * dk, H * dk, H * dv, H * dv], 0)
    xd, wod = x.to(DEV), wo.to(DEV)
    sep = [t.to(DEV) for t in (wq, wk, wv, wg)]
    y_f = rn.msr_layer_fwd(xd, fq, fk, fv, fg, wod, H, dk, dv, 32, g, th, gn_eps=1e-5)
    y_s = rn.msr_layer_fwd(xd, *sep, wod, H, dk, dv, 32, g, th, gn_eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.msr_layer(x, wq, wk, wv, wg, wo, H, dk, dv, g, th, pos0=0, gn_eps=1e-5)
    _tol.assert_bf16(y_f, ref, slice_dims=0, what="fused weights, layer")
    _tol.assert_bf16(y_f, y_s.float().cpu().double().numpy(), slice_dims=0, what="fused vs separate")
    state = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    steps = torch.stack([rn.msr_layer_step(xd[:, t].contiguous(), fq, fk, fv, fg, wod, state, pos, H, dk, dv, g, th)
                         for t in range(8)], 1)
    torch.cuda.synchronize()
    _tol.assert_bf16(steps, ref[:, :8], slice_dims=0, what="fused weights, steps")


def _block_weights(dm, H, dk, dv, dff, seed, w_std=0.05):
    bf = torch.bfloat16
    return _step_weights(dm, H, dk, dv, seed, w_std) + [randn((dff, dm), seed + 8, w_std, bf),
                                                         randn((dm, dff), seed + 9, w_std, bf)]


@pytest.mark.parametrize("B,L,dm,H,dk,dv,dff,chunk", [(2, 130, 256, 2, 64, 128, 512, 64),
                                                      (1, 200, 512, 2, 256, 512, 1024, 128)])
def test_retnet_block_small(B, L, dm, H, dk, dv, dff, chunk):
    """The pre-LN residual block (LayerNorm, gated layer, residual, LayerNorm, gelu
    FFN, residual) against the oracle."""
    x = randn((B, L, dm), 1300 + dk, 1.0, torch.bfloat16)
    w = _block_weights(dm, H, dk, dv, dff, 1300 + dk)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    y = rn.retnet_block_fwd(x.to(DEV), *[t.to(DEV) for t in w], H, dk, dv, chunk, g, th, pos0=2)
    torch.cuda.synchronize()
    ref = oracle.retnet_block(x, *w, H, dk, dv, g, th, pos0=2)
    _tol.assert_bf16(y, ref, slice_dims=0, what="block")
    _tol.assert_bf16(y, ref, slice_dims=1, what="block per batch")


def test_retnet_block_full_size_sampled():
    """The layer workload's dimensions with an FFN of width 2 d_model (4096): sampled
    rows against the oracle (causal, so only the prefix up to each row is used)."""
    wl = MSRWorkload()
    x, wq, wk, wv, wg, wo = wl.inputs()
    dff = 2 * wl.d_model
    w1 = randn((dff, wl.d_model), 5008, wl.w_std, torch.bfloat16)
    w2 = randn((wl.d_model, dff), 5009, wl.w_std, torch.bfloat16)
    g, th = wl.gamma(), wl.theta()
    dev = [t.to(DEV) for t in (x, wq, wk, wv, wg, wo, w1, w2)]
    y = rn.retnet_block_fwd(*dev, wl.H, wl.dk, wl.dv, wl.chunk, g, th, gn_eps=wl.gn_eps)
    torch.cuda.synchronize()
    yc = y.float().cpu().numpy()
    samples = {0: [0, 1, 700], 2: [5, 512]}
    for b, ls in samples.items():
        lmax = max(ls) + 1
        ref = oracle.retnet_block(x[b:b + 1, :lmax], wq, wk, wv, wg, wo, w1, w2, wl.H, wl.dk, wl.dv, g, th,
                                  gn_eps=wl.gn_eps, tokens=[(0, l) for l in ls])
        got = np.stack([yc[b, l] for l in ls])
        _tol.assert_bf16(got, ref, slice_dims=0, what=f"block full-size batch {b}")
