"""GPU parity of the vector (FMA) kernels against the fp64 oracle, through the C ABI.

These cover the fp32 paths (tiny workload: parallel, chunkwise and recurrent
forms), ragged lengths, GroupNorm, incoming/outgoing state, bf16 inputs on
head sizes without an MFMA kernel, and the decode step with per-sequence
positions.
"""
import numpy as np
import pytest
import torch

import oracle
import retentive_network_scale_amd as rn
from tests import _tol
from workloads import TINY, multiscale_gamma, randn, rotation_theta

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu(*ts):
    return [t.to(DEV) for t in ts]


def test_tiny_fp32_three_forms():
    """Tiny workload: B1 H2 L64 dk=dv=16 fp32, chunk 16: every form within 1e-4 of the oracle."""
    q, k, v = TINY.qkv()
    g, th = TINY.gamma(), TINY.theta()
    ref = oracle.parallel(q, k, v, g, th)
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th)
    qd, kd, vd = _gpu(q, k, v)
    o_par = rn.retention_parallel(qd, kd, vd, g, th)
    o_chk, s_chk = rn.retention_chunkwise(qd, kd, vd, g, 16, th, state_out=True)
    state = torch.zeros((1, 2, 16, 16), dtype=torch.float32, device=DEV)
    outs = []
    for n in range(TINY.L):
        pos = torch.full((1,), n, dtype=torch.int32, device=DEV)
        outs.append(rn.retention_recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(),
                                                vd[:, :, n].contiguous(), state, pos, g, th).clone())
    o_rec = torch.stack(outs, 2)
    torch.cuda.synchronize()
    _tol.assert_fp32(o_par, ref, what="parallel")
    _tol.assert_fp32(o_chk, ref, what="chunkwise")
    _tol.assert_fp32(o_rec, ref, what="recurrent")
    _tol.assert_fp32(s_chk, ref_s, what="chunkwise state")
    _tol.assert_fp32(state, ref_s, what="recurrent state")


@pytest.mark.parametrize("chunk", [1, 16, 23, 200])
def test_fp32_ragged_gn_state(chunk):
    B, H, L, dk, dv = 2, 3, 77, 24, 40
    q = randn((B, H, L, dk), 11, 0.3)
    k = randn((B, H, L, dk), 12, 0.3)
    v = randn((B, H, L, dv), 13)
    s0 = randn((B, H, dk, dv), 14)
    g = torch.tensor([0.9, 0.5, 0.999], dtype=torch.float32)
    th = rotation_theta(dk)
    ref_o, ref_s = oracle.chunkwise(q, k, v, g, 7, th, pos0=1000, s_in=s0)
    ref_gn = oracle.groupnorm(ref_o, 1e-5)
    qd, kd, vd, sd = _gpu(q, k, v, s0)
    o, s = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=1000, state_in=sd, state_out=True, gn_eps=1e-5)
    torch.cuda.synchronize()
    _tol.assert_fp32(o, ref_gn, what="chunkwise+GN")
    _tol.assert_fp32(s, ref_s, what="state")
    # state_out aliasing state_in
    s_alias = sd.clone()
    o2, _ = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=1000, state_in=s_alias, state_out=s_alias)
    torch.cuda.synchronize()
    _tol.assert_fp32(o2, ref_o, what="aliased chunkwise")
    _tol.assert_fp32(s_alias, ref_s, what="aliased state")


def test_fp32_parallel_gn_no_theta():
    B, H, L, dk, dv = 1, 2, 130, 8, 24
    q, k, v = randn((B, H, L, dk), 21), randn((B, H, L, dk), 22), randn((B, H, L, dv), 23)
    g = multiscale_gamma(H)
    ref = oracle.groupnorm(oracle.parallel(q, k, v, g), 1e-3)
    o = rn.retention_parallel(*_gpu(q, k, v), g, None, gn_eps=1e-3)
    torch.cuda.synchronize()
    _tol.assert_fp32(o, ref, what="parallel+GN")


def test_bf16_inputs_on_vector_path():
    """bf16 inputs with head sizes that have no MFMA kernel (dk 32, dv 48) run on the
    vector kernels; bf16 bar."""
    B, H, L, dk, dv = 2, 2, 96, 32, 48
    q, k, v = [randn(s, 30 + i, 32 ** -0.5, torch.bfloat16)
               for i, s in enumerate([(B, H, L, dk), (B, H, L, dk), (B, H, L, dv)])]
    g, th = multiscale_gamma(H), rotation_theta(dk)
    ref = oracle.parallel(q, k, v, g, th, pos0=5)
    qd, kd, vd = _gpu(q, k, v)
    _tol.assert_bf16(rn.retention_parallel(qd, kd, vd, g, th, pos0=5), ref, what="parallel bf16->bf16")
    o, _ = rn.retention_chunkwise(qd, kd, vd, g, 32, th, pos0=5, out_dtype=torch.float32)
    _tol.assert_bf16(o, ref, what="chunkwise bf16->fp32")


def test_mask_extraction_on_gpu():
    """theta != 0, q = k = e_0, v_m = e_m: o[n][m] = gamma^(n-m) cos((n-m) theta_0) exactly
    up to fp32 rounding (pins rotation and decay on the device)."""
    L, dk = 64, 16
    q = torch.zeros((1, 1, L, dk)); q[..., 0] = 1.0
    v = torch.eye(L).reshape(1, 1, L, L)
    th = torch.full((dk // 2,), 0.37, dtype=torch.float32)
    g = torch.tensor([1 - 2 ** -5])
    n, m = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    expect = np.where(n >= m, float(g[0]) ** (n - m) * np.cos((n - m) * np.float64(th[0])), 0.0)
    for pos0 in (0, 123456789):
        o = rn.retention_parallel(*_gpu(q, q.clone(), v), g, th, pos0=pos0)
        torch.cuda.synchronize()
        assert np.abs(o[0, 0].double().cpu().numpy() - expect).max() < 2e-6


def test_decode_steps_per_sequence_positions():
    """Prefill with chunkwise, then decode steps where every sequence has its own position."""
    B, H, dk, dv, P, T = 3, 4, 32, 64, 40, 20
    g, th = multiscale_gamma(H), rotation_theta(dk)
    q = randn((B, H, P + T, dk), 41, 0.2)
    k = randn((B, H, P + T, dk), 42, 0.2)
    v = randn((B, H, P + T, dv), 43)
    starts = [0, 7, 1000]  # absolute position of token 0 of each sequence
    qd, kd, vd = _gpu(q, k, v)
    state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=DEV)
    # prefill each sequence at its own origin
    for b in range(B):
        _, s = rn.retention_chunkwise(qd[b:b + 1, :, :P].contiguous(), kd[b:b + 1, :, :P].contiguous(),
                                      vd[b:b + 1, :, :P].contiguous(), g, 16, th, pos0=starts[b],
                                      state_out=True)
        state[b] = s[0]
    outs = []
    for t in range(T):
        pos = torch.tensor([s0 + P + t for s0 in starts], dtype=torch.int32, device=DEV)
        outs.append(rn.retention_recurrent_step(qd[:, :, P + t].contiguous(), kd[:, :, P + t].contiguous(),
                                                vd[:, :, P + t].contiguous(), state, pos, g, th,
                                                gn_eps=1e-5).clone())
    o = torch.stack(outs, 2)
    torch.cuda.synchronize()
    for b in range(B):
        ref_o, ref_s = oracle.recurrent(q[b:b + 1], k[b:b + 1], v[b:b + 1], g, th, pos0=starts[b])
        _tol.assert_fp32(o[b:b + 1], oracle.groupnorm(ref_o[:, :, P:], 1e-5), what=f"decode b={b}")
        _tol.assert_fp32(state[b:b + 1], ref_s, what=f"state b={b}")


def test_empty_sequence_passes_state_through():
    B, H, dk, dv = 1, 2, 16, 16
    g = multiscale_gamma(H)
    s0 = randn((B, H, dk, dv), 51).to(DEV)
    e = torch.empty((B, H, 0, dk), device=DEV)
    ev = torch.empty((B, H, 0, dv), device=DEV)
    o, s = rn.retention_chunkwise(e, e, ev, g, 16, state_in=s0, state_out=True)
    torch.cuda.synchronize()
    assert o.shape == (B, H, 0, dv)
    assert torch.equal(s, s0)
    _, z = rn.retention_chunkwise(e, e, ev, g, 16, state_out=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z) == 0
