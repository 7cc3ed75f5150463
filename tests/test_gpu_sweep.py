"""Seeded random sweeps against the fp64 oracle ("Retentive Network" paper
summary, Sec. 2.1 and 2.2).  Each case draws its shapes (head sizes, batch,
heads, a ragged length, a chunk size), per-head decays (including the edges 0
and 1), a starting position up to 2^31, rotation and GroupNorm on or off, the
output dtype and an incoming state.  Checked: the bf16 MFMA forms (chunkwise
output and final state against the recurrent oracle, parallel against the
parallel oracle), the fp32 vector path, decode steps, the chunkwise backward
and the gated layer, each at its bar."""
import numpy as np
import pytest
import torch

import oracle
import retentive_network_scale_amd as rn
from tests import _tol
from workloads import multiscale_gamma, randn, rotation_theta

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAIRS = [(64, 128), (128, 128), (128, 256), (256, 256), (256, 512)]
GAMMAS = [0.0, 0.5, 0.9, 0.96875, 0.999, 1.0]


def _case(seed):
    r = np.random.default_rng(seed)
    dk, dv = PAIRS[int(r.integers(len(PAIRS)))]
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    L = int(r.integers(1, 400))
    chunk = int(r.integers(16, 321))
    gamma = torch.tensor([GAMMAS[int(i)] for i in r.integers(len(GAMMAS), size=H)], dtype=torch.float32)
    pos0 = min(int(r.integers(0, 2 ** 31)), 2 ** 31 - L)  # positions are int32: pos0 + L <= 2^31
    rot, gn = bool(r.integers(2)), bool(r.integers(2))
    odt = torch.float32 if r.integers(2) else torch.bfloat16
    with_state = bool(r.integers(2))
    return dict(dk=dk, dv=dv, B=B, H=H, L=L, chunk=chunk, gamma=gamma, pos0=pos0, rot=rot, gn=gn, odt=odt,
                with_state=with_state)


@pytest.mark.parametrize("seed", range(16))
def test_random_case(seed):
    c = _case(4000 + seed)
    dk, dv, B, H, L = c["dk"], c["dv"], c["B"], c["H"], c["L"]
    s = dk ** -0.5
    q = randn((B, H, L, dk), 4100 + seed, s, torch.bfloat16)
    k = randn((B, H, L, dk), 4200 + seed, s, torch.bfloat16)
    v = randn((B, H, L, dv), 4300 + seed, 1.0, torch.bfloat16)
    s0 = randn((B, H, dk, dv), 4400 + seed, 0.5) if c["with_state"] else None
    th = rotation_theta(dk) if c["rot"] else None
    g, pos0, eps = c["gamma"], c["pos0"], (1e-5 if c["gn"] else None)
    what = f"seed {seed}: {c}"
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))

    # chunkwise, against the recurrent oracle (output and final state)
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=pos0, s_in=s0)
    o, st = rn.retention_chunkwise(qd, kd, vd, g, c["chunk"], th, pos0=pos0,
                                   state_in=None if s0 is None else s0.to(DEV), state_out=True,
                                   gn_eps=eps, out_dtype=c["odt"])
    torch.cuda.synchronize()
    _tol.assert_bf16(o, oracle.groupnorm(ref_o, eps) if eps is not None else ref_o, what="chunkwise " + what)
    _tol.assert_bf16(st, ref_s, what="final state " + what)

    # parallel, against the parallel oracle
    ref_p = oracle.parallel(q, k, v, g, th, pos0=pos0)
    if eps is not None:
        ref_p = oracle.groupnorm(ref_p, eps)
    op = rn.retention_parallel(qd, kd, vd, g, th, pos0=pos0, gn_eps=eps, out_dtype=c["odt"])
    torch.cuda.synchronize()
    _tol.assert_bf16(op, ref_p, what="parallel " + what)


def _gammas(r, H):
    return torch.tensor([GAMMAS[int(i)] for i in r.integers(len(GAMMAS), size=H)], dtype=torch.float32)


@pytest.mark.parametrize("seed", range(8))
def test_random_fp32_vector_path(seed):
    """fp32 inputs (vector kernels): any even head sizes, fp32 bar."""
    r = np.random.default_rng(5000 + seed)
    dk, dv = 2 * int(r.integers(1, 49)), 4 * int(r.integers(1, 33))
    B, H, L = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.integers(1, 200))
    chunk, g, pos0 = int(r.integers(1, 130)), _gammas(r, H), int(r.integers(0, 2 ** 31))
    pos0 = min(pos0, 2 ** 31 - L)
    th = rotation_theta(dk) if r.integers(2) else None
    eps = 1e-5 if r.integers(2) else None
    s0 = randn((B, H, dk, dv), 5100 + seed, 0.5) if r.integers(2) else None
    q, k = randn((B, H, L, dk), 5200 + seed, dk ** -0.5), randn((B, H, L, dk), 5300 + seed, dk ** -0.5)
    v = randn((B, H, L, dv), 5400 + seed)
    what = f"seed {seed}: dk={dk} dv={dv} B={B} H={H} L={L} chunk={chunk} g={g.tolist()} rot={th is not None} gn={eps}"
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=pos0, s_in=s0)
    o, st = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=pos0,
                                   state_in=None if s0 is None else s0.to(DEV), state_out=True, gn_eps=eps)
    torch.cuda.synchronize()
    _tol.assert_fp32(o, oracle.groupnorm(ref_o, eps) if eps is not None else ref_o, what="chunkwise " + what)
    _tol.assert_fp32(st, ref_s, what="final state " + what)
    ref_p = oracle.parallel(q, k, v, g, th, pos0=pos0)
    op = rn.retention_parallel(qd, kd, vd, g, th, pos0=pos0, gn_eps=eps)
    torch.cuda.synchronize()
    _tol.assert_fp32(op, oracle.groupnorm(ref_p, eps) if eps is not None else ref_p, what="parallel " + what)


@pytest.mark.parametrize("seed", range(6))
def test_random_decode_steps(seed):
    """Decode steps from a random state, every sequence at its own position (up
    to 2^31), fp32 or bf16 inputs, bf16 or fp32 outputs."""
    r = np.random.default_rng(6000 + seed)
    dk, dv = [(16, 24), (64, 128), (128, 256), (256, 512)][int(r.integers(4))]
    B, H, T = int(r.integers(1, 5)), int(r.integers(1, 4)), int(r.integers(1, 6))
    g = _gammas(r, H)
    th = rotation_theta(dk) if r.integers(2) else None
    eps = 1e-5 if r.integers(2) else None
    dt = torch.bfloat16 if r.integers(2) else torch.float32
    odt = torch.bfloat16 if r.integers(2) else torch.float32
    starts = [int(x) for x in r.integers(0, 2 ** 31 - T, size=B)]
    q = randn((B, H, T, dk), 6100 + seed, dk ** -0.5, dt)
    k = randn((B, H, T, dk), 6200 + seed, dk ** -0.5, dt)
    v = randn((B, H, T, dv), 6300 + seed, 1.0, dt)
    s0 = randn((B, H, dk, dv), 6400 + seed, 0.5)
    state = s0.to(DEV)
    outs = []
    for t in range(T):
        pos = torch.tensor([s + t for s in starts], dtype=torch.int32, device=DEV)
        outs.append(rn.retention_recurrent_step(q[:, :, t].contiguous().to(DEV), k[:, :, t].contiguous().to(DEV),
                                                v[:, :, t].contiguous().to(DEV), state, pos, g, th, gn_eps=eps,
                                                out_dtype=odt).clone())
    o = torch.stack(outs, 2)
    torch.cuda.synchronize()
    what = f"seed {seed}: dk={dk} dv={dv} B={B} H={H} T={T} g={g.tolist()} rot={th is not None} gn={eps} {dt} {odt}"
    for b in range(B):
        ref_o, ref_s = oracle.recurrent(q[b:b + 1], k[b:b + 1], v[b:b + 1], g, th, pos0=starts[b], s_in=s0[b:b + 1])
        if eps is not None:
            ref_o = oracle.groupnorm(ref_o, eps)
        if odt == torch.float32:
            _tol.assert_fp32(o[b:b + 1], ref_o, what=f"decode b={b} " + what)
        else:
            _tol.assert_bf16(o[b:b + 1], ref_o, what=f"decode b={b} " + what)
        _tol.assert_fp32(state[b:b + 1], ref_s, what=f"state b={b} " + what)


@pytest.mark.parametrize("seed", range(8))
def test_random_backward(seed):
    """Gradients of chunkwise retention with bf16 inputs (MFMA kernels), fp32 out."""
    r = np.random.default_rng(7000 + seed)
    dk, dv = [(64, 128), (128, 128), (128, 256)][int(r.integers(3))]
    B, H, L = 1, int(r.integers(1, 4)), int(r.integers(1, 300))
    chunk, g, pos0 = int(r.integers(16, 300)), _gammas(r, H), int(r.integers(0, 2 ** 31))
    pos0 = min(pos0, 2 ** 31 - L)
    th = rotation_theta(dk) if r.integers(2) else None
    q = randn((B, H, L, dk), 7100 + seed, dk ** -0.5, torch.bfloat16)
    k = randn((B, H, L, dk), 7200 + seed, dk ** -0.5, torch.bfloat16)
    v = randn((B, H, L, dv), 7300 + seed, 1.0, torch.bfloat16)
    do = randn((B, H, L, dv), 7400 + seed, 1.0, torch.bfloat16)
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, chunk, th, pos0=pos0,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, do, g, th, pos0)
    what = f"seed {seed}: dk={dk} dv={dv} H={H} L={L} chunk={chunk} g={g.tolist()} rot={th is not None}"
    for name, a, b in zip("qkv", got, ref):
        _tol.assert_bf16(a, b, slice_dims=2, what=f"d{name} " + what)


@pytest.mark.parametrize("seed", range(4))
def test_random_msr_layer(seed):
    """The gated layer at small random shapes against the oracle layer."""
    r = np.random.default_rng(8000 + seed)
    dk, dv = [(64, 128), (128, 256), (256, 512)][int(r.integers(3))]
    H = int(r.integers(1, 3))
    dm = 128 * int(r.integers(1, 5))
    if (H * dk) % 128:
        H = 2
    B, L = int(r.integers(1, 3)), int(r.integers(1, 300))
    chunk, pos0 = int(r.integers(16, 300)), int(r.integers(0, 2 ** 31))
    pos0 = min(pos0, 2 ** 31 - L)
    g = multiscale_gamma(H)
    th = rotation_theta(dk)
    x = randn((B, L, dm), 8100 + seed, 1.0, torch.bfloat16)
    w = [randn((H * dk, dm), 8200 + seed, 0.05, torch.bfloat16), randn((H * dk, dm), 8300 + seed, 0.05, torch.bfloat16),
         randn((H * dv, dm), 8400 + seed, 0.05, torch.bfloat16), randn((H * dv, dm), 8500 + seed, 0.05, torch.bfloat16),
         randn((dm, H * dv), 8600 + seed, 0.05, torch.bfloat16)]
    y = rn.msr_layer_fwd(x.to(DEV), *(t.to(DEV) for t in w), H, dk, dv, chunk, g, th, pos0=pos0, gn_eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.msr_layer(x, *w, H, dk, dv, g, th, pos0=pos0, gn_eps=1e-5)
    _tol.assert_bf16(y, ref, slice_dims=0, what=f"msr seed {seed}: dk={dk} dv={dv} H={H} dm={dm} B={B} L={L} chunk={chunk}")


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 256)])
def test_backward_fast_decay_rotated(dk, dv):
    """gamma = 0 and 0.5 with rotation: every gradient row sums one or a few terms,
    so the rounding of the rotated operands does not average out."""
    B, H, L, chunk = 1, 2, 300, 128
    g = torch.tensor([0.0, 0.5], dtype=torch.float32)
    th = rotation_theta(dk)
    q = randn((B, H, L, dk), 7500, dk ** -0.5, torch.bfloat16)
    k = randn((B, H, L, dk), 7501, dk ** -0.5, torch.bfloat16)
    v = randn((B, H, L, dv), 7502, 1.0, torch.bfloat16)
    do = randn((B, H, L, dv), 7503, 1.0, torch.bfloat16)
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, chunk, th, pos0=12345,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, do, g, th, 12345)
    for name, a, b in zip("qkv", got, ref):
        _tol.assert_bf16(a, b, slice_dims=2, what=f"d{name} dk={dk} dv={dv}")


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 256), (256, 512)])
def test_forward_fast_decay_rotated(dk, dv):
    """The forward forms at gamma = 0 and 0.5 with rotation (hi+lo scores)."""
    B, H, L = 1, 2, 300
    g = torch.tensor([0.0, 0.5], dtype=torch.float32)
    th = rotation_theta(dk)
    q = randn((B, H, L, dk), 7600, dk ** -0.5, torch.bfloat16)
    k = randn((B, H, L, dk), 7601, dk ** -0.5, torch.bfloat16)
    v = randn((B, H, L, dv), 7602, 1.0, torch.bfloat16)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ref = oracle.parallel(q, k, v, g, th, pos0=99)
    o, _ = rn.retention_chunkwise(qd, kd, vd, g, 128, th, pos0=99, out_dtype=torch.float32)
    op = rn.retention_parallel(qd, kd, vd, g, th, pos0=99, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _tol.assert_bf16(o, ref, what=f"chunkwise dk={dk} dv={dv}")
    _tol.assert_bf16(op, ref, what=f"parallel dk={dk} dv={dv}")


def test_max_heads_forms_and_step():
    """128 heads (the most the interface takes), each with its own decay, through
    the MFMA forms (chunkwise with GroupNorm, parallel) and one decode step."""
    B, H, L, dk, dv = 1, 128, 70, 64, 128
    g = torch.tensor([1.0 - 2.0 ** (-1.0 - h / 16.0) for h in range(H)], dtype=torch.float32)
    th = rotation_theta(dk)
    q = randn((B, H, L, dk), 9200, dk ** -0.5, torch.bfloat16)
    k = randn((B, H, L, dk), 9201, dk ** -0.5, torch.bfloat16)
    v = randn((B, H, L, dv), 9202, 1.0, torch.bfloat16)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=3)
    o, s = rn.retention_chunkwise(qd, kd, vd, g, 64, th, pos0=3, state_out=True, gn_eps=1e-5,
                                  out_dtype=torch.float32)
    op = rn.retention_parallel(qd, kd, vd, g, th, pos0=3, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _tol.assert_bf16(o, oracle.groupnorm(ref_o, 1e-5), what="chunkwise, 128 heads")
    _tol.assert_bf16(s, ref_s, what="final state, 128 heads")
    _tol.assert_bf16(op, ref_o, what="parallel, 128 heads")
    # one decode step on top of the final state, at position 3 + L
    q1 = randn((B, H, dk), 9203, dk ** -0.5, torch.bfloat16)
    k1 = randn((B, H, dk), 9204, dk ** -0.5, torch.bfloat16)
    v1 = randn((B, H, dv), 9205, 1.0, torch.bfloat16)
    pos = torch.tensor([3 + L], dtype=torch.int32, device=DEV)
    st = s.clone()
    o1 = rn.retention_recurrent_step(q1.to(DEV), k1.to(DEV), v1.to(DEV), st, pos, g, th, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref1, ref_s1 = oracle.recurrent(q1[:, :, None], k1[:, :, None], v1[:, :, None], g, th, pos0=3 + L,
                                    s_in=s.cpu())
    _tol.assert_fp32(o1, ref1[:, :, 0], what="decode step, 128 heads")
    _tol.assert_fp32(st, ref_s1, what="state after the step, 128 heads")


@pytest.mark.parametrize("L", [1, 63, 64, 65, 129])
@pytest.mark.parametrize("dk,dv", [(128, 256), (256, 512)])
def test_tile_edge_lengths(L, dk, dv):
    """Lengths at and around the 64-token tile, both MFMA forms, with GroupNorm
    and rotation (hi+lo first blocks) and without."""
    B, H = 2, 2
    g = multiscale_gamma(H)
    th = rotation_theta(dk)
    q = randn((B, H, L, dk), 9300 + L, dk ** -0.5, torch.bfloat16)
    k = randn((B, H, L, dk), 9301 + L, dk ** -0.5, torch.bfloat16)
    v = randn((B, H, L, dv), 9302 + L, 1.0, torch.bfloat16)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ref = oracle.parallel(q, k, v, g, th, pos0=0)
    for eps in (None, 1e-5):
        r = oracle.groupnorm(ref, eps) if eps is not None else ref
        o, _ = rn.retention_chunkwise(qd, kd, vd, g, 64, th, gn_eps=eps, out_dtype=torch.float32)
        op = rn.retention_parallel(qd, kd, vd, g, th, gn_eps=eps, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _tol.assert_bf16(o, r, what=f"chunkwise L={L} gn={eps}")
        _tol.assert_bf16(op, r, what=f"parallel L={L} gn={eps}")


@pytest.mark.parametrize("dk,dv,chunk,L,gn", [(128, 256, 512, 1100, False), (128, 256, 1024, 2100, True),
                                             (64, 128, 2048, 2100, False), (256, 128, 512, 700, True)])
def test_long_chunks_state_in_registers(dk, dv, chunk, L, gn):
    """Chunks longer than four 64-token key blocks, too few for a segment per CU
    (here 2 heads of a short sequence), with states that fit the segment-output
    kernel run the per-chunk query-block path instead: output (with GroupNorm or
    not), incoming and final state against the recurrent oracle, at ragged
    lengths."""
    B, H = 1, 2
    g = torch.tensor([0.96875, 0.999], dtype=torch.float32)
    th = rotation_theta(dk)
    q = randn((B, H, L, dk), 9400, dk ** -0.5, torch.bfloat16)
    k = randn((B, H, L, dk), 9401, dk ** -0.5, torch.bfloat16)
    v = randn((B, H, L, dv), 9402, 1.0, torch.bfloat16)
    s_in = randn((B, H, dk, dv), 9403, 0.1, torch.float32)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    eps = 1e-5 if gn else None
    ref_o, ref_s = oracle.recurrent(q, k, v, g, th, pos0=777, s_in=s_in)
    o, s = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, pos0=777, state_in=s_in.to(DEV), state_out=True,
                                  gn_eps=eps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    what = f"dk={dk} dv={dv} chunk={chunk} L={L} gn={gn}"
    _tol.assert_bf16(o, oracle.groupnorm(ref_o, eps) if gn else ref_o, what="chunkwise " + what)
    _tol.assert_bf16(s, ref_s, what="final state " + what)


def test_backward_long_chunk():
    """The backward at a chunk longer than four key blocks and too few chunks for
    a segment per CU: its inner retentions then run the per-chunk path, on
    explicitly reversed copies (that path reads inputs in order only)."""
    dk, dv, B, H, L, chunk = 128, 256, 1, 2, 700, 512
    g = torch.tensor([0.96875, 0.999], dtype=torch.float32)
    th = rotation_theta(dk)
    q = randn((B, H, L, dk), 9500, dk ** -0.5, torch.bfloat16)
    k = randn((B, H, L, dk), 9501, dk ** -0.5, torch.bfloat16)
    v = randn((B, H, L, dv), 9502, 1.0, torch.bfloat16)
    do = randn((B, H, L, dv), 9503, 1.0, torch.bfloat16)
    got = rn.retention_chunkwise_bwd(*(t.to(DEV) for t in (q, k, v, do)), g, chunk, th, pos0=4242,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, do, g, th, 4242)
    for name, a, b in zip("qkv", got, ref):
        _tol.assert_bf16(a, b, slice_dims=2, what=f"d{name} chunk={chunk}")
