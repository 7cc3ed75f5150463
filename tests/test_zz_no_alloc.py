"""The allocation-free chunkwise entry point (retention_chunkwise_noalloc, for
callers that cannot allocate device memory) against retention_chunkwise, through
the C ABI: calls in a row, each smaller than the one before, on the segment path,
the query-block path (GroupNorm and rotation on) and the fp32 vector path.  Both
entry points run the same kernels on the same plan, so their outputs and states
are equal bit for bit; each is also held to the bf16 (fp32) bar against the fp64
oracle's recurrent form ("Retentive Network" paper summary, Sec. 2.1 (2))."""
import ctypes

import pytest
import torch

import oracle
import retentive_network_scale_amd as rn
from tests import _tol
from workloads import CHUNKWISE_32K, multiscale_gamma, randn, rotation_theta

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (name, B, H, L, dk, dv, chunk, dtype, gn_eps, with state_in), largest first
CASES = [
    ("segment path, the chunkwise workload", 1, 8, 32768, 128, 256, 256, torch.bfloat16, None, False),
    ("query-block path, GroupNorm", 1, 2, 1000, 256, 512, 128, torch.bfloat16, 1e-5, True),
    ("vector path, fp32", 1, 2, 100, 16, 16, 16, torch.float32, None, True),
]


def _inputs(B, H, L, dk, dv, dtype, seed):
    if (B, H, L, dk, dv) == (CHUNKWISE_32K.B, CHUNKWISE_32K.H, CHUNKWISE_32K.L, CHUNKWISE_32K.dk, CHUNKWISE_32K.dv):
        return CHUNKWISE_32K.qkv()
    s = dk ** -0.5
    return (randn((B, H, L, dk), seed, s, dtype), randn((B, H, L, dk), seed + 1, s, dtype),
            randn((B, H, L, dv), seed + 2, 1.0, dtype))


def test_noalloc_matches_workspace_entry_point_in_a_row():
    for i, (name, B, H, L, dk, dv, chunk, dt, eps, with_s) in enumerate(CASES):
        print(f"\n[noalloc] call {i}: {name} B{B} H{H} L{L} dk{dk} dv{dv} chunk{chunk}", flush=True)
        q, k, v = _inputs(B, H, L, dk, dv, dt, 9000 + 10 * i)
        g, th = multiscale_gamma(H), rotation_theta(dk)
        s0 = randn((B, H, dk, dv), 9005 + 10 * i, 0.3) if with_s else None
        need = rn.retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk, dt)
        assert 0 < need <= rn.NOALLOC_SCRATCH_BYTES
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        sd = None if s0 is None else s0.to(DEV)
        out = torch.empty((B, H, L, dv), dtype=dt, device=DEV)
        st = torch.empty((B, H, dk, dv), dtype=torch.float32, device=DEV)
        o1, s1 = rn.retention_chunkwise_noalloc(qd, kd, vd, g, chunk, th, state_in=sd, state_out=st, gn_eps=eps,
                                                out=out)
        o2, s2 = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, state_in=sd, state_out=True, gn_eps=eps)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), name
        assert torch.equal(s1, s2), name
        ref_o, ref_s = oracle.recurrent(q, k, v, g, th, s_in=s0)
        if eps is not None:
            ref_o = oracle.groupnorm(ref_o, eps)
        check = _tol.assert_fp32 if dt == torch.float32 else _tol.assert_bf16
        check(o1, ref_o, slice_dims=2, what=f"{name}: outputs")
        check(s1, ref_s, slice_dims=2, what=f"{name}: state")


def test_noalloc_rejects_what_does_not_fit():
    """A call whose workspace would exceed the scratch fails on the host with
    UNSUPPORTED (nothing is launched), and the next call still works."""
    B, H, L, dk, dv, chunk = 64, 16, 512, 128, 256, 256  # one 128 KiB state per (b, h): 128 MiB
    assert rn.retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk) > rn.NOALLOC_SCRATCH_BYTES
    g, th = multiscale_gamma(H), rotation_theta(dk)
    f = (ctypes.c_float * H)(*[float(x) for x in g])
    t = (ctypes.c_float * (dk // 2))(*[float(x) for x in th])
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the call fails validation
    r = rn.lib().retention_chunkwise_noalloc(fake, ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20),
                                             ctypes.c_void_p(4 << 20), B, H, L, dk, dv, chunk, f, t, 0, None, None,
                                             -1.0, 1, 1, None)
    assert r == 2, r
    assert b"scratch" in rn.lib().retention_last_error()
    q, k, v = (x.to(DEV) for x in _inputs(1, 2, 300, 128, 256, torch.bfloat16, 9100))
    o1, _ = rn.retention_chunkwise_noalloc(q, k, v, multiscale_gamma(2), 64, rotation_theta(128))
    o2, _ = rn.retention_chunkwise(q, k, v, multiscale_gamma(2), 64, rotation_theta(128))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
