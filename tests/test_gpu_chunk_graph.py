"""Graph capture of the chunkwise form on the segment kernels.

The chunkwise call with the state in the output kernel's registers (segment-state
pass, scan over segments, segment-output pass) is captured into a HIP graph and
replayed; every replay must give the eager call's bits, and the eager result is
checked against the fp64 oracle's recurrent form ("Retentive Network" paper
summary, Sec. 2.1 (2)/(3)).
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


def _qkv(B, H, L, dk, dv, seed):
    s = 1.0 / np.sqrt(dk)
    return (randn((B, H, L, dk), seed, s, torch.bfloat16), randn((B, H, L, dk), seed + 1, s, torch.bfloat16),
            randn((B, H, L, dv), seed + 2, 1.0, torch.bfloat16))


def test_chunkwise_graph_replay():
    """A captured chunkwise call on the segment kernels (state in registers, the
    long-context head sizes) replayed several times, with eager calls between the
    replays: every replay equals the eager result bit for bit."""
    B, H, L, dk, dv, chunk = 1, 4, 2048, 128, 256, 256
    q, k, v = _qkv(B, H, L, dk, dv, 77)
    g, th = multiscale_gamma(H), rotation_theta(dk)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    ws = torch.empty(rn.retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk), dtype=torch.uint8, device=DEV)
    o_eager, s_eager = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, state_out=True, workspace=ws)
    torch.cuda.synchronize()
    o_g = torch.empty_like(o_eager)
    s_g = torch.empty_like(s_eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            rn.retention_chunkwise(qd, kd, vd, g, chunk, th, state_out=s_g, out=o_g, workspace=ws,
                                   stream=stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for i in range(3):
        o_g.zero_()
        s_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_eager), f"replay {i}: output"
        assert torch.equal(s_g, s_eager), f"replay {i}: state"
        o_e, _ = rn.retention_chunkwise(qd, kd, vd, g, chunk, th, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_eager), f"eager call after replay {i}"
    ref_o, _ = oracle.recurrent(q, k, v, g, th)
    _tol.assert_bf16(o_eager, ref_o, what="graph-replay workload")
