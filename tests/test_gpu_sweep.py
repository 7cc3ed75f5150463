"""Seeded random sweep of the bf16 MFMA path against the fp64 oracle ("Retentive
Network" paper summary, Sec. 2.1 and 2.2): each case draws a head-size pair,
batch, heads, a ragged length, a chunk size, per-head decays (including the
edges 0 and 1), a starting position up to 2^31, rotation and GroupNorm on or
off, the output dtype and an incoming state, then checks the chunkwise form
(output and final state, against the recurrent oracle) and the parallel form
(against the parallel oracle) at the bf16 bar."""
import numpy as np
import pytest
import torch

import oracle
import retentive_network_scale_amd as rn
from tests import _tol
from workloads import randn, rotation_theta

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
    pos0 = int(r.integers(0, 2 ** 31))
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
