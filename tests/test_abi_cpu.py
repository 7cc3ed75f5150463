"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch (so no
call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import retentive_network_scale_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: every call below fails validation
FAKE2 = ctypes.c_void_p(0x200000)
FAKE3 = ctypes.c_void_p(0x300000)
FAKE4 = ctypes.c_void_p(0x400000)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(retention_\w+|msr_\w+|retnet_\w+)\s*\(", src)))


def _f(vals):
    return (ctypes.c_float * len(vals))(*vals)


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "retention_parallel" in names and "msr_layer_fwd" in names
    L = rn.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in rn.EXPORTED_SYMBOLS, f"binding does not wrap {n}"
    assert set(rn.EXPORTED_SYMBOLS) == set(names)


def test_version_and_status_strings():
    L = rn.lib()
    assert L.retention_abi_version() == 1
    assert L.retention_status_string(0) == b"ok"
    assert L.retention_status_string(3) == b"workspace too small"


def _par(**kw):
    a = dict(q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, B=1, H=2, L=8, dk=16, dv=16, gamma=_f([0.9, 0.5]),
             theta=None, pos0=0, eps=-1.0, ind=F32, outd=F32)
    a.update(kw)
    return rn.lib().retention_parallel(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["L"], a["dk"],
                                       a["dv"], a["gamma"], a["theta"], a["pos0"], a["eps"], a["ind"],
                                       a["outd"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(dk=0), INVALID), (dict(L=-3), INVALID),
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(gamma=None), INVALID),
    (dict(gamma=_f([1.5, 0.5])), INVALID), (dict(gamma=_f([float("nan"), 0.5])), INVALID),
    (dict(gamma=_f([-0.1, 0.5])), INVALID),
    (dict(dk=15, theta=_f([1.0] * 7)), INVALID), (dict(theta=_f([1.0] * 7 + [float("inf")])), INVALID),
    (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(ind=7), INVALID), (dict(pos0=-1), INVALID),
    (dict(q=ctypes.c_void_p(0x100004)), INVALID),   # misaligned
    (dict(o=FAKE), INVALID),                        # output aliases an input
    (dict(H=129, gamma=_f([0.5] * 129)), UNSUPPORTED), (dict(dv=2048), UNSUPPORTED),
])
def test_parallel_rejects(kw, code):
    assert _par(**kw) == code
    assert rn.lib().retention_last_error() != b""


def test_empty_sequence_is_a_noop():
    assert _par(L=0, q=None, k=None, v=None, o=None) == 0


def test_chunkwise_rejects_and_workspace():
    L = rn.lib()
    g = _f([0.9, 0.5])
    need = L.retention_chunkwise_workspace_bytes(1, 2, 64, 16, 16, 16, F32)
    assert need > 0
    call = lambda chunk=16, ws=None, wsb=0, so=None: L.retention_chunkwise(
        FAKE, FAKE2, FAKE3, FAKE4, 1, 2, 64, 16, 16, chunk, g, None, 0, None, so, -1.0, F32, F32, ws,
        wsb, None)
    assert call(chunk=0) == INVALID
    assert call() == WORKSPACE                      # no state_out: the state needs the workspace
    assert call(ws=FAKE, wsb=need - 1) == WORKSPACE
    assert call(so=FAKE) == INVALID                 # state_out overlaps q
    assert L.retention_chunkwise_workspace_bytes(0, 2, 64, 16, 16, 16, F32) == 0


def test_recurrent_step_rejects():
    L = rn.lib()
    g = _f([0.9, 0.5])
    th = _f([1.0] * 8)
    st = ctypes.c_void_p(0x500000)
    base = dict(q=FAKE, k=FAKE2, v=FAKE3, s=st, o=FAKE4, th=None, pos=None, dv=16)

    def call(**kw):
        a = dict(base); a.update(kw)
        return L.retention_recurrent_step(a["q"], a["k"], a["v"], a["s"], a["o"], 2, 2, 16, a["dv"], g,
                                          a["th"], a["pos"], -1.0, F32, F32, None)
    assert call(s=None) == INVALID
    assert call(th=th) == INVALID                  # rotation needs positions
    assert call(dv=1022) == UNSUPPORTED
    assert call(o=st) == INVALID                    # o aliases the state


def test_msr_rejects_unsupported_shapes():
    L = rn.lib()
    g = _f([0.9] * 2)
    r = L.msr_layer_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, 1, 8, 40, 2, 24, 24, 8, g, None, 0,
                        1e-5, None, 0, None)
    assert r in (INVALID, UNSUPPORTED)


def test_msr_step_rejects_and_workspace():
    """Host-side validation of the decode step: every case fails before any launch."""
    L = rn.lib()
    g = _f([0.9] * 2)
    INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
    need = L.msr_layer_step_workspace_bytes(4, 256, 2, 64, 128)
    assert need >= 4 * (2 * 2 * 64 + 2 * 2 * 128) * 2 + 4 * 2 * 128 * 2
    assert L.msr_layer_step_workspace_bytes(0, 256, 2, 64, 128) == 0
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, FAKE3, FAKE4, 1, 4, 256, 2, 64, 128, g, None, 1e-5]
    # NULL state
    a = list(args)
    a[7] = None
    assert L.msr_layer_step(*a, FAKE, need, None) == INVALID
    # NULL positions
    a = list(args)
    a[8] = None
    assert L.msr_layer_step(*a, FAKE, need, None) == INVALID
    # gamma outside [0, 1]
    a = list(args)
    a[15] = _f([0.9, 1.5])
    assert L.msr_layer_step(*a, FAKE, need, None) == INVALID
    # d_model not a multiple of 128
    a = list(args)
    a[11] = 200
    assert L.msr_layer_step(*a, FAKE, need, None) == UNSUPPORTED
    # negative eps (the layer always normalises)
    a = list(args)
    a[17] = -1.0
    assert L.msr_layer_step(*a, FAKE, need, None) == INVALID
    # workspace too small
    assert L.msr_layer_step(*args, FAKE, need - 1, None) == WORKSPACE
    assert b"workspace" in L.retention_last_error()


def test_backward_rejects_and_workspace():
    L = rn.lib()
    g = _f([0.9] * 2)
    INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
    need = L.retention_chunkwise_bwd_workspace_bytes(1, 2, 64, 16, 32, 16, 1)
    assert need >= 3 * 2 * 64 * 16 * 2 + 2 * 2 * 64 * 32 * 2 + 4 * 2 * 64 * (16 + 16 + 32)
    assert L.retention_chunkwise_bwd_workspace_bytes(1, 2, 0, 16, 32, 16, 1) == 0

    def call(dk=16, dv=32, chunk=16, ws=FAKE4, wsb=need, dq=FAKE2, gamma=g):
        return L.retention_chunkwise_bwd(FAKE, FAKE, FAKE, FAKE, dq, FAKE3, ctypes.c_void_p(0x500000), 1, 2, 64,
                                         dk, dv, chunk, gamma, None, 0, 1, 1, ws, wsb, None)
    assert call(dk=15) in (INVALID, UNSUPPORTED)
    assert call(dv=1026) == UNSUPPORTED
    assert call(chunk=0) == INVALID
    assert call(gamma=_f([0.9, -0.1])) == INVALID
    assert call(wsb=need - 1) == WORKSPACE
    assert call(dq=FAKE) == INVALID  # a gradient overlapping an input


def test_backward_with_forward_states_rejects():
    """The backward that reuses a forward call's segment states validates that
    workspace too: NULL or misaligned, too small for the forward's states, or
    overlapping a gradient."""
    L = rn.lib()
    g = _f([0.9] * 2)
    B, H, Ln, dk, dv, chunk = 1, 2, 4096, 128, 256, 256
    need = L.retention_chunkwise_bwd_workspace_bytes(B, H, Ln, dk, dv, chunk, BF16)
    fwd_need = L.retention_chunkwise_workspace_bytes(B, H, Ln, dk, dv, chunk, BF16)
    DQ, DK_, DV_, WS, FW = (ctypes.c_void_p(a << 32) for a in (1, 2, 3, 4, 5))

    def call(fw=FW, fwb=fwd_need, dq=DQ):
        return L.retention_chunkwise_bwd_saved(FAKE, FAKE2, FAKE3, FAKE4, dq, DK_, DV_, B, H, Ln, dk, dv, chunk, g,
                                               None, 0, BF16, BF16, fw, fwb, WS, need, None)
    assert call(fw=ctypes.c_void_p(0)) == INVALID
    assert call(fw=ctypes.c_void_p((5 << 32) + 8)) == INVALID  # not 16-byte aligned
    assert call(fwb=fwd_need // 2) == WORKSPACE
    assert b"forward workspace" in L.retention_last_error()
    assert call(dq=FW) == INVALID  # a gradient overlapping the forward's states
    assert call(fw=WS) == INVALID  # the forward's states inside the backward's workspace
    assert b"overlaps the backward" in L.retention_last_error()


def test_block_rejects():
    L = rn.lib()
    g = _f([0.9] * 2)
    INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
    need = L.retnet_block_fwd_workspace_bytes(1, 64, 256, 2, 64, 128, 512, 64)
    assert need > L.msr_layer_fwd_workspace_bytes(1, 64, 256, 2, 64, 128, 64)

    def call(d_ffn=512, ln_eps=1e-5, wsb=need, w_1=FAKE3):
        return L.retnet_block_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, w_1, FAKE3, FAKE2, 1, 64, 256, 2, 64, 128,
                                  d_ffn, 64, g, None, 0, 1e-5, ln_eps, FAKE4, wsb, None)
    assert call(d_ffn=500) == UNSUPPORTED
    assert call(ln_eps=-1.0) == INVALID
    assert call(w_1=None) == INVALID
    assert call(wsb=need - 1) == WORKSPACE


@pytest.mark.parametrize("B,H,L,dk,dv,ind", [(1, 8, 32768, 128, 256, BF16), (4, 8, 4096, 256, 512, BF16),
                                            (1, 2, 200, 16, 16, F32), (2, 8, 700, 256, 512, BF16)])
def test_chunk_longer_than_sequence_is_the_sequence(B, H, L, dk, dv, ind):
    """A chunk longer than L plans exactly like chunk = L (one chunk), with no int
    overflow in the planning arithmetic, for every query that takes a chunk size."""
    lib = rn.lib()
    big = (2 ** 31 - 1, 4 * L, L + 1)
    ref = lib.retention_chunkwise_workspace_bytes(B, H, L, dk, dv, L, ind)
    assert ref > 0
    for c in big:
        assert lib.retention_chunkwise_workspace_bytes(B, H, L, dk, dv, c, ind) == ref, c
    ref = lib.retention_chunkwise_bwd_workspace_bytes(B, H, L, dk, dv, L, ind)
    for c in big:
        assert lib.retention_chunkwise_bwd_workspace_bytes(B, H, L, dk, dv, c, ind) == ref, c
    if ind == BF16:
        dm = 2048
        ref = lib.msr_layer_fwd_workspace_bytes(B, L, dm, H, dk, dv, L)
        assert ref > 0
        for c in big:
            assert lib.msr_layer_fwd_workspace_bytes(B, L, dm, H, dk, dv, c) == ref, c
            assert (lib.retnet_block_fwd_workspace_bytes(B, L, dm, H, dk, dv, 4096, c) ==
                    lib.retnet_block_fwd_workspace_bytes(B, L, dm, H, dk, dv, 4096, L)), c


def test_position_and_size_limits():
    """Positions are int32 (pos0 + L <= 2^31); at most 2^28 token-heads per call."""
    assert _par(pos0=2 ** 31 - 7) == INVALID
    assert _par(pos0=2 ** 40) == INVALID
    assert b"2^31" in rn.lib().retention_last_error()
    assert _par(B=2 ** 14, H=2, L=2 ** 14, gamma=_f([0.9, 0.5])) == UNSUPPORTED
    lib = rn.lib()
    assert lib.retention_chunkwise_workspace_bytes(2 ** 14, 2, 2 ** 14, 128, 256, 256, BF16) == 0
    g = _f([0.9] * 2)
    r = lib.msr_layer_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, 1, 8, 256, 2, 128, 256, 8, g, None, 2 ** 31 - 7,
                          1e-5, None, 0, None)
    assert r == INVALID


_STEP_NO_DEVICE = r"""
import ctypes, sys
import retentive_network_scale_amd as rn
L = rn.lib()
g = (ctypes.c_float * 2)(0.9, 0.95)
need = L.msr_layer_step_workspace_bytes(4, 256, 2, 64, 128)
P = ctypes.c_void_p
# non-overlapping stand-in addresses; the host never dereferences them and the
# first HIP call fails for want of a device
r = L.msr_layer_step(P(0x100000), P(0x100000), P(0x100000), P(0x100000), P(0x100000), P(0x100000),
                     P(0x200000), P(0x300000), P(0x400000), 1, 4, 256, 2, 64, 128, g, None, 1e-5,
                     P(0x10000000), need, None)
msg = L.retention_last_error()
print(r, msg)
sys.exit(0 if r == 4 and b"device" in msg else 1)
"""


def test_launch_error_is_reported_not_recursed():
    """A HIP failure inside the gated layer's launch sequence comes back as the
    HIP-error status with the runtime's message."""
    import subprocess
    import sys
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a host without a usable GPU: the call would launch on stand-in pointers")
    r = subprocess.run([sys.executable, "-c", _STEP_NO_DEVICE], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout[-500:], r.stderr[-500:])
