"""Python binding of the MI355X retention library (libretention.so).

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in include/retention.h.  torch provides device memory and
streams.  There is no fallback: if the library is not built, importing the
functions raises.

Functions (same names as the C ABI):
    retention_parallel, retention_chunkwise, retention_chunkwise_workspace_bytes,
    retention_recurrent_step, msr_layer_fwd, msr_layer_fwd_workspace_bytes
"""
import ctypes
import os

import torch

__all__ = [
    "RetentionError", "lib", "retention_parallel", "retention_chunkwise",
    "retention_chunkwise_workspace_bytes", "retention_chunkwise_noalloc", "retention_recurrent_step",
    "msr_layer_fwd",
    "msr_layer_fwd_workspace_bytes", "msr_layer_step", "msr_layer_step_workspace_bytes",
    "retention_chunkwise_bwd", "retention_chunkwise_bwd_workspace_bytes",
    "retnet_block_fwd",
    "retnet_block_fwd_workspace_bytes", "LIB_PATH",
    "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libretention.so")

RET_F32, RET_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

_vp, _i, _f, _ll, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong, ctypes.c_size_t
_fp = ctypes.POINTER(ctypes.c_float)

# name -> (restype, argtypes), mirroring include/retention.h
_SIGS = {
    "retention_abi_version": (_i, []),
    "retention_status_string": (ctypes.c_char_p, [_i]),
    "retention_last_error": (ctypes.c_char_p, []),
    "retention_parallel": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _fp, _fp, _ll, _f, _i, _i, _vp]),
    "retention_chunkwise_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "retention_chunkwise": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _fp, _fp, _ll, _vp, _vp,
                                 _f, _i, _i, _vp, _sz, _vp]),
    "retention_chunkwise_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _fp, _fp, _ll, _vp, _vp,
                                         _f, _i, _i, _vp]),
    "retention_recurrent_step": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _fp, _fp, _vp, _f, _i,
                                      _i, _vp]),
    "retention_chunkwise_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "retention_chunkwise_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _fp, _fp, _ll,
                                     _i, _i, _vp, _sz, _vp]),
    "retention_chunkwise_bwd_saved": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _fp, _fp,
                                           _ll, _i, _i, _vp, _sz, _vp, _sz, _vp]),
    "msr_layer_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "msr_layer_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _fp, _fp, _ll,
                           _f, _vp, _sz, _vp]),
    "msr_layer_step_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "retnet_block_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "retnet_block_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _fp,
                              _fp, _ll, _f, _f, _vp, _sz, _vp]),
    "msr_layer_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _fp, _fp,
                            _f, _vp, _sz, _vp]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None


class RetentionError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m retentive_network_scale_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise RetentionError(status, lib().retention_last_error().decode())


def _dt(t):
    return _dtc(t.dtype)


def _dtc(dtype):
    if dtype == torch.bfloat16:
        return RET_BF16
    if dtype == torch.float32:
        return RET_F32
    raise TypeError(f"unsupported dtype {dtype}")


def _torch_dt(code):
    return torch.bfloat16 if code == RET_BF16 else torch.float32


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _host_f32(x, n, name):
    if x is None:
        return None, None
    t = torch.as_tensor(x, dtype=torch.float32).detach().cpu().contiguous()
    if t.numel() != n:
        raise ValueError(f"{name} needs {n} values, got {t.numel()}")
    return t, ctypes.cast(t.data_ptr(), _fp)


def _stream(s):
    s = torch.cuda.current_stream() if s is None else s
    return ctypes.c_void_p(s.cuda_stream)


def _eps(gn_eps):
    return -1.0 if gn_eps is None else float(gn_eps)


def retention_parallel(q, k, v, gamma, theta=None, pos0=0, gn_eps=None, out_dtype=None, out=None,
                       stream=None):
    """O = (Q_rot K_rot^T (.) D) V per head, optional GroupNorm.  q, k [B,H,L,dk];
    v [B,H,L,dv]; gamma [H] and theta [dk/2] are host values."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    odt = _dt(q) if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=_torch_dt(odt), device=q.device)
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    _check(lib().retention_parallel(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "o"), B, H, L, dk,
                                    dv, gp, thp, int(pos0), _eps(gn_eps), _dt(q), _dt(out),
                                    _stream(stream)))
    return out


def retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk, in_dtype=torch.bfloat16):
    return int(lib().retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk,
                                                          _dt(torch.empty(0, dtype=in_dtype))))


def retention_chunkwise(q, k, v, gamma, chunk, theta=None, pos0=0, state_in=None, state_out=None,
                        gn_eps=None, out_dtype=None, out=None, workspace=None, stream=None):
    """Chunkwise recurrent form.  Returns (o, state_out); pass state_out=True to
    have a [B,H,dk,dv] fp32 final state allocated, or a tensor (may be state_in)."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    odt = _dt(q) if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=_torch_dt(odt), device=q.device)
    if state_out is True:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    need = retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk, q.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    sin = None if state_in is None else _dev(state_in, "state_in")
    sout = None if state_out is None else _dev(state_out, "state_out")
    ws = None if workspace is None else _dev(workspace, "workspace")
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().retention_chunkwise(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "o"), B, H, L, dk,
                                     dv, int(chunk), gp, thp, int(pos0), sin, sout, _eps(gn_eps), _dt(q),
                                     _dt(out), ws, wsb, _stream(stream)))
    return out, state_out


NOALLOC_SCRATCH_BYTES = 64 << 20  # RETENTION_NOALLOC_SCRATCH_BYTES of the C header


def retention_chunkwise_noalloc(q, k, v, gamma, chunk, theta=None, pos0=0, state_in=None, state_out=None,
                                gn_eps=None, out_dtype=None, out=None, stream=None):
    """retention_chunkwise with the library's own device scratch instead of a
    workspace: the C call allocates nothing.  `out` and a `state_out` tensor should
    be passed by callers that cannot allocate (as under graph capture); with None /
    True they are allocated here, before the call.  Returns (o, state_out)."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    odt = _dt(q) if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=_torch_dt(odt), device=q.device)
    if state_out is True:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    sin = None if state_in is None else _dev(state_in, "state_in")
    sout = None if state_out is None else _dev(state_out, "state_out")
    _check(lib().retention_chunkwise_noalloc(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "o"), B, H, L, dk,
                                             dv, int(chunk), gp, thp, int(pos0), sin, sout, _eps(gn_eps), _dt(q),
                                             _dt(out), _stream(stream)))
    return out, state_out


def retention_recurrent_step(q, k, v, state, pos, gamma, theta=None, gn_eps=None, out_dtype=None,
                             out=None, stream=None):
    """One decode step; updates `state` [B,H,dk,dv] fp32 in place and returns o [B,H,dv].
    pos: int32 GPU tensor [B] of absolute positions (None allowed without rotation)."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    odt = _dt(q) if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, H, dv), dtype=_torch_dt(odt), device=q.device)
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    if pos is not None and pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    pp = None if pos is None else _dev(pos, "pos")
    _check(lib().retention_recurrent_step(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(state, "state"),
                                          _dev(out, "o"), B, H, dk, dv, gp, thp, pp, _eps(gn_eps), _dt(q),
                                          _dt(out), _stream(stream)))
    return out


def msr_layer_fwd_workspace_bytes(B, L, d_model, H, dk, dv, chunk):
    return int(lib().msr_layer_fwd_workspace_bytes(B, L, d_model, H, dk, dv, chunk))


def msr_layer_fwd(x, w_q, w_k, w_v, w_g, w_o, H, dk, dv, chunk, gamma, theta=None, pos0=0, gn_eps=1e-5,
                  out=None, workspace=None, stream=None):
    """Gated multi-scale retention layer, bf16.  x [B,L,d_model]; weights stored
    [out, in]: w_q, w_k [H*dk, d_model], w_v, w_g [H*dv, d_model], w_o [d_model, H*dv]."""
    B, L, dm = x.shape
    if out is None:
        out = torch.empty((B, L, dm), dtype=torch.bfloat16, device=x.device)
    need = msr_layer_fwd_workspace_bytes(B, L, dm, H, dk, dv, chunk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    ws = None if workspace is None else _dev(workspace, "workspace")
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msr_layer_fwd(_dev(x, "x"), _dev(w_q, "w_q"), _dev(w_k, "w_k"), _dev(w_v, "w_v"),
                               _dev(w_g, "w_g"), _dev(w_o, "w_o"), _dev(out, "y"), B, L, dm, H, dk, dv,
                               int(chunk), gp, thp, int(pos0), float(gn_eps), ws, wsb, _stream(stream)))
    return out


def msr_layer_step_workspace_bytes(B, d_model, H, dk, dv):
    return int(lib().msr_layer_step_workspace_bytes(B, d_model, H, dk, dv))


def msr_layer_step(x, w_q, w_k, w_v, w_g, w_o, state, pos, H, dk, dv, gamma, theta=None, gn_eps=1e-5,
                   advance_pos=True, out=None, workspace=None, stream=None):
    """One decode step of the gated layer, bf16: x [B, d_model] (one token per
    sequence), state [B, H, dk, dv] fp32 updated in place, pos int32 [B] on the
    device (advanced by one on the device when advance_pos).  Weights as
    msr_layer_fwd.  Returns y [B, d_model]."""
    B, dm = x.shape
    if out is None:
        out = torch.empty((B, dm), dtype=torch.bfloat16, device=x.device)
    need = msr_layer_step_workspace_bytes(B, dm, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if pos.dtype != torch.int32:
        raise RetentionError(1, "pos must be int32")
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    _check(lib().msr_layer_step(_dev(x, "x"), _dev(w_q, "w_q"), _dev(w_k, "w_k"), _dev(w_v, "w_v"),
                                _dev(w_g, "w_g"), _dev(w_o, "w_o"), _dev(out, "y"), _dev(state, "state"),
                                _dev(pos, "pos"), int(bool(advance_pos)), B, dm, H, dk, dv, gp, thp,
                                float(gn_eps), _dev(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def retention_chunkwise_bwd_workspace_bytes(B, H, L, dk, dv, chunk, in_dtype=torch.bfloat16):
    return int(lib().retention_chunkwise_bwd_workspace_bytes(B, H, L, dk, dv, chunk, _dtc(in_dtype)))


def retention_chunkwise_bwd(q, k, v, d_o, gamma, chunk, theta=None, pos0=0, out_dtype=None, out=None,
                            workspace=None, stream=None, fwd_workspace=None):
    """Gradients (dq, dk, dv) of chunkwise retention (no GroupNorm, zero initial
    state) for the output gradient d_o.  q, k [B,H,L,dk]; v, d_o [B,H,L,dv].
    fwd_workspace: the workspace of the forward retention_chunkwise call on the
    same inputs (no state_in), whose segment states the dq sum then reuses
    (retention_chunkwise_bwd_saved)."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    od = out_dtype or q.dtype
    if out is None:
        out = (torch.empty((B, H, L, dk), dtype=od, device=q.device),
               torch.empty((B, H, L, dk), dtype=od, device=q.device),
               torch.empty((B, H, L, dv), dtype=od, device=q.device))
    need = retention_chunkwise_bwd_workspace_bytes(B, H, L, dk, dv, chunk, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    common = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(d_o, "d_o"), _dev(out[0], "dq"), _dev(out[1], "dk"),
              _dev(out[2], "dv"), B, H, L, dk, dv, int(chunk), gp, thp, int(pos0), _dtc(q.dtype), _dtc(od))
    tail = (_dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    if fwd_workspace is None:
        _check(lib().retention_chunkwise_bwd(*common, *tail))
    else:
        _check(lib().retention_chunkwise_bwd_saved(*common, _dev(fwd_workspace, "fwd_workspace"),
                                                   fwd_workspace.numel() * fwd_workspace.element_size(), *tail))
    return out


def retnet_block_fwd_workspace_bytes(B, L, d_model, H, dk, dv, d_ffn, chunk):
    return int(lib().retnet_block_fwd_workspace_bytes(B, L, d_model, H, dk, dv, d_ffn, chunk))


def retnet_block_fwd(x, w_q, w_k, w_v, w_g, w_o, w_1, w_2, H, dk, dv, chunk, gamma, theta=None, pos0=0,
                     gn_eps=1e-5, ln_eps=1e-5, out=None, workspace=None, stream=None):
    """Pre-LN residual block: Y = MSR(LN(x)) + x, out = gelu(LN(Y) W_1^T) W_2^T + Y (bf16).
    Weights stored [out, in]; w_1 [d_ffn, d_model], w_2 [d_model, d_ffn]."""
    B, L, dm = x.shape
    dff = w_1.shape[0]
    if out is None:
        out = torch.empty((B, L, dm), dtype=torch.bfloat16, device=x.device)
    need = retnet_block_fwd_workspace_bytes(B, L, dm, H, dk, dv, dff, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    g, gp = _host_f32(gamma, H, "gamma")
    th, thp = _host_f32(theta, dk // 2, "theta")
    _check(lib().retnet_block_fwd(_dev(x, "x"), _dev(w_q, "w_q"), _dev(w_k, "w_k"), _dev(w_v, "w_v"),
                                  _dev(w_g, "w_g"), _dev(w_o, "w_o"), _dev(w_1, "w_1"), _dev(w_2, "w_2"),
                                  _dev(out, "out"), B, L, dm, H, dk, dv, dff, int(chunk), gp, thp, int(pos0),
                                  float(gn_eps), float(ln_eps), _dev(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return out
