"""ctypes marshalling for libssm_mi355x.so (argument checks and pointers only)."""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssm_mi355x.so")
_lock = threading.Lock()
_lib = None

SSM_F32, SSM_BF16 = 0, 1
_DT = {torch.float32: SSM_F32, torch.bfloat16: SSM_BF16}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t


class SSMError(RuntimeError):
    """A non-zero status from the library (message includes its detail text)."""

    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__("%s failed: status %d (%s)" % (fn, status, detail))


def library_path() -> str:
    return _LIB_PATH


def check_library(lib_path: str = _LIB_PATH, csrc: str = _build.CSRC, include: str = _build.INCLUDE) -> None:
    """Raise unless `lib_path` was built from the sources in `csrc` and `include` (the digest the
    build embeds in the library file must equal the digest of those sources)."""
    why = _build.stale_reason(lib_path, csrc, include)
    if why is not None:
        raise RuntimeError(why + "; rebuild with __graft_entry__.build() or "
                           "python selective_state_space_58_amd/build.py")


def load_library():
    """Load the HIP library; raises if it has not been built (no fallback exists)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libssm_mi355x.so is not built; run __graft_entry__.build() or "
                               "python selective_state_space_58_amd/build.py")
        check_library(_LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.ssm_source_digest.argtypes = []
        lib.ssm_source_digest.restype = ctypes.c_char_p
        if lib.ssm_source_digest().decode() != _build.source_digest():
            raise RuntimeError("%s reports another source digest than its file holds" % _LIB_PATH)
        lib.ssm_scan_fwd.argtypes = [_P] * 8 + [_I, _P, _P, _P] + [_I64] * 4 + [_I, _I, _P, _SZ, _P]
        lib.ssm_scan_fwd.restype = _I
        lib.ssm_scan_fwd_noalloc.argtypes = [_P] * 8 + [_I, _P, _P, _P] + [_I64] * 4 + [_I, _I, _P]
        lib.ssm_scan_fwd_noalloc.restype = _I
        lib.ssm_scan_fwd_noalloc_max_workspace_bytes.argtypes = []
        lib.ssm_scan_fwd_noalloc_max_workspace_bytes.restype = _SZ
        lib.ssm_scan_fwd_ex.argtypes = [_P] * 8 + [_I, _P, _P, _P] + [_I64] * 4 + [_I, _I, _I, _P, _SZ, _P]
        lib.ssm_scan_fwd_ex.restype = _I
        lib.ssm_scan_fwd_train.argtypes = [_P] * 8 + [_I, _P, _P, _P] + [_I64] * 4 + [_I, _I, _I, _P, _P, _SZ, _P]
        lib.ssm_scan_fwd_train.restype = _I
        lib.ssm_scan_train_states_bytes.argtypes = [_I64] * 4
        lib.ssm_scan_train_states_bytes.restype = _SZ
        lib.ssm_scan_final_state.argtypes = [_P] * 5 + [_I, _P, _P] + [_I64] * 4 + [_I, _I, _P, _SZ, _P]
        lib.ssm_scan_final_state.restype = _I
        lib.ssd_chunk_scan_fwd.argtypes = [_P] * 8 + [_I, _P, _P, _P] + [_I64] * 7 + [_I, _I, _P, _SZ, _P]
        lib.ssd_chunk_scan_fwd.restype = _I
        lib.ssm_scan_workspace_bytes.argtypes = [_I64] * 4
        lib.ssm_scan_workspace_bytes.restype = _SZ
        lib.ssd_workspace_bytes.argtypes = [_I64] * 7
        lib.ssd_workspace_bytes.restype = _SZ
        lib.ssm_state_update.argtypes = [_P] * 8 + [_I, _P, _P] + [_I64] * 3 + [_I, _I, _P]
        lib.ssm_state_update.restype = _I
        lib.ssd_state_update.argtypes = [_P] * 8 + [_I, _P, _P] + [_I64] * 5 + [_I, _I, _P]
        lib.ssd_state_update.restype = _I
        lib.ssm_causal_conv1d_fwd.argtypes = [_P] * 4 + [_I, _P, _P] + [_I64] * 4 + [_I, _P]
        lib.ssm_causal_conv1d_fwd.restype = _I
        lib.ssm_scan_bwd.argtypes = [_P] * 8 + [_I] + [_P] * 12 + [_I64] * 4 + [_I, _I, _P, _SZ, _P]
        lib.ssm_scan_bwd.restype = _I
        lib.ssm_scan_bwd_ex.argtypes = [_P] * 8 + [_I] + [_P] * 12 + [_I64] * 4 + [_I, _I, _I, _P, _SZ, _P]
        lib.ssm_scan_bwd_ex.restype = _I
        lib.ssm_scan_bwd_train.argtypes = [_P] * 8 + [_I] + [_P] * 12 + [_I64] * 4 + [_I, _I, _I, _P, _P, _SZ, _P]
        lib.ssm_scan_bwd_train.restype = _I
        lib.ssm_scan_bwd_train_workspace_bytes.argtypes = [_I64] * 4 + [_I]
        lib.ssm_scan_bwd_train_workspace_bytes.restype = _SZ
        lib.ssm_scan_bwd_workspace_bytes.argtypes = [_I64] * 4
        lib.ssm_scan_bwd_workspace_bytes.restype = _SZ
        lib.ssm_scan_bwd_ex_workspace_bytes.argtypes = [_I64] * 4 + [_I]
        lib.ssm_scan_bwd_ex_workspace_bytes.restype = _SZ
        lib.ssm_status_string.argtypes = [_I]
        lib.ssm_status_string.restype = ctypes.c_char_p
        lib.ssm_last_error.argtypes = []
        lib.ssm_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(lib, fn, rc):
    if rc != 0:
        detail = lib.ssm_last_error().decode() or lib.ssm_status_string(rc).decode()
        raise SSMError(fn, rc, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _act_code(t, name):
    if t.dtype not in _DT:
        raise TypeError("%s must be float32 or bfloat16" % name)
    return _DT[t.dtype]


def ssm_scan_workspace_bytes(batch, seqlen, dim, dstate) -> int:
    return int(load_library().ssm_scan_workspace_bytes(batch, seqlen, dim, dstate))


def ssd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size) -> int:
    return int(load_library().ssd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size))


# flag bits of ssm_scan_fwd_ex (enum ssm_scan_flag)
SSM_SCAN_REVERSE = 1
SSM_SCAN_EULER = 2
SSM_SCAN_DELTA_PER_TOKEN = 4


def ssm_scan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                 return_final_state=False, y=None, h_final=None, workspace=None):
    """Selective scan forward.  x, delta, z: (batch, seqlen, dim); A: (dim, dstate) fp32;
    B, C: (batch, seqlen, dstate); D, delta_bias: (dim) fp32; h0: (batch, dim, dstate) fp32.
    Returns y, or (y, h_final) with return_final_state."""
    return _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, return_final_state, y, h_final,
                     workspace, None)


def ssm_scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                         return_final_state=False, y=None, h_final=None):
    """ssm_scan_fwd whose library call allocates nothing: the time-split chunk states live in the
    library's fixed per-GPU workspace (ssm_scan_fwd_noalloc_max_workspace_bytes()).  Outputs not
    passed are allocated here, by torch, before the call."""
    return _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, return_final_state, y, h_final,
                     None, None, noalloc=True)


def ssm_scan_fwd_noalloc_max_workspace_bytes() -> int:
    return int(load_library().ssm_scan_fwd_noalloc_max_workspace_bytes())


def ssm_scan_fwd_ex(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                    return_final_state=False, y=None, h_final=None, workspace=None, reverse=False, euler=False):
    """ssm_scan_fwd with the variant flags: reverse (scan from the last token to the first),
    euler (Bbar = dt * B).  delta may be (batch, seqlen), one step size per token for all channels."""
    flags = (SSM_SCAN_REVERSE if reverse else 0) | (SSM_SCAN_EULER if euler else 0)
    if isinstance(delta, torch.Tensor) and delta.dim() == 2:
        flags |= SSM_SCAN_DELTA_PER_TOKEN
    return _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, return_final_state, y, h_final,
                     workspace, flags)


def ssm_scan_fwd_train(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                       return_final_state=False, y=None, h_final=None, states=None, workspace=None, reverse=False,
                       euler=False):
    """ssm_scan_fwd_ex that also returns the states entering every 16th token (processing order),
    fp32 (ceil(seqlen/16), batch, dim, dstate), for ssm_scan_bwd_train.  Returns (y, states) or
    (y, h_final, states) with return_final_state."""
    flags = (SSM_SCAN_REVERSE if reverse else 0) | (SSM_SCAN_EULER if euler else 0)
    if isinstance(delta, torch.Tensor) and delta.dim() == 2:
        flags |= SSM_SCAN_DELTA_PER_TOKEN
    batch, seqlen, dim = x.shape
    dstate = A.shape[1] if A.dim() == 2 else 0
    shape = ((seqlen + 15) // 16, batch, dim, dstate)
    if states is None:
        states = torch.empty(shape, dtype=torch.float32, device=x.device)
    _need(states, "states", torch.float32, shape, x.device)
    out = _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, return_final_state, y, h_final,
                    workspace, flags, states)
    return (*out, states) if isinstance(out, tuple) else (out, states)


def ssm_scan_train_states_bytes(batch, seqlen, dim, dstate) -> int:
    return int(load_library().ssm_scan_train_states_bytes(batch, seqlen, dim, dstate))


def _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, return_final_state, y, h_final, workspace,
              flags, states=None, noalloc=False):
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    batch, seqlen, dim = x.shape
    act = _act_code(x, "x")
    per_token = flags is not None and (flags & SSM_SCAN_DELTA_PER_TOKEN) != 0
    _need(delta, "delta", shape=(batch, seqlen) if per_token else x.shape, device=dev)
    dcode = _act_code(delta, "delta")
    _need(A, "A", torch.float32, device=dev)
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (dim, dstate)")
    dstate = A.shape[1]
    _need(B, "B", x.dtype, (batch, seqlen, dstate), dev)
    _need(C, "C", x.dtype, (batch, seqlen, dstate), dev)
    _need(D, "D", torch.float32, (dim,), dev)
    _need(z, "z", x.dtype, x.shape, dev)
    _need(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _need(h0, "h0", torch.float32, (batch, dim, dstate), dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, x.shape, dev)
    if return_final_state and h_final is None:
        h_final = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    _need(h_final, "h_final", torch.float32, (batch, dim, dstate), dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(delta_softplus)), _ptr(h0), _ptr(y), _ptr(h_final), batch, seqlen, dim, dstate, act, dcode)
    if noalloc:
        rc = lib.ssm_scan_fwd_noalloc(*args, _stream(dev))
        _check(lib, "ssm_scan_fwd_noalloc", rc)
    elif states is not None:
        rc = lib.ssm_scan_fwd_train(*args, int(flags), _ptr(states), _ptr(workspace), wsb, _stream(dev))
        _check(lib, "ssm_scan_fwd_train", rc)
    elif flags is None:
        rc = lib.ssm_scan_fwd(*args, _ptr(workspace), wsb, _stream(dev))
        _check(lib, "ssm_scan_fwd", rc)
    else:
        rc = lib.ssm_scan_fwd_ex(*args, int(flags), _ptr(workspace), wsb, _stream(dev))
        _check(lib, "ssm_scan_fwd_ex", rc)
    return (y, h_final) if (return_final_state or h_final is not None) else y


def ssm_scan_final_state(x, delta, A, B, delta_bias=None, delta_softplus=False, h0=None, h_final=None,
                         workspace=None):
    """Final state h_L (batch, dim, dstate) fp32 of the selective scan, without y."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    batch, seqlen, dim = x.shape
    act = _act_code(x, "x")
    _need(delta, "delta", shape=x.shape, device=dev)
    dcode = _act_code(delta, "delta")
    _need(A, "A", torch.float32, device=dev)
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (dim, dstate)")
    dstate = A.shape[1]
    _need(B, "B", x.dtype, (batch, seqlen, dstate), dev)
    _need(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _need(h0, "h0", torch.float32, (batch, dim, dstate), dev)
    if h_final is None:
        h_final = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    _need(h_final, "h_final", torch.float32, (batch, dim, dstate), dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.ssm_scan_final_state(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(delta_bias),
                                  int(bool(delta_softplus)), _ptr(h0), _ptr(h_final),
                                  batch, seqlen, dim, dstate, act, dcode, _ptr(workspace), wsb, _stream(dev))
    _check(lib, "ssm_scan_final_state", rc)
    return h_final


def ssd_chunk_scan_fwd(x, dt, A, B, C, chunk_size=256, D=None, z=None, dt_bias=None, dt_softplus=False,
                       h0=None, return_final_state=False, y=None, h_final=None, workspace=None):
    """Mamba-2 SSD forward.  x, z: (batch, seqlen, nheads, headdim); dt: (batch, seqlen, nheads);
    A, D, dt_bias: (nheads) fp32; B, C: (batch, seqlen, ngroups, dstate);
    h0: (batch, nheads, headdim, dstate) fp32.  Returns y, or (y, h_final)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    batch, seqlen, nheads, headdim = x.shape
    act = _act_code(x, "x")
    _need(dt, "dt", shape=(batch, seqlen, nheads), device=dev)
    dcode = _act_code(dt, "dt")
    _need(A, "A", torch.float32, (nheads,), dev)
    _need(B, "B", x.dtype, device=dev)
    if B.dim() != 4 or B.shape[:2] != (batch, seqlen):
        raise ValueError("B must be (batch, seqlen, ngroups, dstate)")
    ngroups, dstate = B.shape[2], B.shape[3]
    _need(C, "C", x.dtype, B.shape, dev)
    _need(D, "D", torch.float32, (nheads,), dev)
    _need(z, "z", x.dtype, x.shape, dev)
    _need(dt_bias, "dt_bias", torch.float32, (nheads,), dev)
    _need(h0, "h0", torch.float32, (batch, nheads, headdim, dstate), dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, x.shape, dev)
    if return_final_state and h_final is None:
        h_final = torch.empty((batch, nheads, headdim, dstate), dtype=torch.float32, device=dev)
    _need(h_final, "h_final", torch.float32, (batch, nheads, headdim, dstate), dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.ssd_chunk_scan_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                                int(bool(dt_softplus)), _ptr(h0), _ptr(y), _ptr(h_final),
                                batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size, act, dcode,
                                _ptr(workspace), wsb, _stream(dev))
    _check(lib, "ssd_chunk_scan_fwd", rc)
    return (y, h_final) if (return_final_state or h_final is not None) else y


def ssm_state_update(x, delta, A, B, C, state, D=None, z=None, delta_bias=None, delta_softplus=False, y=None):
    """One recurrent step.  x, delta, z: (batch, dim); A: (dim, dstate) fp32; B, C: (batch, dstate);
    state: (batch, dim, dstate) fp32, updated in place.  Returns y (batch, dim)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    if x.dim() != 2:
        raise ValueError("x must be (batch, dim)")
    batch, dim = x.shape
    act = _act_code(x, "x")
    _need(delta, "delta", shape=x.shape, device=dev)
    dcode = _act_code(delta, "delta")
    _need(A, "A", torch.float32, device=dev)
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (dim, dstate)")
    dstate = A.shape[1]
    _need(B, "B", x.dtype, (batch, dstate), dev)
    _need(C, "C", x.dtype, (batch, dstate), dev)
    _need(state, "state", torch.float32, (batch, dim, dstate), dev)
    _need(D, "D", torch.float32, (dim,), dev)
    _need(z, "z", x.dtype, x.shape, dev)
    _need(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, x.shape, dev)
    rc = lib.ssm_state_update(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                              int(bool(delta_softplus)), _ptr(state), _ptr(y), batch, dim, dstate, act, dcode,
                              _stream(dev))
    _check(lib, "ssm_state_update", rc)
    return y


def ssd_state_update(x, dt, A, B, C, state, D=None, z=None, dt_bias=None, dt_softplus=False, y=None):
    """One recurrent Mamba-2 step.  x, z: (batch, nheads, headdim); dt: (batch, nheads);
    A, D, dt_bias: (nheads) fp32; B, C: (batch, ngroups, dstate);
    state: (batch, nheads, headdim, dstate) fp32, updated in place.  Returns y."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    if x.dim() != 3:
        raise ValueError("x must be (batch, nheads, headdim)")
    batch, nheads, headdim = x.shape
    act = _act_code(x, "x")
    _need(dt, "dt", shape=(batch, nheads), device=dev)
    dcode = _act_code(dt, "dt")
    _need(A, "A", torch.float32, (nheads,), dev)
    _need(B, "B", x.dtype, device=dev)
    if B.dim() != 3 or B.shape[0] != batch:
        raise ValueError("B must be (batch, ngroups, dstate)")
    ngroups, dstate = B.shape[1], B.shape[2]
    _need(C, "C", x.dtype, B.shape, dev)
    _need(state, "state", torch.float32, (batch, nheads, headdim, dstate), dev)
    _need(D, "D", torch.float32, (nheads,), dev)
    _need(z, "z", x.dtype, x.shape, dev)
    _need(dt_bias, "dt_bias", torch.float32, (nheads,), dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, x.shape, dev)
    rc = lib.ssd_state_update(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                              int(bool(dt_softplus)), _ptr(state), _ptr(y), batch, nheads, headdim, ngroups, dstate,
                              act, dcode, _stream(dev))
    _check(lib, "ssd_state_update", rc)
    return y


def ssm_causal_conv1d_fwd(x, weight, bias=None, state_in=None, silu=True, out=None, state_out=None,
                          return_state=False):
    """Causal depthwise conv1d (+ SiLU).  x: (batch, seqlen, dim); weight: (dim, width) fp32;
    bias: (dim) fp32; state_in/state_out: (batch, dim, width-1) in x's dtype (state_out may be
    state_in for an in-place update).  Returns out, or (out, state_out) with return_state."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, dim)")
    batch, seqlen, dim = x.shape
    act = _act_code(x, "x")
    _need(weight, "weight", torch.float32, device=dev)
    if weight.dim() != 2 or weight.shape[0] != dim:
        raise ValueError("weight must be (dim, width)")
    width = weight.shape[1]
    _need(bias, "bias", torch.float32, (dim,), dev)
    _need(state_in, "state_in", x.dtype, (batch, dim, width - 1), dev)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, x.shape, dev)
    if return_state and state_out is None:
        state_out = torch.empty((batch, dim, width - 1), dtype=x.dtype, device=dev)
    _need(state_out, "state_out", x.dtype, (batch, dim, width - 1), dev)
    rc = lib.ssm_causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(state_in), int(bool(silu)), _ptr(out),
                                   _ptr(state_out), batch, seqlen, dim, width, act, _stream(dev))
    _check(lib, "ssm_causal_conv1d_fwd", rc)
    return (out, state_out) if (return_state or state_out is not None) else out


def ssm_scan_bwd_ex(x, delta, A, B, C, dout, reverse=False, euler=False, **kw):
    """Backward of ssm_scan_fwd_ex's variants (reverse and/or euler, and delta of shape (batch, seqlen):
    one step size per token, whose ddelta is summed over the channels); the arguments of ssm_scan_bwd."""
    return ssm_scan_bwd(x, delta, A, B, C, dout, reverse=reverse, euler=euler, **kw)


def ssm_scan_bwd_train(x, delta, A, B, C, dout, states, **kw):
    """ssm_scan_bwd(_ex) that reads the states ssm_scan_fwd_train wrote for the same inputs, h0 and flags
    instead of running its own forward pass; the same arguments and results."""
    return ssm_scan_bwd(x, delta, A, B, C, dout, states=states, **kw)


def ssm_scan_bwd_train_workspace_bytes(batch, seqlen, dim, dstate, reverse=False, euler=False,
                                       delta_per_token=False) -> int:
    flags = ((SSM_SCAN_REVERSE if reverse else 0) | (SSM_SCAN_EULER if euler else 0) |
             (SSM_SCAN_DELTA_PER_TOKEN if delta_per_token else 0))
    return int(load_library().ssm_scan_bwd_train_workspace_bytes(batch, seqlen, dim, dstate, flags))


def ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate) -> int:
    return int(load_library().ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate))


def ssm_scan_bwd_ex_workspace_bytes(batch, seqlen, dim, dstate, reverse=False, euler=False, delta_per_token=False) -> int:
    flags = ((SSM_SCAN_REVERSE if reverse else 0) | (SSM_SCAN_EULER if euler else 0) |
             (SSM_SCAN_DELTA_PER_TOKEN if delta_per_token else 0))
    return int(load_library().ssm_scan_bwd_ex_workspace_bytes(batch, seqlen, dim, dstate, flags))


def ssm_scan_bwd(x, delta, A, B, C, dout, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                 dh_final=None, want_dh0=False, workspace=None, reverse=False, euler=False, states=None):
    """Gradients of sum(dout * y) + sum(dh_final * h_final) for ssm_scan_fwd with the same inputs
    (for ssm_scan_fwd_ex's reverse / euler variants when those are set: ssm_scan_bwd_ex).
    Returns a dict: dx, ddelta (input dtypes), dA, dB, dC (fp32) and, for the optional inputs given,
    dD, dz, ddelta_bias, and dh0 (with h0 or want_dh0)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    batch, seqlen, dim = x.shape
    act = _act_code(x, "x")
    per_token = isinstance(delta, torch.Tensor) and delta.dim() == 2
    _need(delta, "delta", shape=(batch, seqlen) if per_token else x.shape, device=dev)
    dcode = _act_code(delta, "delta")
    _need(A, "A", torch.float32, device=dev)
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError("A must be (dim, dstate)")
    dstate = A.shape[1]
    _need(B, "B", x.dtype, (batch, seqlen, dstate), dev)
    _need(C, "C", x.dtype, (batch, seqlen, dstate), dev)
    _need(dout, "dout", x.dtype, x.shape, dev)
    _need(D, "D", torch.float32, (dim,), dev)
    _need(z, "z", x.dtype, x.shape, dev)
    _need(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _need(h0, "h0", torch.float32, (batch, dim, dstate), dev)
    _need(dh_final, "dh_final", torch.float32, (batch, dim, dstate), dev)
    _need(states, "states", torch.float32, ((seqlen + 15) // 16, batch, dim, dstate), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty_like(x), ddelta=torch.empty_like(delta), dA=torch.empty((dim, dstate), **f32),
             dB=torch.empty((batch, seqlen, dstate), **f32), dC=torch.empty((batch, seqlen, dstate), **f32))
    if D is not None:
        g["dD"] = torch.empty((dim,), **f32)
    if z is not None:
        g["dz"] = torch.empty_like(x)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty((dim,), **f32)
    if h0 is not None or want_dh0:
        g["dh0"] = torch.empty((batch, dim, dstate), **f32)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(delta_softplus)), _ptr(h0), _ptr(dout), _ptr(dh_final), _ptr(g["dx"]), _ptr(g["ddelta"]),
            _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")), _ptr(g.get("dz")),
            _ptr(g.get("ddelta_bias")), _ptr(g.get("dh0")), batch, seqlen, dim, dstate, act, dcode)
    flags = ((SSM_SCAN_REVERSE if reverse else 0) | (SSM_SCAN_EULER if euler else 0) |
             (SSM_SCAN_DELTA_PER_TOKEN if per_token else 0))
    if states is not None:
        rc = lib.ssm_scan_bwd_train(*args, flags, _ptr(states), _ptr(workspace), wsb, _stream(dev))
        _check(lib, "ssm_scan_bwd_train", rc)
    elif flags == 0:
        rc = lib.ssm_scan_bwd(*args, _ptr(workspace), wsb, _stream(dev))
        _check(lib, "ssm_scan_bwd", rc)
    else:
        rc = lib.ssm_scan_bwd_ex(*args, flags, _ptr(workspace), wsb, _stream(dev))
        _check(lib, "ssm_scan_bwd_ex", rc)
    return g
