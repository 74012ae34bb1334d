"""fp64 CPU oracle for the selective scan and the SSD form -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The GPU library and its Python binding never
import it, and it imports nothing of theirs.

The arithmetic lives in ``oracle.c`` (plain C, double precision, sequential per
slice; see the header comment there for the sources and the readings taken).
This module only builds it with gcc, marshals numpy arrays, and splits
independent (batch, channel) or (batch, head) slices over host threads.

Parity pins: every function is pinned by CPU tests against closed forms, the
convolution view, limits and invariants (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            I = ctypes.c_int
            lib.oracle_selective_scan.argtypes = [P] * 8 + [I, P, P, P] + [I64] * 6
            lib.oracle_selective_scan_euler.argtypes = [P] * 8 + [I, P, P, P] + [I64] * 6
            lib.oracle_selective_scan_euler.restype = None
            lib.oracle_selective_scan.restype = None
            lib.oracle_ssd_recurrent.argtypes = [P] * 8 + [I, P, P, P] + [I64] * 8
            lib.oracle_ssd_recurrent.restype = None
            lib.oracle_ssd_quadratic.argtypes = [P] * 8 + [I, P, P] + [I64] * 8
            lib.oracle_ssd_quadratic.restype = None
            lib.oracle_lti_conv.argtypes = [P, P, P, P, ctypes.c_double, ctypes.c_double, P, I64, I64]
            lib.oracle_lti_conv.restype = None
            lib.oracle_selective_scan_bwd.argtypes = [P] * 8 + [I] + [P] * 12 + [I64] * 6
            lib.oracle_selective_scan_bwd.restype = None
            lib.oracle_selective_scan_bwd_euler.argtypes = [P] * 8 + [I] + [P] * 12 + [I64] * 6
            lib.oracle_selective_scan_bwd_euler.restype = None
            lib.oracle_causal_conv1d.argtypes = [P] * 4 + [I, P, P] + [I64] * 6
            lib.oracle_causal_conv1d.restype = None
            _lib = lib
    return _lib


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _run_slices(fn, total: int, threads: int | None):
    threads = threads or default_threads()
    threads = max(1, min(threads, total))
    if threads == 1 or total == 0:
        fn(0, total)
        return
    bounds = [total * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(threads) as ex:   # ctypes releases the GIL during each call
        list(ex.map(lambda i: fn(bounds[i], bounds[i + 1]), range(threads)))


def selective_scan(x, delta, A, B, C, Dskip=None, z=None, delta_bias=None,
                   delta_softplus=False, h0=None, want_y=True, threads=None, euler=False, reverse=False):
    """O1: y (batch, seqlen, dim) and h_final (batch, dim, dstate), both float64.
    euler: the Euler input discretization Bbar = dt * B (O1e).  reverse: the scan run over the
    time-reversed sequence, by definition flip(scan(flip(inputs))): h0 is the state before the last
    token, h_final the state after token 0, and y_t depends on tokens t .. L-1.
    delta of shape (batch, seqlen): one step size per token, read by every channel ("SSM & Mamba",
    the numpy selective SSM implementation projects one step size per token), i.e. O1 with delta
    broadcast over the channel axis."""
    if reverse:
        flip = lambda a: None if a is None else np.ascontiguousarray(np.flip(np.asarray(a, dtype=np.float64), 1))
        y, hf = selective_scan(flip(x), flip(delta), A, flip(B), flip(C), Dskip=Dskip, z=flip(z),
                               delta_bias=delta_bias, delta_softplus=delta_softplus, h0=h0, want_y=want_y,
                               threads=threads, euler=euler)
        return (flip(y) if y is not None else None), hf
    x = _f64(x)
    batch, seqlen, dim = x.shape
    A = _f64(A)
    dstate = A.shape[1]
    if np.ndim(delta) == 2:
        delta = np.repeat(_f64(delta, (batch, seqlen))[:, :, None], dim, axis=2)
    delta = _f64(delta, x.shape)
    B = _f64(B, (batch, seqlen, dstate))
    C = _f64(C, (batch, seqlen, dstate))
    Dskip = _f64(Dskip, (dim,))
    z = _f64(z, x.shape)
    delta_bias = _f64(delta_bias, (dim,))
    h0 = _f64(h0, (batch, dim, dstate))
    y = np.empty_like(x) if want_y else None
    hf = np.empty((batch, dim, dstate), dtype=np.float64)
    lib = _load()
    fn = lib.oracle_selective_scan_euler if euler else lib.oracle_selective_scan
    _run_slices(lambda s0, s1: fn(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(delta_bias),
        int(bool(delta_softplus)), _ptr(h0), _ptr(y), _ptr(hf),
        batch, seqlen, dim, dstate, s0, s1), batch * dim, threads)
    return y, hf


def selective_scan_bwd(x, delta, A, B, C, dout, Dskip=None, z=None, delta_bias=None, delta_softplus=False,
                       h0=None, dh_final=None, threads=None, euler=False, reverse=False):
    """O5: gradients of sum(dout * y) + sum(dh_final * h_final) for O1, float64.  Returns a dict with
    dx, ddelta, dA, dB, dC and, for the optional inputs given, dDskip, dz, ddelta_bias, dh0.
    Threads accumulate the shared gradients (dA, dB, dC, dDskip, ddelta_bias) in private buffers.
    euler: the gradient of O1e (O5e).  reverse: the gradient of the reversed scan flip(scan(flip)), by
    definition the flipped gradients of the scan of the flipped inputs.  delta of shape (batch, seqlen)
    (one step size per token, shared by the channels): O1 with delta broadcast over the channels, so
    ddelta is the broadcast form's ddelta summed over the channel axis (the chain rule of a broadcast)."""
    if reverse:
        flip = lambda a: None if a is None else np.ascontiguousarray(np.flip(np.asarray(a, dtype=np.float64), 1))
        g = selective_scan_bwd(flip(x), flip(delta), A, flip(B), flip(C), flip(dout), Dskip=Dskip, z=flip(z),
                               delta_bias=delta_bias, delta_softplus=delta_softplus, h0=h0, dh_final=dh_final,
                               threads=threads, euler=euler)
        for k in ("dx", "ddelta", "dB", "dC", "dz"):
            if k in g:
                g[k] = flip(g[k])
        return g
    if np.ndim(delta) == 2:
        nd = np.shape(x)[2]
        full = np.repeat(_f64(delta)[:, :, None], nd, axis=2)
        g = selective_scan_bwd(x, full, A, B, C, dout, Dskip=Dskip, z=z, delta_bias=delta_bias,
                               delta_softplus=delta_softplus, h0=h0, dh_final=dh_final, threads=threads, euler=euler)
        g["ddelta"] = g["ddelta"].sum(axis=2)
        return g
    x = _f64(x)
    batch, seqlen, dim = x.shape
    A = _f64(A)
    dstate = A.shape[1]
    delta = _f64(delta, x.shape)
    B = _f64(B, (batch, seqlen, dstate))
    C = _f64(C, (batch, seqlen, dstate))
    dout = _f64(dout, x.shape)
    Dskip = _f64(Dskip, (dim,))
    z = _f64(z, x.shape)
    delta_bias = _f64(delta_bias, (dim,))
    h0 = _f64(h0, (batch, dim, dstate))
    dh_final = _f64(dh_final, (batch, dim, dstate))
    dx = np.empty_like(x)
    ddelta = np.empty_like(x)
    dz = np.empty_like(x) if z is not None else None
    dh0 = np.empty((batch, dim, dstate)) if h0 is not None else None
    total = batch * dim
    threads = max(1, min(threads or default_threads(), total))
    bounds = [total * i // threads for i in range(threads + 1)]
    acc = [dict(dA=np.zeros((dim, dstate)), dB=np.zeros((batch, seqlen, dstate)), dC=np.zeros((batch, seqlen, dstate)),
                dD=np.zeros(dim), dbias=np.zeros(dim)) for _ in range(threads)]
    lib = _load()

    def run(i):
        a = acc[i]
        fn = lib.oracle_selective_scan_bwd_euler if euler else lib.oracle_selective_scan_bwd
        fn(
            _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(delta_bias),
            int(bool(delta_softplus)), _ptr(h0), _ptr(dout), _ptr(dh_final), _ptr(dx), _ptr(ddelta), _ptr(a["dA"]),
            _ptr(a["dB"]), _ptr(a["dC"]), _ptr(a["dD"]) if Dskip is not None else None, _ptr(dz),
            _ptr(a["dbias"]) if delta_bias is not None else None, _ptr(dh0),
            batch, seqlen, dim, dstate, bounds[i], bounds[i + 1])
    if threads == 1:
        run(0)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, range(threads)))
    out = dict(dx=dx, ddelta=ddelta, dA=sum(a["dA"] for a in acc), dB=sum(a["dB"] for a in acc),
               dC=sum(a["dC"] for a in acc))
    if Dskip is not None:
        out["dDskip"] = sum(a["dD"] for a in acc)
    if z is not None:
        out["dz"] = dz
    if delta_bias is not None:
        out["ddelta_bias"] = sum(a["dbias"] for a in acc)
    if h0 is not None:
        out["dh0"] = dh0
    return out


def _ssd_args(x, dt, A, B, C, Dskip, z, dt_bias, h0):
    x = _f64(x)
    batch, seqlen, nheads, headdim = x.shape
    B = _f64(B)
    ngroups, dstate = B.shape[2], B.shape[3]
    if nheads % ngroups:
        raise ValueError("oracle: nheads must be a multiple of ngroups")
    return (x, _f64(dt, (batch, seqlen, nheads)), _f64(A, (nheads,)), _f64(B, (batch, seqlen, ngroups, dstate)),
            _f64(C, (batch, seqlen, ngroups, dstate)), _f64(Dskip, (nheads,)), _f64(z, x.shape),
            _f64(dt_bias, (nheads,)), _f64(h0, (batch, nheads, headdim, dstate)),
            (batch, seqlen, nheads, headdim, ngroups, dstate))


def ssd_recurrent(x, dt, A, B, C, Dskip=None, z=None, dt_bias=None, dt_softplus=False,
                  h0=None, want_y=True, threads=None):
    """O2: SSD by its recurrence; y (b, L, H, P) and h_final (b, H, P, N), float64."""
    x, dt, A, B, C, Dskip, z, dt_bias, h0, dims = _ssd_args(x, dt, A, B, C, Dskip, z, dt_bias, h0)
    batch, seqlen, nheads, headdim, ngroups, dstate = dims
    y = np.empty_like(x) if want_y else None
    hf = np.empty((batch, nheads, headdim, dstate), dtype=np.float64)
    lib = _load()
    _run_slices(lambda s0, s1: lib.oracle_ssd_recurrent(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(dt_bias),
        int(bool(dt_softplus)), _ptr(h0), _ptr(y), _ptr(hf), *dims, s0, s1), batch * nheads, threads)
    return y, hf


def ssd_quadratic(x, dt, A, B, C, Dskip=None, z=None, dt_bias=None, dt_softplus=False,
                  h0=None, threads=None):
    """O2': SSD by its O(L^2) matrix form; y (b, L, H, P), float64."""
    x, dt, A, B, C, Dskip, z, dt_bias, h0, dims = _ssd_args(x, dt, A, B, C, Dskip, z, dt_bias, h0)
    batch, seqlen, nheads, headdim, ngroups, dstate = dims
    y = np.empty_like(x)
    lib = _load()
    _run_slices(lambda s0, s1: lib.oracle_ssd_quadratic(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(dt_bias),
        int(bool(dt_softplus)), _ptr(h0), _ptr(y), *dims, s0, s1), batch * nheads, threads)
    return y


def state_update(x, delta, A, B, C, state, Dskip=None, z=None, delta_bias=None, delta_softplus=False,
                 threads=None):
    """One recurrent step (O1 over a single token, starting from `state`).
    x, delta, z: (batch, dim); B, C: (batch, dstate); state: (batch, dim, dstate).
    Returns (y (batch, dim), new state (batch, dim, dstate)), float64."""
    x = _f64(x)
    one = lambda a: None if a is None else _f64(a)[:, None]
    y, hf = selective_scan(x[:, None], one(delta), A, one(B), one(C), Dskip=Dskip, z=one(z), delta_bias=delta_bias,
                           delta_softplus=delta_softplus, h0=state, threads=threads)
    return y[:, 0], hf


def ssd_state_update(x, dt, A, B, C, state, Dskip=None, z=None, dt_bias=None, dt_softplus=False, threads=None):
    """One recurrent Mamba-2 step (O2 over a single token, starting from `state`).
    x, z: (batch, nheads, headdim); dt: (batch, nheads); B, C: (batch, ngroups, dstate);
    state: (batch, nheads, headdim, dstate).  Returns (y, new state), float64."""
    x = _f64(x)
    one = lambda a: None if a is None else _f64(a)[:, None]
    y, hf = ssd_recurrent(x[:, None], one(dt), A, one(B), one(C), Dskip=Dskip, z=one(z), dt_bias=dt_bias,
                          dt_softplus=dt_softplus, h0=state, threads=threads)
    return y[:, 0], hf


def lti_conv(x, A, B, C, dt, Dskip=0.0):
    """O3: one LTI channel as a causal convolution with K_i = C Abar^i Bbar; y (seqlen,)."""
    x = _f64(x)
    A = _f64(A)
    B = _f64(B, A.shape)
    C = _f64(C, A.shape)
    y = np.empty_like(x)
    _load().oracle_lti_conv(_ptr(x), _ptr(A), _ptr(B), _ptr(C), float(dt), float(Dskip), _ptr(y),
                            x.shape[0], A.shape[0])
    return y


def causal_conv1d(x, weight, bias=None, state_in=None, silu=True, want_state=False, threads=None):
    """O4: causal depthwise conv1d (+ SiLU) of x (batch, seqlen, dim) with weight (dim, width).
    state_in: (batch, dim, width-1) inputs carried in from a previous segment (zeros if None).
    Returns out (batch, seqlen, dim) and, with want_state, state_out (batch, dim, width-1); float64."""
    x = _f64(x)
    batch, seqlen, dim = x.shape
    weight = _f64(weight)
    if weight.ndim != 2 or weight.shape[0] != dim:
        raise ValueError("oracle: weight must be (dim, width)")
    width = weight.shape[1]
    bias = _f64(bias, (dim,))
    state_in = _f64(state_in, (batch, dim, width - 1))
    out = np.empty_like(x)
    st = np.empty((batch, dim, width - 1), dtype=np.float64) if want_state else None
    lib = _load()
    _run_slices(lambda s0, s1: lib.oracle_causal_conv1d(
        _ptr(x), _ptr(weight), _ptr(bias), _ptr(state_in), int(bool(silu)), _ptr(out), _ptr(st),
        batch, seqlen, dim, width, s0, s1), batch * dim, threads)
    return (out, st) if want_state else out
