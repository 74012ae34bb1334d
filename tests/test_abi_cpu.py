"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_mi355x.h")


def _lib():
    from selective_state_space_58_amd import _binding
    import __graft_entry__
    __graft_entry__._ensure_built()
    return _binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_\w+|ssd_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib()
    names = declared_functions()
    assert {"ssm_scan_fwd", "ssm_scan_final_state", "ssd_chunk_scan_fwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_microbench_library_exports_its_header():
    # the measurement-only library (bench.py --only ubench) exports what include/ssm_microbench.h declares
    import ctypes
    from selective_state_space_58_amd import build as _build
    _lib()
    if not os.path.exists(_build.MB_LIB):
        _build.build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ssm_microbench.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ssm_mb_\w+)\s*\(", text)))
    assert len(names) == 5
    lib = ctypes.CDLL(_build.MB_LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = _lib()
    for code in range(8):
        s = lib.ssm_status_string(code)
        assert s and isinstance(s, bytes)
    assert lib.ssm_status_string(0) == b"ok"
    assert lib.ssm_status_string(99) == b"unknown status"


# fake but aligned device addresses: validation must reject before any dereference
P = 0x10000


def scan(lib, **kw):
    a = dict(x=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=0, h0=None, y=P, hf=None,
             batch=1, seqlen=4, dim=4, dstate=4, act=1, ddt=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.ssm_scan_fwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"], a["h0"],
                            a["y"], a["hf"], a["batch"], a["seqlen"], a["dim"], a["dstate"], a["act"], a["ddt"],
                            a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(delta=None), 1), (dict(A=None), 1), (dict(B=None), 1), (dict(C=None), 1),
    (dict(y=None), 1),
    (dict(batch=-1), 2), (dict(seqlen=-1), 2), (dict(dim=-2), 2), (dict(dstate=0), 2), (dict(sp=2), 2),
    (dict(batch=1 << 40, seqlen=1 << 20, dim=1 << 10), 2),
    (dict(act=5), 3), (dict(ddt=-1), 3),
    (dict(dstate=257), 4),
    (dict(x=P + 1), 7), (dict(A=P + 2), 7), (dict(h0=P + 2), 7),
])
def test_scan_argument_errors(kw, code):
    lib = _lib()
    assert scan(lib, **kw) == code
    assert lib.ssm_last_error() != b""


def scan_ex(lib, flags, **kw):
    a = dict(x=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=0, h0=None, y=P, hf=None,
             batch=1, seqlen=4, dim=4, dstate=4, act=1, ddt=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.ssm_scan_fwd_ex(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"],
                               a["h0"], a["y"], a["hf"], a["batch"], a["seqlen"], a["dim"], a["dstate"], a["act"],
                               a["ddt"], flags, a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("flags", [8, 16, 1 << 30, -1])
def test_scan_ex_rejects_unknown_flags(flags):
    lib = _lib()
    assert scan_ex(lib, flags) == 4
    assert b"flag" in lib.ssm_last_error()


@pytest.mark.parametrize("kw,code", [(dict(x=None), 1), (dict(delta=None), 1), (dict(batch=-1), 2),
                                     (dict(dstate=257), 4), (dict(ddt=5), 3), (dict(x=P + 1), 7)])
def test_scan_ex_argument_errors(kw, code):
    # every flag combination goes through the same validation as ssm_scan_fwd
    lib = _lib()
    for flags in range(8):
        assert scan_ex(lib, flags, **kw) == code, (flags, kw)


def test_empty_batch_is_noop():
    lib = _lib()
    assert scan(lib, batch=0) == 0
    assert scan(lib, dim=0) == 0


def test_final_state_requires_output():
    lib = _lib()
    rc = lib.ssm_scan_final_state(P, P, P, P, None, 0, None, None, 1, 4, 4, 4, 1, 1, None, 0, None)
    assert rc == 1


def ssd(lib, **kw):
    a = dict(x=P, dt=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=0, h0=None, y=P, hf=None,
             batch=1, seqlen=256, nheads=2, headdim=64, ngroups=1, dstate=128, chunk=256, act=1, ddt=0,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.ssd_chunk_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"],
                                  a["h0"], a["y"], a["hf"], a["batch"], a["seqlen"], a["nheads"], a["headdim"],
                                  a["ngroups"], a["dstate"], a["chunk"], a["act"], a["ddt"], a["ws"], a["wsb"],
                                  a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(nheads=3, ngroups=2), 2), (dict(headdim=-1), 2),
    (dict(act=7), 3), (dict(dstate=257), 4), (dict(dstate=1024, act=0), 4), (dict(chunk=100), 4),
    (dict(x=P + 2), 7),
])
def test_ssd_argument_errors(kw, code):
    lib = _lib()
    assert ssd(lib, **kw) == code


def test_workspace_queries():
    lib = _lib()
    assert lib.ssm_scan_workspace_bytes(0, 10, 10, 16) == 0
    # few slices, long sequence: the time-split path needs workspace
    assert lib.ssm_scan_workspace_bytes(1, 131072, 2048, 16) > 0
    assert lib.ssm_scan_workspace_bytes(8, 2048, 1536, 16) == 0
    # 129..256 states run 8 rows of 32 states per wave; 257 is unsupported
    assert lib.ssm_scan_workspace_bytes(1, 65536, 64, 256) > 0
    assert lib.ssm_scan_workspace_bytes(1, 65536, 64, 257) == 0
    # SSD: every call keeps the C B^T products of each (batch, 64-token block, group): 10 causal 16 x 16 fp32
    # tiles.  The b2 x 64-head layer fills the CUs (no split); 1 x 4 heads x 3000 tokens splits into 5 chunks
    # of 640 tokens: 5 fp32 states of 4 x 64 x 128, then 5 x 4 decay sums, each part 256-byte aligned
    cb = 10 * 256 * 4
    assert lib.ssd_workspace_bytes(2, 8192, 64, 64, 1, 128, 256) == 2 * 128 * cb
    assert lib.ssd_workspace_bytes(2, 8192, 64, 64, 4, 128, 256) == 2 * 128 * 4 * cb
    assert lib.ssd_workspace_bytes(1, 3000, 4, 64, 1, 128, 256) == 5 * 4 * 64 * 128 * 4 + 256 + 47 * cb
    assert lib.ssd_workspace_bytes(1, 500, 4, 64, 1, 128, 256) == 8 * cb   # chunks would be shorter than 8 blocks
    assert lib.ssd_workspace_bytes(1, 0, 4, 64, 1, 128, 256) == 0
    # shapes the blocked kernel does not take run the recurrence, which needs none
    assert lib.ssd_workspace_bytes(2, 8192, 64, 32, 1, 128, 256) == 0
    assert lib.ssd_workspace_bytes(2, 8192, 64, 64, 1, 16, 256) == 0


def step(lib, **kw):
    a = dict(x=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=0, state=P + 0x100000, y=P,
             batch=2, dim=8, dstate=16, act=1, ddt=1, stream=None)
    a.update(kw)
    return lib.ssm_state_update(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"],
                                a["state"], a["y"], a["batch"], a["dim"], a["dstate"], a["act"], a["ddt"],
                                a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(state=None), 1), (dict(y=None), 1), (dict(C=None), 1), (dict(A=None), 1),
    (dict(batch=-1), 2), (dict(dstate=0), 2), (dict(sp=3), 2), (dict(y=P + 0x100000), 2),
    (dict(act=2), 3), (dict(dstate=257), 4), (dict(state=P + 0x100002), 7), (dict(x=P + 1), 7),
])
def test_state_update_argument_errors(kw, code):
    lib = _lib()
    assert step(lib, **kw) == code
    assert lib.ssm_last_error() != b""


def ssd_step(lib, **kw):
    a = dict(x=P, dt=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=0, state=P + 0x100000, y=P,
             batch=2, nheads=4, headdim=64, ngroups=2, dstate=128, act=1, ddt=0, stream=None)
    a.update(kw)
    return lib.ssd_state_update(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"],
                                a["state"], a["y"], a["batch"], a["nheads"], a["headdim"], a["ngroups"], a["dstate"],
                                a["act"], a["ddt"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dt=None), 1), (dict(state=None), 1), (dict(nheads=3), 2), (dict(headdim=0), 2), (dict(nheads=-4), 2),
    (dict(ddt=9), 3), (dict(dstate=300), 4), (dict(A=P + 1), 7),
])
def test_ssd_state_update_argument_errors(kw, code):
    lib = _lib()
    assert ssd_step(lib, **kw) == code


def test_state_update_empty_is_noop():
    lib = _lib()
    assert step(lib, batch=0) == 0
    assert step(lib, dim=0) == 0
    assert ssd_step(lib, nheads=0) == 0


def conv(lib, **kw):
    a = dict(x=P, w=P, bias=None, sin=None, silu=1, out=P + 0x100000, sout=None, batch=2, seqlen=8, dim=16, width=4,
             act=1, stream=None)
    a.update(kw)
    return lib.ssm_causal_conv1d_fwd(a["x"], a["w"], a["bias"], a["sin"], a["silu"], a["out"], a["sout"], a["batch"],
                                     a["seqlen"], a["dim"], a["width"], a["act"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(out=None), 1), (dict(width=0), 2), (dict(silu=2), 2),
    (dict(seqlen=-1), 2), (dict(out=P + 8), 2), (dict(act=4), 3), (dict(width=9), 4), (dict(x=P + 1), 7),
    (dict(w=P + 2), 7),
])
def test_conv_argument_errors(kw, code):
    lib = _lib()
    assert conv(lib, **kw) == code
    assert lib.ssm_last_error() != b""


def test_conv_empty_is_noop():
    lib = _lib()
    assert conv(lib, batch=0) == 0
    assert conv(lib, dim=0) == 0


def bwd(lib, **kw):
    Q = P + 0x100000
    a = dict(x=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=0, h0=None, dout=P, dhf=None,
             dx=Q, ddelta=Q + 0x10000, dA=Q + 0x20000, dB=Q + 0x30000, dC=Q + 0x40000, dD=None, dz=None, dbias=None,
             dh0=None, batch=1, seqlen=4, dim=4, dstate=4, act=1, ddt=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.ssm_scan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"], a["h0"],
                            a["dout"], a["dhf"], a["dx"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"],
                            a["dbias"], a["dh0"], a["batch"], a["seqlen"], a["dim"], a["dstate"], a["act"], a["ddt"],
                            a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), 1), (dict(dx=None), 1), (dict(ddelta=None), 1), (dict(dA=None), 1), (dict(dB=None), 1),
    (dict(z=P), 1), (dict(D=P), 1), (dict(bias=P), 1), (dict(seqlen=-1), 2), (dict(act=3), 3),
    (dict(dstate=257), 4), (dict(dx=P + 0x100001), 7), (dict(dA=P + 0x100002), 7),
])
def test_scan_bwd_argument_errors(kw, code):
    lib = _lib()
    assert bwd(lib, **kw) == code
    assert lib.ssm_last_error() != b""


def test_scan_bwd_ex_flag_checks():
    lib = _lib()
    # x .. delta_bias, softplus, h0, dout, dh_final, dx, ddelta, dA, dB, dC, dDskip, dz, ddelta_bias, dh0,
    # batch, seqlen, dim, dstate, act, delta dtype
    base = [P] * 8 + [0] + [None, P, None, P, P, P, P, P, None, None, None, None] + [1, 4, 4, 4, 1, 1]
    for flags, code in ((8, 4), (12, 4), (1 << 20, 4)):    # unknown bits
        assert lib.ssm_scan_bwd_ex(*base, flags, None, 0, None) == code
        assert lib.ssm_last_error() != b""
    # every known flag combination goes through the same validation as ssm_scan_bwd
    bad = list(base)
    bad[0] = None
    for flags in range(8):
        assert lib.ssm_scan_bwd_ex(*bad, flags, None, 0, None) == 1


def test_scan_bwd_workspace_query():
    lib = _lib()
    # states at the start of each of the 7 16-token tiles (rounded up to 256 bytes), then the dB and dC
    # partials of the 3 groups of 16 channels per token and state
    ckpt = (7 * 2 * 40 * 16 * 4 + 255) // 256 * 256
    part = (2 * 3 * 2 * 100 * 16 * 4 + 255) // 256 * 256
    assert lib.ssm_scan_bwd_workspace_bytes(2, 100, 40, 16) == ckpt + part
    # more than 16 states: the same per-block buffers plus three fp32 accumulators of dx, ddelta, dz
    assert lib.ssm_scan_bwd_workspace_bytes(2, 100, 40, 17) == ckpt + part + 3 * 2 * 100 * 40 * 4
    assert lib.ssm_scan_bwd_workspace_bytes(2, 100, 40, 128) == ckpt + part + 3 * 2 * 100 * 40 * 4
    assert lib.ssm_scan_bwd_workspace_bytes(2, 100, 40, 256) == ckpt + part + 3 * 2 * 100 * 40 * 4
    assert lib.ssm_scan_bwd_workspace_bytes(2, 100, 40, 257) == 0
    # the _ex query: the same for the reverse / Euler flags (bits 1 and 2); one delta per token (bit 4) adds
    # the fp32 per-channel ddelta buffer; unknown bits give 0
    for flags in (0, 1, 2, 3):
        assert lib.ssm_scan_bwd_ex_workspace_bytes(2, 100, 40, 16, flags) == ckpt + part
    assert lib.ssm_scan_bwd_ex_workspace_bytes(2, 100, 40, 16, 4) == ckpt + part + 2 * 100 * 40 * 4
    assert lib.ssm_scan_bwd_ex_workspace_bytes(2, 100, 40, 17, 5) == ckpt + part + 4 * 2 * 100 * 40 * 4
    assert lib.ssm_scan_bwd_ex_workspace_bytes(2, 100, 40, 16, 8) == 0
    assert bwd(lib, batch=0) == 0


def test_train_pair_argument_checks():
    lib = _lib()
    S = P + 0x200000
    fwd = [P] * 8 + [0, None, P, None] + [1, 4, 4, 4, 1, 1]
    # the states buffer is required for a non-empty scan and must be 4-byte aligned; flags as ssm_scan_fwd_ex
    assert lib.ssm_scan_fwd_train(*fwd, 0, None, None, 0, None) == 1
    assert b"states" in lib.ssm_last_error()
    assert lib.ssm_scan_fwd_train(*fwd, 0, S + 2, None, 0, None) == 7
    assert lib.ssm_scan_fwd_train(*fwd, 8, S, None, 0, None) == 4
    empty = list(fwd)
    empty[13] = 0    # seqlen 0: nothing to save, nothing launched
    assert lib.ssm_scan_fwd_train(*empty, 0, None, None, 0, None) == 0
    bad = list(fwd)
    bad[15] = 257
    assert lib.ssm_scan_fwd_train(*bad, 0, S, None, 0, None) == 4
    # x, delta, A, B, C (no Dskip, z, delta_bias), softplus, h0, dout, dh_final, dx, ddelta, dA, dB, dC, ...
    base = [P] * 5 + [None] * 3 + [0] + [None, P, None, P, P, P, P, P, None, None, None, None] + [1, 4, 4, 4, 1, 1]
    assert lib.ssm_scan_bwd_train(*base, 0, None, None, 0, None) == 1
    assert b"states" in lib.ssm_last_error()
    assert lib.ssm_scan_bwd_train(*base, 0, S + 1, None, 0, None) == 7
    assert lib.ssm_scan_bwd_train(*base, 16, S, None, 0, None) == 4
    nox = list(base)
    nox[0] = None
    assert lib.ssm_scan_bwd_train(*nox, 0, S, None, 0, None) == 1


def test_train_pair_queries():
    lib = _lib()
    # one fp32 state per (16-token tile, batch, channel, state): ceil(100/16) = 7 tiles
    assert lib.ssm_scan_train_states_bytes(2, 100, 40, 16) == 7 * 2 * 40 * 16 * 4
    assert lib.ssm_scan_train_states_bytes(2, 96, 40, 256) == 6 * 2 * 40 * 256 * 4
    assert lib.ssm_scan_train_states_bytes(2, 100, 40, 257) == 0
    assert lib.ssm_scan_train_states_bytes(2, 0, 40, 16) == 0
    # the backward's workspace without its own stored states: the dB/dC partials (and the accumulators
    # for dstate > 16, the per-channel ddelta with one delta per token)
    part = (2 * 3 * 2 * 100 * 16 * 4 + 255) // 256 * 256
    for flags in (0, 1, 2, 3):
        assert lib.ssm_scan_bwd_train_workspace_bytes(2, 100, 40, 16, flags) == part
    assert lib.ssm_scan_bwd_train_workspace_bytes(2, 100, 40, 17, 0) == part + 3 * 2 * 100 * 40 * 4
    assert lib.ssm_scan_bwd_train_workspace_bytes(2, 100, 40, 16, 4) == part + 2 * 100 * 40 * 4
    assert lib.ssm_scan_bwd_train_workspace_bytes(2, 100, 40, 16, 8) == 0
    assert lib.ssm_scan_bwd_train_workspace_bytes(2, 100, 40, 257, 0) == 0


def scan_noalloc(lib, **kw):
    a = dict(x=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=0, h0=None, y=P, hf=None,
             batch=1, seqlen=4, dim=4, dstate=4, act=1, ddt=1, stream=None)
    a.update(kw)
    return lib.ssm_scan_fwd_noalloc(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"],
                                    a["h0"], a["y"], a["hf"], a["batch"], a["seqlen"], a["dim"], a["dstate"],
                                    a["act"], a["ddt"], a["stream"])


@pytest.mark.parametrize("kw,code", [(dict(x=None), 1), (dict(y=None), 1), (dict(batch=-1), 2), (dict(dstate=0), 2),
                                     (dict(act=5), 3), (dict(dstate=257), 4), (dict(x=P + 1), 7)])
def test_noalloc_scan_argument_errors(kw, code):
    # the same validation as ssm_scan_fwd, before anything is enqueued
    lib = _lib()
    assert scan_noalloc(lib, **kw) == code
    assert lib.ssm_last_error() != b""


def test_noalloc_scan_rejects_shapes_beyond_its_workspace():
    lib = _lib()
    cap = lib.ssm_scan_fwd_noalloc_max_workspace_bytes()
    assert cap == 32 << 20
    # 256 states on 2048 channels over 131072 tokens: the time split needs more than the fixed array
    need = lib.ssm_scan_workspace_bytes(1, 131072, 2048, 256)
    assert need > cap
    assert scan_noalloc(lib, seqlen=131072, dim=2048, dstate=256) == 5
    msg = lib.ssm_last_error()
    assert b"no-allocation" in msg and str(need).encode() in msg
    # the long-sequence layer (16 states) fits
    assert 0 < lib.ssm_scan_workspace_bytes(1, 131072, 2048, 16) <= cap
    assert scan_noalloc(lib, batch=0) == 0
