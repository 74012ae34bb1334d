"""GPU parity of the selective scan (C ABI via the binding) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import TOL, err_report, fmt_report, oracle_scan, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    import __graft_entry__
    __graft_entry__._ensure_built()
    import selective_state_space_58_amd as m
    m.load_library()
    torch.cuda.set_device(0)
    return m


DEV = torch.device("cuda:0")


def run(ssm, inp, final=True, y=None, h_final=None):
    t = workloads.to_device(inp, DEV)
    out = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           delta_bias=t["delta_bias"], delta_softplus=inp["meta"]["softplus"], h0=t["h0"],
                           return_final_state=final)
    torch.cuda.synchronize()
    if final:
        return out[0].float().cpu().numpy(), out[1].cpu().numpy()
    return out.float().cpu().numpy(), None


def check(ssm, inp, tol=None, label=""):
    print("case", label, flush=True)
    tol = tol or TOL[inp["meta"]["dtype"]]
    y, hf = run(ssm, inp)
    y_ref, h_ref = oracle_scan(inp)
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    print("  y rel err %.3g  h_final rel err %.3g  (tol %g)" % (ey, eh, tol))
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    assert ey <= tol and eh <= tol, (label, ey, eh)
    return ey, eh


def test_workload_f32_b1_d16_l256_n16(ssm):
    inp, cfg = workloads.config_inputs(0)
    check(ssm, inp, label=cfg["name"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 300, 40, 16), (2, 700, 40, 16), (3, 97, 33, 16), (1, 1, 17, 16),
                                   (1, 33, 16, 16), (2, 2000, 24, 16)])
def test_ragged_shapes_gate_softplus_h0(ssm, dtype, shape):
    b, L, D, N = shape
    inp = workloads.scan_inputs(b, L, D, N, dtype=dtype, seed=sum(shape), dt="softplus_bias", gate=True,
                                softplus=True, skip=True, h0=True)
    check(ssm, inp, label="%s %s" % (dtype, shape))


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 12, 16, 17, 32, 64, 100, 128, 129, 200, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_sizes(ssm, N, dtype):
    inp = workloads.scan_inputs(2, 150, 20, N, dtype=dtype, seed=1000 + N, dt="loguniform", gate=False,
                                skip=True, h0=True)
    check(ssm, inp, label="N=%d %s" % (N, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 21, 8, 256), (2, 150, 64, 256), (2, 70, 48, 128), (1, 90, 16, 32),
                                   (2, 100, 64, 16), (2, 100, 32, 8)])
def test_vector_tile_path_with_gate(ssm, dtype, shape):
    # channel counts that fill whole channel groups (and whole 4-wave workgroups for 64 channels) with
    # dstate equal to the lane layout's padded width: the vectorised tile loads, here with the z gate
    # (fp32 with 256 states moves two channels per x chunk)
    b, L, D, N = shape
    inp = workloads.scan_inputs(b, L, D, N, dtype=dtype, seed=sum(shape) + 97, dt="softplus_bias", gate=True,
                                softplus=True, skip=True, h0=True)
    check(ssm, inp, label="vector tiles %s %s" % (dtype, shape))


@pytest.mark.parametrize("xd,dd,per_token", [("bf16", "f32", False), ("f32", "bf16", False), ("bf16", "bf16", True),
                                              ("bf16", "f32", True), ("f32", "f32", True)])
@pytest.mark.parametrize("shape", [(2, 100, 64, 16), (1, 77, 8, 16), (8, 40, 2048, 16), (16, 24, 2048, 16),
                                   (2, 90, 32, 64), (1, 21, 8, 256), (1, 2048, 64, 16)])
def test_vector_tile_path_delta_forms(ssm, xd, dd, per_token, shape):
    # the vectorised tile loads with delta in the other dtype (its own chunks of the same channels) or one
    # delta per token (one value per chunk); the shapes pick the 16-, 8- and 4-row layouts (one state
    # per lane, two, four), the wide 4- and 8-row layouts and a time-split sequence
    b, L, D, N = shape
    inp = workloads.scan_inputs(b, L, D, N, dtype=xd, delta_dtype=dd, seed=sum(shape) + 131, dt="softplus_bias",
                                gate=True, softplus=True, skip=True, h0=True)
    if per_token:
        inp["delta"] = np.ascontiguousarray(inp["delta"][:, :, 0])
    print("case vector tiles x %s delta %s per_token=%s %s" % (xd, dd, per_token, shape), flush=True)
    t = workloads.to_device(inp, DEV)
    y, hf = ssm.ssm_scan_fwd_ex(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"], return_final_state=True)
    torch.cuda.synchronize()
    f = workloads.to_f64(inp)
    y_ref, h_ref = oracle.selective_scan(f["x"], f["delta"], f["A"], f["B"], f["C"], Dskip=f["D"], z=f["z"],
                                         delta_bias=f["delta_bias"], delta_softplus=True, h0=f["h0"])
    tol = TOL["bf16"] if "bf16" in (xd, dd) else TOL["f32"]
    ey, eh = rel_err(y.float().cpu().numpy(), y_ref), rel_err(hf.cpu().numpy(), h_ref)
    print("  y rel err %.3g  h_final rel err %.3g  (tol %g)" % (ey, eh, tol))
    assert ey <= tol and eh <= tol


@pytest.mark.parametrize("xd,dd", [("f32", "bf16"), ("bf16", "f32")])
def test_mixed_dtypes(ssm, xd, dd):
    inp = workloads.scan_inputs(2, 400, 36, 16, dtype=xd, delta_dtype=dd, seed=5, dt="softplus_bias", gate=True,
                                softplus=True, h0=True)
    check(ssm, inp, tol=TOL["bf16"] if "bf16" in (xd, dd) else TOL["f32"], label="x %s delta %s" % (xd, dd))


@pytest.mark.parametrize("dtype,L,D", [("f32", 9000, 16), ("bf16", 20000, 48), ("f32", 4127, 5)])
def test_long_sequence_time_split(ssm, dtype, L, D):
    inp = workloads.scan_inputs(1, L, D, 16, dtype=dtype, seed=L, dt="loguniform", dt_lo=1e-4, dt_hi=1e-1,
                                skip=True, gate=(dtype == "bf16"), h0=True)
    assert ssm.ssm_scan_workspace_bytes(1, L, D, 16) > 0       # exercises the chunk + carry path
    check(ssm, inp, label="long %s L=%d D=%d" % (dtype, L, D))


@pytest.mark.parametrize("dtype,N", [("bf16", 256), ("f32", 200)])
def test_wide_state_time_split(ssm, dtype, N):
    # 129..256 states (8 rows of 32 states per wave) on few channels and a long sequence: chunk states
    # computed in parallel and carried
    inp = workloads.scan_inputs(1, 6000, 16, N, dtype=dtype, seed=6000 + N, dt="loguniform", dt_lo=1e-4, dt_hi=1e-1,
                                skip=True, gate=True, h0=True)
    assert ssm.ssm_scan_workspace_bytes(1, 6000, 16, N) > 0
    check(ssm, inp, label="wide time split %s N=%d" % (dtype, N))


# Sequence lengths of one token, a few, exactly one tile and just past a power of two, each
# with and without skip and gate, softplus on and off.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 7, 64, 4097])
@pytest.mark.parametrize("skip,gate,softplus", [(False, False, False), (True, True, True)])
def test_lengths_and_optional_terms(ssm, dtype, L, skip, gate, softplus):
    inp = workloads.scan_inputs(2, L, 24, 16, dtype=dtype, seed=L * 7 + skip * 3 + gate,
                                dt="softplus_bias" if softplus else "loguniform", gate=gate, softplus=softplus,
                                skip=skip, h0=True)
    check(ssm, inp, label="L=%d %s skip=%s gate=%s softplus=%s" % (L, dtype, skip, gate, softplus))


# Lane layouts and workgroup shapes, compared in full: with 16 states and four waves per workgroup,
# 8 rows (8x2048 channels: one 4-row wave per SIMD), 16 rows (10x2048: 1.25 per SIMD) and 4 rows
# (16x2048: two per SIMD); 4 rows of wide lanes (dstate 64 and 128 at 128 / 64 channels); 16 rows
# with four waves and a ragged tile, and 16 rows with one wave per workgroup (channel groups not a
# multiple of four), each in bf16 and fp32.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(8, 100, 2048, 16), (10, 60, 2048, 16), (16, 80, 2048, 16), (2, 300, 128, 64),
                                   (2, 150, 64, 128), (2, 257, 48, 16), (3, 100, 20, 16)])
def test_workgroup_layouts(ssm, dtype, shape):
    b, L, D, N = shape
    inp = workloads.scan_inputs(b, L, D, N, dtype=dtype, seed=sum(shape) + 5, dt="softplus_bias", gate=True,
                                softplus=True, skip=True, h0=True)
    check(ssm, inp, label="layout %s %s" % (dtype, shape))


@pytest.mark.parametrize("L,N", [(300, 16), (5000, 16), (700, 256)])
def test_final_state_entry(ssm, L, N):
    inp = workloads.scan_inputs(2, L, 24, N, dtype="bf16", seed=L + N + 1, dt="softplus_bias", softplus=True, h0=True)
    t = workloads.to_device(inp, DEV)
    hf = ssm.ssm_scan_final_state(t["x"], t["delta"], t["A"], t["B"], delta_bias=t["delta_bias"],
                                  delta_softplus=True, h0=t["h0"])
    torch.cuda.synchronize()
    _, h_ref = oracle_scan(inp, want_y=False)
    assert rel_err(hf.cpu().numpy(), h_ref) <= TOL["bf16"]


@pytest.mark.parametrize("N", [16, 256])
def test_empty_sequence_passes_state(ssm, N):
    inp = workloads.scan_inputs(2, 0, 8, N, dtype="f32", seed=3, h0=True)
    y, hf = run(ssm, inp)
    assert y.shape == (2, 0, 8)
    assert np.array_equal(hf, inp["h0"])


@pytest.mark.parametrize("N", [16, 200])
def test_single_token_decode_in_place(ssm, N):
    # one token, state updated in place (h_final aliases h0): the recurrent inference step
    inp = workloads.scan_inputs(3, 1, 50, N, dtype="f32", seed=9 + N, dt="softplus_bias", gate=True, softplus=True,
                                h0=True)
    t = workloads.to_device(inp, DEV)
    state = t["h0"].clone()
    y = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                         delta_softplus=True, h0=state, h_final=state)[0]
    torch.cuda.synchronize()
    y_ref, h_ref = oracle_scan(inp)
    assert rel_err(y.cpu().numpy(), y_ref) <= TOL["f32"]
    assert rel_err(state.cpu().numpy(), h_ref) <= TOL["f32"]


def test_zero_decay_and_large_dt(ssm):
    # a == 0 entries (gain -> dt, prefix sum) and dt = 1e3 (memoryless) in one run
    inp = workloads.scan_inputs(2, 260, 20, 16, dtype="f32", seed=11, h0=True)
    inp["A"][:, ::3] = 0.0
    inp["delta"][:, 100:110, :] = 1e3
    check(ssm, inp, label="a=0 and dt=1e3")
    inp2 = workloads.scan_inputs(2, 260, 20, 16, dtype="bf16", seed=12, h0=True)
    inp2["A"][3, :] = 0.0
    inp2["A"][4, :] = -1e-4
    check(ssm, inp2, label="bf16 tiny |a|")


def test_nan_stays_in_its_channel(ssm):
    inp = workloads.scan_inputs(1, 120, 20, 16, dtype="f32", seed=13)
    inp["x"][0, 50, 7] = np.nan
    y, hf = run(ssm, inp)
    assert np.all(np.isnan(y[0, 50:, 7]))
    assert np.all(np.isfinite(np.delete(y, 7, axis=2)))
    assert np.all(np.isfinite(y[0, :50, 7]))


def test_explicit_workspace(ssm):
    inp = workloads.scan_inputs(1, 6000, 16, 16, dtype="bf16", seed=21, h0=True)
    t = workloads.to_device(inp, DEV)
    nb = ssm.ssm_scan_workspace_bytes(1, 6000, 16, 16)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    y, hf = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], h0=t["h0"],
                             return_final_state=True, workspace=ws)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle_scan(inp)
    assert rel_err(y.float().cpu().numpy(), y_ref) <= TOL["bf16"]
    small = torch.empty(max(nb - 256, 1), dtype=torch.uint8, device=DEV)
    with pytest.raises(ssm.SSMError):
        ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], workspace=small)


# ------------------------------------------------------------------ long sequences in one pass
# Few (batch, channel) slices and a long sequence: with 16 states, whole groups of 8 channels and aligned
# rows the lanes of a wave split the time axis (one pass, no workspace); otherwise the sequence is split
# into chunks computed in a first pass (workspace).  A one-byte workspace is therefore accepted only by the
# one-pass kernel, which shows which path ran.
LONG_CASES = [((1, 3000, 2048), "bf16", "bf16", True), ((2, 1100, 1024), "f32", "f32", True),
              ((4, 777, 512), "bf16", "f32", False), ((1, 2048, 4096), "bf16", "bf16", False),
              ((1, 513, 2048), "f32", "bf16", True),
              # exactly two tiles over two batch rows; whole tiles only
              ((2, 512, 2048), "bf16", "bf16", True), ((1, 1024, 2048), "bf16", "bf16", False)]


def _call_ws(ssm, t, inp, ws):
    y, hf = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             delta_bias=t["delta_bias"], delta_softplus=inp["meta"]["softplus"], h0=t["h0"],
                             return_final_state=True, workspace=ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), hf.cpu().numpy()


@pytest.mark.parametrize("shape,dtype,ddtype,gate", LONG_CASES)
def test_long_sequence_one_pass(ssm, shape, dtype, ddtype, gate):
    b, L, D = shape
    print("case one-pass long scan", shape, dtype, ddtype, "gate" if gate else "", flush=True)
    inp = workloads.scan_inputs(b, L, D, 16, dtype=dtype, delta_dtype=ddtype, seed=L + D + b,
                                dt="softplus_bias" if gate else "loguniform", dt_lo=1e-4, gate=gate, softplus=gate,
                                skip=True, h0=True)
    assert ssm.ssm_scan_workspace_bytes(b, L, D, 16) > 0     # the chunked split would need workspace
    t = workloads.to_device(inp, DEV)
    y, hf = _call_ws(ssm, t, inp, torch.empty(1, dtype=torch.uint8, device=DEV))
    y_ref, h_ref = oracle_scan(inp)
    ry, rh = err_report(y, y_ref), err_report(hf, h_ref)
    print("  " + fmt_report("y", ry) + "\n  " + fmt_report("h_final", rh), flush=True)
    assert ry["bar"] <= TOL[dtype] and rh["bar"] <= TOL[dtype]


def test_long_sequence_one_pass_matches_chunked_path(ssm):
    # the same inputs through both paths: a view two bytes off 16-byte alignment takes the chunked split
    b, L, D = 1, 1500, 2048
    inp = workloads.scan_inputs(b, L, D, 16, dtype="bf16", seed=77, dt="softplus_bias", gate=True, softplus=True,
                                skip=True, h0=True)
    t = workloads.to_device(inp, DEV)
    y1, h1 = _call_ws(ssm, t, inp, torch.empty(1, dtype=torch.uint8, device=DEV))
    xs = torch.empty(t["x"].numel() + 8, dtype=t["x"].dtype, device=DEV)
    xv = xs[1:1 + t["x"].numel()].view(t["x"].shape)
    xv.copy_(t["x"])
    t2 = dict(t)
    t2["x"] = xv
    with pytest.raises(ssm.SSMError):   # the chunked split needs its workspace
        _call_ws(ssm, t2, inp, torch.empty(1, dtype=torch.uint8, device=DEV))
    y2, h2 = _call_ws(ssm, t2, inp, None)
    y_ref, h_ref = oracle_scan(inp)
    for y, hf in ((y1, h1), (y2, h2)):
        assert rel_err(y, y_ref) <= TOL["bf16"] and rel_err(hf, h_ref) <= TOL["bf16"]
    assert rel_err(h1, h2) <= 1e-5


def test_long_sequence_one_pass_special_values(ssm):
    # a = 0 and tiny |a| (the series form of the gain), and dt = 1e3 bursts (memoryless steps)
    inp = workloads.scan_inputs(1, 1200, 2048, 16, dtype="bf16", seed=501, h0=True)
    inp["A"][::3, 5] = 0.0
    inp["A"][7, :] = -1e-4
    inp["delta"][:, 300:310, :] = 1e3
    t = workloads.to_device(inp, DEV)
    y, hf = _call_ws(ssm, t, inp, torch.empty(1, dtype=torch.uint8, device=DEV))
    y_ref, h_ref = oracle_scan(inp)
    ey, eh = rel_err(y, y_ref), rel_err(hf, h_ref)
    print("case one-pass special values: y %.3g h_final %.3g" % (ey, eh), flush=True)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


# ------------------------------------------------------------------ full-size workloads, every element
def _full_compare(label, got, ref, tol):
    rep = err_report(got, ref)
    print("  " + fmt_report(label, rep), flush=True)
    assert rep["bar"] <= tol, (label, rep)
    return rep


@pytest.mark.parametrize("index", [1, 2])
def test_full_size_layer_workloads_every_element(ssm, index):
    # the 130M-like and 2.8B-like layers: every y and every h_final element against the oracle
    inp, cfg = workloads.config_inputs(index)
    print("case", cfg["name"], "(GPU run)", flush=True)
    y, hf = run(ssm, inp, final=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    print("  oracle on %d host threads" % oracle.default_threads(), flush=True)
    y_ref, h_ref = oracle_scan(inp)
    _full_compare("y", y, y_ref, TOL["bf16"])
    _full_compare("h_final", hf, h_ref, TOL["bf16"])


def test_full_size_long_sequence_every_element(ssm):
    # the 131072-token layer (one pass with time-split lanes): the workload's own check -- every 4096th
    # output of all 2048 channels plus the whole final state -- and every other output as well
    inp, cfg = workloads.config_inputs(3)
    print("case", cfg["name"], "(GPU run)", flush=True)
    y, hf = run(ssm, inp, final=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    print("  oracle on %d host threads" % oracle.default_threads(), flush=True)
    y_ref, h_ref = oracle_scan(inp)
    L = cfg["seqlen"]
    idx = np.sort(np.concatenate([np.arange(4095, L, 4096), np.arange(0, L, 4096)]))
    _full_compare("y at every 4096th token (t = 4095 mod 4096 and t = 0 mod 4096)", y[:, idx], y_ref[:, idx],
                  TOL["bf16"])
    _full_compare("h_final", hf, h_ref, TOL["bf16"])
    _full_compare("y, every token", y, y_ref, TOL["bf16"])
