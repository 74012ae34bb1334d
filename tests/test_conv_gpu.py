"""GPU parity of the causal depthwise conv1d + SiLU (C ABI via the binding) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import TOL, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def ssm():
    import __graft_entry__
    __graft_entry__._ensure_built()
    import selective_state_space_58_amd as m
    m.load_library()
    torch.cuda.set_device(0)
    return m


def check(ssm, inp, silu=True, label=""):
    print("case", label, flush=True)
    tol = TOL[inp["meta"]["dtype"]]
    t = workloads.to_device(inp, DEV)
    out, st = ssm.ssm_causal_conv1d_fwd(t["x"], t["weight"], t["bias"], state_in=t["state_in"], silu=silu,
                                        return_state=True)
    torch.cuda.synchronize()
    f = workloads.to_f64(inp)
    ref, st_ref = oracle.causal_conv1d(f["x"], f["weight"], f["bias"], state_in=f["state_in"], silu=silu,
                                       want_state=True)
    e = rel_err(out.float().cpu().numpy(), ref)
    print("  out rel err %.3g (tol %g)" % (e, tol))
    assert e <= tol, (label, e)
    # the carried state is a copy of inputs: exact
    assert np.array_equal(st.float().cpu().numpy(), st_ref), label


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 100, 64, 4), (1, 17, 24, 4), (3, 5, 40, 2), (2, 33, 13, 3), (1, 1, 16, 4),
                                   (2, 64, 16, 1), (2, 40, 32, 8), (1, 2, 8, 4), (2, 3, 21, 6)])
@pytest.mark.parametrize("state", [False, True])
def test_conv_shapes(ssm, dtype, shape, state):
    b, L, D, W = shape
    inp = workloads.conv_inputs(b, L, D, W, dtype=dtype, seed=b * 100 + L + D + W, state=state)
    check(ssm, inp, label="%s %s state=%s" % (dtype, shape, state))


@pytest.mark.parametrize("silu,bias", [(False, True), (True, False), (False, False)])
def test_conv_optional_terms(ssm, silu, bias):
    inp = workloads.conv_inputs(2, 50, 48, 4, dtype="f32", seed=5, bias=bias, state=True)
    check(ssm, inp, silu=silu, label="silu=%s bias=%s" % (silu, bias))


def test_conv_empty_sequence_passes_state(ssm):
    inp = workloads.conv_inputs(2, 0, 16, 4, dtype="bf16", seed=6, state=True)
    t = workloads.to_device(inp, DEV)
    out, st = ssm.ssm_causal_conv1d_fwd(t["x"], t["weight"], t["bias"], state_in=t["state_in"], return_state=True)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 16) and torch.equal(st, t["state_in"])


def test_conv_decode_in_place_matches_whole_sequence(ssm):
    # prefill 37 tokens, then 12 single-token updates with the state updated in place
    b, L0, T, D, W = 3, 37, 12, 40, 4
    inp = workloads.conv_inputs(b, L0 + T, D, W, dtype="bf16", seed=7, state=True)
    f = workloads.to_f64(inp)
    ref = oracle.causal_conv1d(f["x"], f["weight"], f["bias"], state_in=f["state_in"])
    t = workloads.to_device(inp, DEV)
    pre, state = ssm.ssm_causal_conv1d_fwd(t["x"][:, :L0].contiguous(), t["weight"], t["bias"],
                                           state_in=t["state_in"], return_state=True)
    outs = [pre]
    for i in range(L0, L0 + T):
        outs.append(ssm.ssm_causal_conv1d_fwd(t["x"][:, i:i + 1].contiguous(), t["weight"], t["bias"],
                                              state_in=state, state_out=state)[0])
    got = torch.cat(outs, 1).float().cpu().numpy()
    torch.cuda.synchronize()
    e = rel_err(got, ref)
    print("prefill + %d in-place decode steps: rel err %.3g" % (T, e))
    assert e <= TOL["bf16"]


def test_conv_feeding_the_scan(ssm):
    # the block order: u = silu(conv(x)) is the scan's input (and its skip term)
    b, L, D, N, W = 2, 300, 48, 16, 4
    cin = workloads.conv_inputs(b, L, D, W, dtype="bf16", seed=8)
    sin = workloads.scan_inputs(b, L, D, N, dtype="bf16", seed=9, dt="softplus_bias", gate=True, softplus=True,
                                skip=True)
    fc, fs = workloads.to_f64(cin), workloads.to_f64(sin)
    u_ref = oracle.causal_conv1d(fc["x"], fc["weight"], fc["bias"])
    y_ref, _ = oracle.selective_scan(u_ref, fs["delta"], fs["A"], fs["B"], fs["C"], Dskip=fs["D"], z=fs["z"],
                                     delta_bias=fs["delta_bias"], delta_softplus=True)
    tc, ts = workloads.to_device(cin, DEV), workloads.to_device(sin, DEV)
    u = ssm.ssm_causal_conv1d_fwd(tc["x"], tc["weight"], tc["bias"])
    y = ssm.ssm_scan_fwd(u, ts["delta"], ts["A"], ts["B"], ts["C"], D=ts["D"], z=ts["z"], delta_bias=ts["delta_bias"],
                         delta_softplus=True)
    torch.cuda.synchronize()
    e = rel_err(y.float().cpu().numpy(), y_ref)
    print("conv -> scan: y rel err %.3g" % e)
    # u is rounded to bf16 between the two kernels (the block stores it in the activation dtype)
    assert e <= TOL["bf16"]


def test_full_size_conv_workload(ssm):
    inp = workloads.conv_inputs(seed=242, **workloads.CONV_CONFIGS[0])
    check(ssm, inp, label=workloads.CONV_CONFIGS[0]["name"])
