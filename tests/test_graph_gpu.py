"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph on ROCm): with the workspace
passed in and the outputs preallocated, a call enqueues only kernels (no allocation, no memset), so
launch-bound callers can capture it once and replay it.  Every replay is compared with the eager
result, with other eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import workloads

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


def replay_and_compare(fn, outs_ref, outs, exact=True, reset=None):
    """Capture fn (which writes into `outs`), replay it 4 times, check every replay."""
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on a side stream, as torch asks before capture
        if reset is not None:
            reset()
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    if reset is not None:
        reset()
    with torch.cuda.graph(g):
        fn()
    noise = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))            # stale values must not survive a replay
        if reset is not None:
            reset()
        noise.mul_(1.0001)                   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, outs_ref):
            if exact:
                assert torch.equal(o, r), rep
            else:
                assert torch.allclose(o.float(), r.float(), rtol=1e-5, atol=1e-6), rep


def test_scan_fwd_long_sequence_in_graph(ssm):
    # time-split path: chunk-state kernel, carry kernel and output pass, all in the graph
    inp = workloads.scan_inputs(1, 6000, 32, 16, dtype="bf16", seed=31, dt="softplus_bias", gate=True,
                                softplus=True, skip=True, h0=True)
    t = workloads.to_device(inp, DEV)
    nb = ssm.ssm_scan_workspace_bytes(1, 6000, 32, 16)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    y, hf = torch.empty_like(t["x"]), torch.empty((1, 32, 16), dtype=torch.float32, device=DEV)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"], workspace=ws)
    y_ref, hf_ref = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], return_final_state=True, **kw)
    fn = lambda: ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], y=y, h_final=hf, **kw)
    replay_and_compare(fn, [y_ref, hf_ref], [y, hf])


def test_ssd_time_split_in_graph(ssm):
    inp = workloads.ssd_inputs(1, 3000, 4, 64, 128, seed=32, h0=True)
    t = workloads.to_device(inp, DEV)
    nb = ssm.ssd_workspace_bytes(1, 3000, 4, 64, 1, 128, 256)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    y, hf = torch.empty_like(t["x"]), torch.empty((1, 4, 64, 128), dtype=torch.float32, device=DEV)
    y_ref, hf_ref = ssm.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], h0=t["h0"], workspace=ws,
                                           return_final_state=True)
    fn = lambda: ssm.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], h0=t["h0"], y=y, h_final=hf,
                                        workspace=ws)
    replay_and_compare(fn, [y_ref, hf_ref], [y, hf])


def test_decode_step_and_conv_in_graph(ssm):
    # one decode step (state updated in place: restored before each replay) and the conv1d update
    inp = workloads.step_inputs(8, 256, 16, dtype="bf16", seed=33)
    t = workloads.to_device(inp, DEV)
    state0 = t["state"].clone()
    state = t["state"]
    y = torch.empty_like(t["x"])
    reset = lambda: state.copy_(state0)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True)
    reset()
    y_ref = ssm.ssm_state_update(t["x"], t["delta"], t["A"], t["B"], t["C"], state, **kw).clone()
    s_ref = state.clone()
    fn = lambda: ssm.ssm_state_update(t["x"], t["delta"], t["A"], t["B"], t["C"], state, y=y, **kw)
    replay_and_compare(fn, [y_ref, s_ref], [y, state], reset=reset)

    cinp = workloads.conv_inputs(2, 300, 64, 4, dtype="bf16", seed=34, state=True)
    c = workloads.to_device(cinp, DEV)
    out, st_out = torch.empty_like(c["x"]), torch.empty_like(c["state_in"])
    o_ref, s_ref = ssm.ssm_causal_conv1d_fwd(c["x"], c["weight"], c["bias"], state_in=c["state_in"], return_state=True)
    fn = lambda: ssm.ssm_causal_conv1d_fwd(c["x"], c["weight"], c["bias"], state_in=c["state_in"], out=out,
                                           state_out=st_out)
    replay_and_compare(fn, [o_ref, s_ref], [out, st_out])


def test_backward_in_graph(ssm):
    # the backward's clears are fill kernels and its dB/dC partials live in the workspace; dA, dDskip and
    # the bias gradient use atomics, so those compare to rounding
    inp = workloads.scan_inputs(2, 300, 48, 16, dtype="bf16", seed=35, dt="softplus_bias", gate=True,
                                softplus=True, skip=True, h0=True)
    t = workloads.to_device(inp, DEV)
    dout = torch.randn_like(t["x"].float()).to(t["x"].dtype)
    nb = ssm.ssm_scan_bwd_workspace_bytes(2, 300, 48, 16)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, h0=t["h0"], workspace=ws)
    ref = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dout, **kw)
    ref = {k: v.clone() for k, v in ref.items()}
    holder = {}

    def fn():
        holder.update(ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dout, **kw))

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    for rep in range(3):
        for v in holder.values():
            v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k in ("dx", "ddelta", "dB", "dC", "dz", "dh0"):
            assert torch.equal(holder[k], ref[k]), (rep, k)
        for k in ("dA", "dD", "ddelta_bias"):
            assert torch.allclose(holder[k], ref[k], rtol=1e-5, atol=1e-5), (rep, k)
        assert np.isfinite(holder["dA"].cpu().numpy()).all()
