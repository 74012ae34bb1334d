"""Benchmark of the selective scan on one MI355X.

One step = one full selective-scan forward (discretize + recurrence + readout
+ skip, final state) over the long-sequence layer workload, the largest of the
five workloads that fits one GPU: batch 1, 2048 channels, 131072 tokens, 16
states, bf16 x/delta/B/C/y, fp32 A, skip and state, delta log-uniform in
[1e-4, 1e-1], h_final returned.  Inputs are resident in HBM before the timed
region (1.1 GB of x and delta per step, several times the 256 MB last-level
cache, so every step reads them from HBM).

Prints one JSON line with the headline throughput (token*channels/s), the
roofline of the scan measured with HIP events on the launch stream, the oracle
timed on the host cores (rank 0, N=1 only), and the other workloads (the
small fp32 layer, the 130M-like and 2.8B-like layers, SSD, decode steps,
conv1d + SiLU, the backward and the training pair).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X figures used by the roofline (vendor-published).
HBM_PEAK_GBS = 8000.0
CUS, SIMDS_PER_CU, LANES_PER_SIMD, CLOCK_GHZ = 256, 4, 16, 2.4
# VALU issue capacity in lane-slots/s: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz.
VALU_PEAK_TSLOTS = CUS * SIMDS_PER_CU * LANES_PER_SIMD * CLOCK_GHZ * 1e9 / 1e12
# Algorithmic VALU slots per (token, channel, state) element: q = dt*a, the
# ZOH gain fma, B*x, gain*(B*x), the state fma, the readout fma (6 full-rate
# ops) plus one exp, which issues at half rate on gfx950 (2 slots).
SLOTS_PER_ELEMENT = 8
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle", type=float, default=SETTLE_S,
                   help="seconds of untimed launches before the warmup steps (clocks settle)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-others", action="store_true")
    p.add_argument("--only", choices=["scan-small", "scan-130m", "scan-2.8b", "scan-long", "ssd", "step", "ssd-step",
                                      "conv", "bwd", "train", "copy", "ubench"],
                   default=None,
                   help="time only this workload (for profiling); skips the headline JSON line")
    return p.parse_args()


# The headline workload (index into workloads.CONFIGS): the long-sequence layer, the largest single-GPU one.
HEADLINE = 3

# Committed rocprofv3 summaries that carry HBM byte counters, with the sources of the kernels they cover.
# A summary's traffic figure is used only while the SHA-256 of those sources still matches the one recorded
# in it (kernel_sources_sha256_16); otherwise the traffic is reported as null.
COUNTER_SUMMARIES = {
    "scan_long": ("profiles/scan_bf16_b1_d2048_l131072_n16_hbm_counters.md",
                  ["selective_state_space_58_amd/csrc/scan_long.hip", "selective_state_space_58_amd/csrc/scan_impl.h",
                   "selective_state_space_58_amd/csrc/device_common.h"]),
    "scan_130m": ("profiles/scan_bf16_b8_d1536_l2048_n16_hbm_counters.md",
                  ["selective_state_space_58_amd/csrc/scan_impl.h", "selective_state_space_58_amd/csrc/scan_inst.hip",
                   "selective_state_space_58_amd/csrc/scan_host.hip", "selective_state_space_58_amd/csrc/device_common.h"]),
    "ssd": ("profiles/ssd_bf16_b2_h64_p64_n128_l8192_q256_kernel.md",
            ["selective_state_space_58_amd/csrc/ssd_kernels.hip", "selective_state_space_58_amd/csrc/device_common.h"]),
}


# workloads whose scan line carries the counter summary's traffic
SCAN_SUMMARY_KEYS = {"scan_bf16_b8_d1536_l2048_n16": "scan_130m", "scan_bf16_b1_d2048_l131072_n16": "scan_long"}


def sources_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE and WRITE_SIZE scaled by a
    copy-kernel calibration); None when the summary is missing or its kernels' sources changed since the
    counters were taken."""
    path, files = COUNTER_SUMMARIES[key]
    try:
        with open(os.path.join(ROOT, path)) as fh:
            text = fh.read()
    except OSError:
        return None
    d = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]{16})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if d is None or t is None or d.group(1) != sources_digest(files):
        return None
    return int(t.group(1))


def scan_bytes(cfg):
    """Algorithmic HBM bytes: every input read once, every output written once."""
    b, L, D, N = cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"]
    e = 2 if cfg["dtype"] == "bf16" else 4
    ed = 2 if cfg["delta_dtype"] == "bf16" else 4
    per_tc = e * 2 + ed + (e if cfg["gate"] else 0)            # x, y, delta, z
    per_channel = (1 if cfg["skip"] else 0) + (1 if cfg["dt"] == "softplus_bias" else 0)   # Dskip, delta bias
    total = b * L * D * per_tc + 2 * b * L * N * e + D * N * 4 + per_channel * D * 4
    if cfg.get("final_state"):
        total += b * D * N * 4
    return total


def ssd_bytes(cfg):
    b, L, H, P, N, G = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"]
    total = b * L * H * P * 2 * 2 + 2 * b * L * G * N * 2 + b * L * H * 4 + H * 4
    if cfg.get("final_state"):
        total += b * H * P * N * 4
    return total


def ssd_flops(cfg, block=None):
    """Algorithmic matrix FLOPs of the blockwise form with blocks of `block` tokens (the causal half of
    each block x block product): C B^T once per group, (C B^T o L) X, the block states B^T X and the
    off-diagonal C H.  block=None uses the workload's chunk size."""
    b, L, H, P, N, G = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"]
    Q = block or cfg["chunk"]
    blocks = L // Q
    cb = b * blocks * G * Q * Q * N * 2 / 2          # C B^T, lower triangle, once per group
    diag = b * H * blocks * Q * Q * P * 2 / 2        # (CB^T o L) X, lower triangle
    states = b * H * blocks * Q * N * P * 2          # block states
    off = b * H * blocks * Q * N * P * 2             # C H
    return cb + diag + states + off


# The SSD kernel passes the state every 64 tokens whatever chunk_size is (a block decomposition gives the
# same map for any block length), so its own algorithmic FLOPs are those of 64-token blocks.
SSD_BLOCK = 64


def step_bytes(cfg):
    """Algorithmic HBM bytes of one decode step: the fp32 state read and written once, the per-channel
    (and per-head) inputs read once, y written once."""
    e = 2 if cfg["dtype"] == "bf16" else 4
    b, N = cfg["batch"], cfg["dstate"]
    if cfg["kind"] == "step":
        D = cfg["dim"]
        ed = 2 if cfg.get("delta_dtype", cfg["dtype"]) == "bf16" else 4
        return (8 * b * D * N + 4 * D * N + b * D * (e * (3 if cfg["gate"] else 2) + ed) + 2 * b * N * e
                + 8 * D)
    H, P, G = cfg["nheads"], cfg["headdim"], cfg["ngroups"]
    edt = 2 if cfg["dt_dtype"] == "bf16" else 4
    return (8 * b * H * P * N + b * H * P * e * (3 if cfg["gate"] else 2) + b * H * edt + 2 * b * G * N * e
            + 12 * H)


SETTLE_S = 0.5


def graph_call_ms(fn, torch, reps=50, replays=5):
    """GPU time per call of fn with `reps` calls recorded once in a HIP graph and replayed, so that no host
    launch gap sits between the kernels (the eager timing of a kernel of a few tens of microseconds includes
    the binding's host work per call).  The calls must allocate nothing and record no memset."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * reps)
    del g
    return ms


def time_calls(fn, steps, warmup, torch, settle_s=None):
    """Run fn(i) for settle_s seconds of wall time and then warmup times, untimed; then `steps` times
    bracketed by events.  Returns (total_ms, [per-call ms]).  The settle phase is there because the GPU's
    clocks rise over the first tenths of a second of sustained work: the headline scan measured 0.20 ms
    per launch right after start and 0.168 ms after about 0.3 s of launches."""
    settle_s = SETTLE_S if settle_s is None else settle_s
    t_end = time.perf_counter() + settle_s
    i = 0
    while time.perf_counter() < t_end:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(st)
    for i in range(steps):
        evs[i].record(st)
        fn(i)
    evs[steps].record(st)
    end.record(st)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return start.elapsed_time(end), per


def run_microbench(workloads):
    """Measured unit rates (libssm_microbench.so) and the scan ceilings they imply."""
    import ctypes
    from selective_state_space_58_amd import build as _build
    lib = ctypes.CDLL(_build.MB_LIB)
    for name in ("ssm_mb_fma_rate", "ssm_mb_exp_rate", "ssm_mb_scan_element_rate", "ssm_mb_mfma_bf16_flops"):
        getattr(lib, name).restype = ctypes.c_double
        getattr(lib, name).argtypes = []
    lib.ssm_mb_copy_bytes_per_s.restype = ctypes.c_double
    lib.ssm_mb_copy_bytes_per_s.argtypes = [ctypes.c_size_t]
    fma, ex, el = lib.ssm_mb_fma_rate(), lib.ssm_mb_exp_rate(), lib.ssm_mb_scan_element_rate()
    mfma, copy = lib.ssm_mb_mfma_bf16_flops(), lib.ssm_mb_copy_bytes_per_s(1 << 30)
    if min(fma, ex, el, mfma, copy) <= 0:
        raise RuntimeError("a microbenchmark failed")
    out = {"fma_T_lane_ops_s": round(fma / 1e12, 3), "exp_T_lane_ops_s": round(ex / 1e12, 3),
           "scan_element_T_s": round(el / 1e12, 4), "mfma_bf16_TFLOPs": round(mfma / 1e12, 1),
           "copy_GBs_read_plus_write": round(copy / 1e9, 1),
           "published": {"valu_T_lane_slots_s": round(VALU_PEAK_TSLOTS, 3), "mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                         "hbm_GBs": HBM_PEAK_GBS}}
    # floor of each scan workload at the measured per-element rate (one exp + six VALU ops per element)
    ceil = {}
    for cfg in workloads.CONFIGS:
        if cfg["kind"] != "scan":
            continue
        elems = cfg["batch"] * cfg["seqlen"] * cfg["dim"] * cfg["dstate"]
        ceil[cfg["name"]] = {"elements": elems, "valu_floor_ms": round(elems / el * 1e3, 4),
                             "hbm_floor_ms_measured_copy": round(scan_bytes(cfg) / copy * 1e3, 4)}
    out["scan_ceilings"] = ceil
    return out


def _pct(per, q, np):
    return round(float(np.percentile(per, q)), 5)


def run_scan(oi, steps, warmup, ssm, workloads, torch, dev, np, ncopy=1):
    """Time ssm_scan_fwd on scan workload `oi` through the C ABI (outputs and workspace preallocated, `ncopy`
    rotating input copies).  Returns the per-call event times and the derived rates."""
    inp, cfg = workloads.config_inputs(oi)
    copies = [workloads.to_device(inp, dev) for _ in range(ncopy)]
    del inp
    y = torch.empty_like(copies[0]["x"])
    hf = torch.empty((cfg["batch"], cfg["dim"], cfg["dstate"]), dtype=torch.float32, device=dev)
    nb = ssm.ssm_scan_workspace_bytes(cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"])
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    sp = copies[0]["meta"]["softplus"]
    want_hf = bool(cfg.get("final_state"))

    def fn(i):
        t = copies[i % ncopy]
        ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                         delta_softplus=sp, y=y, h_final=hf if want_hf else None, workspace=ws)
    tot, per = time_calls(fn, steps, warmup, torch)
    ms = tot / steps
    kern_ms = float(np.mean(per))
    tc = cfg["batch"] * cfg["seqlen"] * cfg["dim"]
    elems = tc * cfg["dstate"]
    nbytes = scan_bytes(cfg)
    slots = elems * SLOTS_PER_ELEMENT / (kern_ms * 1e-3) / 1e12
    res = {"name": cfg["name"], "ms": round(ms, 5), "Gtc_s": round(tc / (ms * 1e-3) / 1e9, 2),
           "kernel_ms": round(kern_ms, 5), "kernel_ms_p10": _pct(per, 10, np), "kernel_ms_p50": _pct(per, 50, np),
           "kernel_ms_p90": _pct(per, 90, np), "steps": steps,
           "hbm_frac": round(nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "valu_frac": round(slots / VALU_PEAK_TSLOTS, 4), "algorithmic_bytes": nbytes, "elements": elems,
           "workspace_bytes": nb}
    if cfg["name"] in SCAN_SUMMARY_KEYS:
        res["traffic"] = measured_traffic(SCAN_SUMMARY_KEYS[cfg["name"]])
    if kern_ms < 0.1:   # launch-bound when called eagerly: also the time per call inside a graph
        res["graph_ms"] = round(graph_call_ms(fn, torch), 5)
    del copies, y, hf, ws
    torch.cuda.empty_cache()
    return res, cfg


def run_ssd(steps, warmup, ssm, workloads, torch, dev, np):
    """Time ssd_chunk_scan_fwd on the Mamba-2 workload; HBM and MFMA rooflines of the call."""
    oinp, ocfg = workloads.config_inputs(4)
    t = workloads.to_device(oinp, dev)
    y = torch.empty_like(t["x"])
    hf = torch.empty((ocfg["batch"], ocfg["nheads"], ocfg["headdim"], ocfg["dstate"]), dtype=torch.float32, device=dev)
    nb = ssm.ssd_workspace_bytes(ocfg["batch"], ocfg["seqlen"], ocfg["nheads"], ocfg["headdim"], ocfg["ngroups"],
                                 ocfg["dstate"], ocfg["chunk"])
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)

    def sstep(i):
        ssm.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], chunk_size=ocfg["chunk"], y=y, h_final=hf,
                               workspace=ws)
    tot, per = time_calls(sstep, steps, warmup, torch)
    oms = tot / steps
    kern_ms = float(np.mean(per))
    otc = ocfg["batch"] * ocfg["seqlen"] * ocfg["nheads"] * ocfg["headdim"]
    nbytes = ssd_bytes(ocfg)
    fl64 = ssd_flops(ocfg, SSD_BLOCK)
    flq = ssd_flops(ocfg)
    hbm = nbytes / (kern_ms * 1e-3) / 1e9
    tf = fl64 / (kern_ms * 1e-3) / 1e12
    res = {"name": ocfg["name"], "ms": round(oms, 5), "Gtc_s": round(otc / (oms * 1e-3) / 1e9, 2),
           "kernel_ms": round(kern_ms, 5), "kernel_ms_p50": _pct(per, 50, np), "steps": steps,
           "roofline_hbm": {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(hbm / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
                            "traffic": measured_traffic("ssd")},
           "roofline_mfma": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s (bf16 dense; algorithmic FLOPs of the 64-token blocks the kernel runs)",
                             "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": fl64,
                             "frac_if_counted_as_256_token_chunks": round(
                                 flq / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                             "flops_256_token_chunks": flq},
           "note": "one call = the C B^T pre-pass and the fused SSD kernel"}
    return res


def run_step(si, steps, warmup, ssm, workloads, torch, dev):
    """Time one decode-step workload (state updated in place on every call)."""
    inp, cfg = workloads.step_config_inputs(si)
    t = workloads.to_device(inp, dev)
    y = torch.empty_like(t["x"])
    sp = inp["meta"]["softplus"]
    if cfg["kind"] == "step":
        def fn(i):
            ssm.ssm_state_update(t["x"], t["delta"], t["A"], t["B"], t["C"], t["state"], D=t["D"], z=t["z"],
                                 delta_bias=t["delta_bias"], delta_softplus=sp, y=y)
        chans = cfg["batch"] * cfg["dim"]
    else:
        def fn(i):
            ssm.ssd_state_update(t["x"], t["dt"], t["A"], t["B"], t["C"], t["state"], D=t["D"], z=t["z"],
                                 dt_bias=t["dt_bias"], dt_softplus=sp, y=y)
        chans = cfg["batch"] * cfg["nheads"] * cfg["headdim"]
    tot, _ = time_calls(fn, steps, warmup, torch)
    ms = tot / steps
    nb = step_bytes(cfg)
    gms = graph_call_ms(fn, torch)
    return {"name": cfg["name"], "us": round(ms * 1e3, 2), "Gchannel_steps_s": round(chans / (ms * 1e-3) / 1e9, 2),
            "hbm_GBs": round(nb / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "graph_us": round(gms * 1e3, 2), "graph_hbm_frac": round(nb / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def run_conv(ci, steps, warmup, ssm, workloads, torch, dev):
    """Time the causal conv1d + SiLU on its workload (x read once, out written once)."""
    cfg = workloads.CONV_CONFIGS[ci]
    inp = workloads.conv_inputs(seed=242 + ci, **cfg)
    t = workloads.to_device(inp, dev)
    out = torch.empty_like(t["x"])

    def fn(i):
        ssm.ssm_causal_conv1d_fwd(t["x"], t["weight"], t["bias"], out=out)
    tot, _ = time_calls(fn, steps, warmup, torch)
    ms = tot / steps
    e = 2 if cfg["dtype"] == "bf16" else 4
    tc = cfg["batch"] * cfg["seqlen"] * cfg["dim"]
    nb = 2 * tc * e + cfg["dim"] * (cfg["width"] + 1) * 4
    gms = graph_call_ms(fn, torch)
    return {"name": cfg["name"], "us": round(ms * 1e3, 2), "Gtc_s": round(tc / (ms * 1e-3) / 1e9, 2),
            "hbm_GBs": round(nb / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "graph_us": round(gms * 1e3, 2), "graph_hbm_frac": round(nb / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def run_bwd(steps, warmup, ssm, workloads, torch, dev, np):
    """Time the selective-scan backward on the headline layer (all gradients)."""
    inp, cfg = workloads.config_inputs(1)
    t = workloads.to_device(inp, dev)
    rng = np.random.default_rng(7)
    dout = torch.from_numpy(workloads.round_to(rng.standard_normal(inp["x"].shape, dtype=np.float32), "bf16")).to(
        dev, torch.bfloat16)
    nb = ssm.ssm_scan_bwd_workspace_bytes(cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"])
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)

    def fn(i):
        ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dout, D=t["D"], z=t["z"],
                         delta_bias=t["delta_bias"], delta_softplus=True, workspace=ws)
    tot, _ = time_calls(fn, steps, warmup, torch)
    ms = tot / steps
    tc = cfg["batch"] * cfg["seqlen"] * cfg["dim"]
    return {"name": "scan_bwd_" + cfg["name"][len("scan_"):], "ms": round(ms, 4),
            "Gtc_s": round(tc / (ms * 1e-3) / 1e9, 2)}


def run_train(steps, warmup, ssm, workloads, torch, dev, np):
    """Time one training step of the headline layer's scan two ways: ssm_scan_fwd + ssm_scan_bwd (the
    backward reruns the recurrence to store its tile states), and the training pair ssm_scan_fwd_train +
    ssm_scan_bwd_train (the forward stores them on the way)."""
    inp, cfg = workloads.config_inputs(1)
    t = workloads.to_device(inp, dev)
    rng = np.random.default_rng(7)
    dout = torch.from_numpy(workloads.round_to(rng.standard_normal(inp["x"].shape, dtype=np.float32), "bf16")).to(
        dev, torch.bfloat16)
    b, L, D, N = cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"]
    ws = torch.empty(max(ssm.ssm_scan_bwd_workspace_bytes(b, L, D, N), 1), dtype=torch.uint8, device=dev)
    states = torch.empty(((L + 15) // 16, b, D, N), dtype=torch.float32, device=dev)
    y = torch.empty_like(t["x"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True)

    def plain(i):
        ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], y=y, **kw)
        ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dout, workspace=ws, **kw)

    def fwd_train(i):
        ssm.ssm_scan_fwd_train(t["x"], t["delta"], t["A"], t["B"], t["C"], y=y, states=states, **kw)

    def bwd_train(i):
        ssm.ssm_scan_bwd_train(t["x"], t["delta"], t["A"], t["B"], t["C"], dout, states, workspace=ws, **kw)

    res = {"name": "scan_train_step_" + cfg["name"][len("scan_"):]}
    for key, fn in (("fwd_plus_bwd_ms", plain), ("fwd_train_ms", fwd_train), ("bwd_train_ms", bwd_train)):
        tot, _ = time_calls(fn, steps, warmup, torch)
        res[key] = round(tot / steps, 4)
    res["train_pair_ms"] = round(res["fwd_train_ms"] + res["bwd_train_ms"], 4)
    res["states_bytes"] = states.numel() * 4
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the scan's (batch, channel) slices "
              "would shard with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads
    import __graft_entry__
    __graft_entry__._ensure_built()   # builds only when the library is missing or stale
    import selective_state_space_58_amd as ssm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps, warmup = args.steps, args.warmup
    global SETTLE_S
    SETTLE_S = args.settle
    if args.only == "copy":
        # plain device copy of a known size: calibrates the HBM byte counters
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        tot, _ = time_calls(lambda i: dst.copy_(src), steps, warmup, torch)
        print(json.dumps({"only": "copy", "bytes_read_per_call": nbytes, "bytes_written_per_call": nbytes,
                          "ms": round(tot / steps, 4), "GBs_read_plus_write": round(2 * nbytes / (tot / steps * 1e-3) / 1e9, 1)}),
              flush=True)
        return
    if args.only == "ubench":
        print(json.dumps({"only": "ubench", **run_microbench(workloads)}), flush=True)
        return
    if args.only == "bwd":
        print(json.dumps({"only": "bwd", **run_bwd(steps, warmup, ssm, workloads, torch, dev, np)}), flush=True)
        return
    if args.only == "train":
        print(json.dumps({"only": "train", **run_train(steps, warmup, ssm, workloads, torch, dev, np)}), flush=True)
        return
    if args.only == "conv":
        print(json.dumps({"only": "conv", **run_conv(0, steps, warmup, ssm, workloads, torch, dev)}), flush=True)
        return
    if args.only in ("step", "ssd-step"):
        si = {"step": 0, "ssd-step": 1}[args.only]
        print(json.dumps({"only": args.only, **run_step(si, steps, warmup, ssm, workloads, torch, dev)}), flush=True)
        return
    if args.only == "ssd":
        print(json.dumps({"only": "ssd", **run_ssd(steps, warmup, ssm, workloads, torch, dev, np)}), flush=True)
        return
    if args.only is not None:
        oi = {"scan-small": 0, "scan-130m": 1, "scan-2.8b": 2, "scan-long": 3}[args.only]
        # the 130M-like layer rotates six input copies (1.2 GB, beyond the 256 MB last-level cache)
        res, _ = run_scan(oi, steps, warmup, ssm, workloads, torch, dev, np, ncopy=6 if oi == 1 else 1)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return

    # ---------------------------------------------------------------- headline workload
    res, cfg = run_scan(HEADLINE, steps, warmup, ssm, workloads, torch, dev, np)
    ms, kern_ms = res["ms"], res["kernel_ms"]
    tc = cfg["batch"] * cfg["seqlen"] * cfg["dim"]
    value = tc / (ms * 1e-3) / 1e9
    nbytes = res["algorithmic_bytes"]
    hbm_gbs = nbytes / (kern_ms * 1e-3) / 1e9
    slots = res["elements"] * SLOTS_PER_ELEMENT / (kern_ms * 1e-3) / 1e12
    out = {
        "metric": "selective-scan Gtoken*channel/s at 1 MI355X + % of HBM roofline",
        "value": round(value, 3),
        "unit": "Gtoken*channel/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": cfg["batch"], "dim": cfg["dim"], "seqlen": cfg["seqlen"],
                   "dstate": cfg["dstate"], "io_dtype": "bf16", "state_dtype": "f32", "delta": "log-uniform [1e-4, 1e-1]",
                   "softplus_dt": False, "gate": False, "skip": True, "final_state": True},
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBs": round(hbm_gbs, 1), "peak_GBs": HBM_PEAK_GBS,
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4)},
        "timing": {"call_ms_p10": res["kernel_ms_p10"], "call_ms_p50": res["kernel_ms_p50"],
                   "call_ms_p90": res["kernel_ms_p90"], "input_copies": 1,
                   "workspace_bytes": res["workspace_bytes"]},
        "roofline": {"bound": "alu", "achieved": round(slots, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                     "unit": "T VALU lane-slots/s (algorithmic: 8 per state element)",
                     "frac": round(slots / VALU_PEAK_TSLOTS, 4), "traffic": measured_traffic("scan_long"),
                     "kernel_ms": round(kern_ms, 5),
                     "timed": "HIP events around each ssm_scan_fwd call on its stream (all of the call's kernels)"},
    }

    # ---------------------------------------------------------------- other workloads
    if not args.no_others:
        others = {}
        torch.cuda.empty_cache()
        for oi in (0, 1, 2):
            r, _ = run_scan(oi, 20, 5, ssm, workloads, torch, dev, np, ncopy=6 if oi == 1 else 1)
            others[r.pop("name")] = r
        r = run_ssd(20, 5, ssm, workloads, torch, dev, np)
        others[r.pop("name")] = r
        torch.cuda.empty_cache()
        for si in range(len(workloads.STEP_CONFIGS)):
            r = run_step(si, 20, 5, ssm, workloads, torch, dev)
            others[r.pop("name")] = r
            torch.cuda.empty_cache()
        for ci in range(len(workloads.CONV_CONFIGS)):
            r = run_conv(ci, 20, 5, ssm, workloads, torch, dev)
            others[r.pop("name")] = r
            torch.cuda.empty_cache()
        r = run_bwd(20, 5, ssm, workloads, torch, dev, np)
        others[r.pop("name")] = r
        torch.cuda.empty_cache()
        r = run_train(20, 5, ssm, workloads, torch, dev, np)
        others[r.pop("name")] = r
        torch.cuda.empty_cache()
        out["other_workloads"] = others

    # ---------------------------------------------------------------- CPU baseline (oracle)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(workloads, np)
    print(json.dumps(out), flush=True)


def cpu_baseline(workloads, np):
    """The fp64 oracle timed on the host cores: the headline workload in full (every one of its 4.3e9
    state updates), the per-workload wall times of all five workloads, and one-thread figures for the
    two smallest scan workloads."""
    import oracle
    from tests.helpers import oracle_scan, oracle_ssd
    threads = oracle.default_threads()
    per = {}
    head = None
    for i, cfg in enumerate(workloads.CONFIGS):
        inp, cfg = workloads.config_inputs(i)
        t0 = time.perf_counter()
        if cfg["kind"] == "ssd":
            oracle_ssd(inp, threads=threads)
            tc = cfg["batch"] * cfg["seqlen"] * cfg["nheads"] * cfg["headdim"]
        else:
            oracle_scan(inp, threads=threads)
            tc = cfg["batch"] * cfg["seqlen"] * cfg["dim"]
        sec = time.perf_counter() - t0
        per[cfg["name"]] = {"seconds": round(sec, 3), "Gtc_s": round(tc / sec / 1e9, 5), "threads": threads}
        if i == HEADLINE:
            head = (tc, sec)
        if i in (0, 1):
            # one thread: the whole small layer, batch row 0 of the 130M-like layer
            sub = inp if i == 0 else {k: (v[:1] if k in ("x", "delta", "z", "B", "C") else v) for k, v in inp.items()}
            t1 = time.perf_counter()
            oracle_scan(sub, threads=1)
            s1 = time.perf_counter() - t1
            tc1 = tc if i == 0 else tc // cfg["batch"]
            per[cfg["name"]]["one_thread"] = {"seconds": round(s1, 3), "Gtc_s": round(tc1 / s1 / 1e9, 5),
                                              "sample": "whole workload" if i == 0 else "batch row 0"}
        del inp
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    tc, sec = head
    return {"value": round(tc / sec / 1e9, 5), "unit": "Gtoken*channel/s", "cores": threads, "kind": "oracle",
            "sample": "the whole headline workload (1 x 131072 x 2048 token-channels, 16 states, 4.3e9 state "
                      "updates), fp64, %.1f s wall" % sec,
            "per_workload": per, "host": {"cpu_model": model, "cpu_count": os.cpu_count()}}


if __name__ == "__main__":
    main()
