"""Seeded synthetic inputs for the selective scan and SSD workloads.

This module only draws and rounds inputs; it holds none of the scan's
arithmetic.  Both the fp64 oracle and the HIP library consume exactly the
values drawn here (bf16 tensors are rounded to nearest even once, here, and
the oracle reads those rounded values).

Distributions follow the sources' parameterisation ("Mamba / SSM complete
guide", sec. 5: A = -exp(log(1..N)) = -(n+1) per channel, dt drawn between
dt_min = 1e-3 and dt_max = 1e-1, skip initialised from a normal range; "SSM &
Mamba" experiment: seed 42) and the five workload shapes below.
"""
from __future__ import annotations

import numpy as np
import torch

# The five workloads: four selective-scan layer shapes and one SSD shape.
CONFIGS = [
    dict(name="scan_f32_b1_d16_l256_n16", kind="scan", batch=1, dim=16, seqlen=256, dstate=16, dtype="f32",
         delta_dtype="f32", dt="loguniform", dt_lo=1e-3, dt_hi=1e-1, gate=False, softplus=False, skip=True,
         final_state=False),
    dict(name="scan_bf16_b8_d1536_l2048_n16", kind="scan", batch=8, dim=1536, seqlen=2048, dstate=16, dtype="bf16",
         delta_dtype="bf16", dt="softplus_bias", dt_lo=1e-3, dt_hi=1e-1, gate=True, softplus=True, skip=True,
         final_state=False),
    dict(name="scan_bf16_b4_d5120_l4096_n16", kind="scan", batch=4, dim=5120, seqlen=4096, dstate=16, dtype="bf16",
         delta_dtype="bf16", dt="softplus_bias", dt_lo=1e-3, dt_hi=1e-1, gate=True, softplus=True, skip=True,
         final_state=True),
    dict(name="scan_bf16_b1_d2048_l131072_n16", kind="scan", batch=1, dim=2048, seqlen=131072, dstate=16,
         dtype="bf16", delta_dtype="bf16", dt="loguniform", dt_lo=1e-4, dt_hi=1e-1, gate=False, softplus=False,
         skip=True, final_state=True),
    dict(name="ssd_bf16_b2_h64_p64_n128_l8192_q256", kind="ssd", batch=2, nheads=64, headdim=64, dstate=128,
         seqlen=8192, ngroups=1, chunk=256, dtype="bf16", dt_dtype="f32", dt_lo=1e-3, dt_hi=1e-1,
         a_lo=1.0, a_hi=16.0, gate=False, skip=False, final_state=True),
]

# Single-token decode steps (recurrent inference) at serving batch sizes: the
# 2.8B-like Mamba layer (5120 channels, 16 states) and a Mamba-2 2.7B-like
# layer (80 heads of 64 channels, 128 states, one group).
STEP_CONFIGS = [
    dict(name="step_bf16_b128_d5120_n16", kind="step", batch=128, dim=5120, dstate=16, dtype="bf16",
         delta_dtype="bf16", dt_lo=1e-3, dt_hi=1e-1, gate=True, softplus=True, skip=True),
    dict(name="ssd_step_bf16_b128_h80_p64_n128", kind="ssd_step", batch=128, nheads=80, headdim=64, ngroups=1,
         dstate=128, dtype="bf16", dt_dtype="f32", dt_lo=1e-3, dt_hi=1e-1, a_lo=1.0, a_hi=16.0, gate=True,
         skip=True, dt_softplus=True),
]


def round_to(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to `dtype` ("f32" or "bf16", nearest even); returns float32 holding them."""
    a = np.ascontiguousarray(arr, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def _loguniform(rng, lo, hi, size):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=size)).astype(np.float32)


def scan_inputs(batch, seqlen, dim, dstate, dtype="bf16", delta_dtype=None, seed=0, dt="loguniform",
                dt_lo=1e-3, dt_hi=1e-1, gate=False, softplus=False, skip=True, h0=False, **_):
    """Inputs of the selective scan.  Returns a dict of float32 numpy arrays (values already
    rounded to their storage dtype) plus "meta" (dtypes and flags)."""
    delta_dtype = delta_dtype or dtype
    rng = np.random.default_rng(seed)
    out = {}
    out["A"] = np.broadcast_to(-np.arange(1, dstate + 1, dtype=np.float32), (dim, dstate)).copy()
    out["x"] = round_to(rng.standard_normal((batch, seqlen, dim), dtype=np.float32), dtype)
    if dt == "loguniform":
        out["delta"] = round_to(_loguniform(rng, dt_lo, dt_hi, (batch, seqlen, dim)), delta_dtype)
        out["delta_bias"] = None
    elif dt == "softplus_bias":
        # per-channel bias placing softplus(0 + bias) log-uniformly in [dt_lo, dt_hi]
        dt0 = _loguniform(rng, dt_lo, dt_hi, (dim,)).astype(np.float64)
        out["delta_bias"] = np.log(np.expm1(dt0)).astype(np.float32)
        out["delta"] = round_to(rng.standard_normal((batch, seqlen, dim), dtype=np.float32), delta_dtype)
    else:
        raise ValueError(dt)
    out["B"] = round_to(rng.standard_normal((batch, seqlen, dstate), dtype=np.float32), dtype)
    out["C"] = round_to(rng.standard_normal((batch, seqlen, dstate), dtype=np.float32), dtype)
    out["D"] = rng.standard_normal(dim, dtype=np.float32) if skip else None
    out["z"] = round_to(rng.standard_normal((batch, seqlen, dim), dtype=np.float32), dtype) if gate else None
    out["h0"] = rng.standard_normal((batch, dim, dstate), dtype=np.float32) if h0 else None
    out["meta"] = dict(kind="scan", dtype=dtype, delta_dtype=delta_dtype, softplus=bool(softplus))
    return out


def ssd_inputs(batch, seqlen, nheads, headdim, dstate, ngroups=1, dtype="bf16", dt_dtype="f32", seed=0,
               dt_lo=1e-3, dt_hi=1e-1, a_lo=1.0, a_hi=16.0, gate=False, skip=False, h0=False, dt_softplus=False,
               **_):
    """Inputs of the SSD form: scalar A per head ~ -U[a_lo, a_hi], dt log-uniform per (b, t, h)."""
    rng = np.random.default_rng(seed)
    out = {}
    out["x"] = round_to(rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32), dtype)
    if dt_softplus:
        dt0 = _loguniform(rng, dt_lo, dt_hi, (nheads,)).astype(np.float64)
        out["dt_bias"] = np.log(np.expm1(dt0)).astype(np.float32)
        out["dt"] = round_to(rng.standard_normal((batch, seqlen, nheads), dtype=np.float32), dt_dtype)
    else:
        out["dt_bias"] = None
        out["dt"] = round_to(_loguniform(rng, dt_lo, dt_hi, (batch, seqlen, nheads)), dt_dtype)
    out["A"] = (-rng.uniform(a_lo, a_hi, nheads)).astype(np.float32)
    out["B"] = round_to(rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32), dtype)
    out["C"] = round_to(rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32), dtype)
    out["D"] = rng.standard_normal(nheads, dtype=np.float32) if skip else None
    out["z"] = round_to(rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32), dtype) if gate else None
    out["h0"] = rng.standard_normal((batch, nheads, headdim, dstate), dtype=np.float32) if h0 else None
    out["meta"] = dict(kind="ssd", dtype=dtype, dt_dtype=dt_dtype, softplus=bool(dt_softplus))
    return out


def step_inputs(batch, dim, dstate, dtype="bf16", delta_dtype=None, seed=0, dt_lo=1e-3, dt_hi=1e-1, gate=True,
                softplus=True, skip=True, **_):
    """Inputs of one selective-scan decode step: x, delta, z (batch, dim); B, C (batch, dstate);
    state (batch, dim, dstate) ~ N(0, 1) fp32.  With softplus, delta ~ N(0, 1) plus a per-channel bias
    placing softplus(bias) log-uniformly in [dt_lo, dt_hi]; otherwise delta is log-uniform itself."""
    delta_dtype = delta_dtype or dtype
    rng = np.random.default_rng(seed)
    out = {}
    out["A"] = np.broadcast_to(-np.arange(1, dstate + 1, dtype=np.float32), (dim, dstate)).copy()
    out["x"] = round_to(rng.standard_normal((batch, dim), dtype=np.float32), dtype)
    if softplus:
        dt0 = _loguniform(rng, dt_lo, dt_hi, (dim,)).astype(np.float64)
        out["delta_bias"] = np.log(np.expm1(dt0)).astype(np.float32)
        out["delta"] = round_to(rng.standard_normal((batch, dim), dtype=np.float32), delta_dtype)
    else:
        out["delta_bias"] = None
        out["delta"] = round_to(_loguniform(rng, dt_lo, dt_hi, (batch, dim)), delta_dtype)
    out["B"] = round_to(rng.standard_normal((batch, dstate), dtype=np.float32), dtype)
    out["C"] = round_to(rng.standard_normal((batch, dstate), dtype=np.float32), dtype)
    out["D"] = rng.standard_normal(dim, dtype=np.float32) if skip else None
    out["z"] = round_to(rng.standard_normal((batch, dim), dtype=np.float32), dtype) if gate else None
    out["state"] = rng.standard_normal((batch, dim, dstate), dtype=np.float32)
    out["meta"] = dict(kind="step", dtype=dtype, delta_dtype=delta_dtype, softplus=bool(softplus))
    return out


def ssd_step_inputs(batch, nheads, headdim, dstate, ngroups=1, dtype="bf16", dt_dtype="f32", seed=0, dt_lo=1e-3,
                    dt_hi=1e-1, a_lo=1.0, a_hi=16.0, gate=True, skip=True, dt_softplus=True, **_):
    """Inputs of one Mamba-2 decode step: x, z (batch, nheads, headdim); dt (batch, nheads);
    A ~ -U[a_lo, a_hi] per head; B, C (batch, ngroups, dstate); state ~ N(0, 1) fp32."""
    rng = np.random.default_rng(seed)
    out = {}
    out["x"] = round_to(rng.standard_normal((batch, nheads, headdim), dtype=np.float32), dtype)
    if dt_softplus:
        dt0 = _loguniform(rng, dt_lo, dt_hi, (nheads,)).astype(np.float64)
        out["dt_bias"] = np.log(np.expm1(dt0)).astype(np.float32)
        out["dt"] = round_to(rng.standard_normal((batch, nheads), dtype=np.float32), dt_dtype)
    else:
        out["dt_bias"] = None
        out["dt"] = round_to(_loguniform(rng, dt_lo, dt_hi, (batch, nheads)), dt_dtype)
    out["A"] = (-rng.uniform(a_lo, a_hi, nheads)).astype(np.float32)
    out["B"] = round_to(rng.standard_normal((batch, ngroups, dstate), dtype=np.float32), dtype)
    out["C"] = round_to(rng.standard_normal((batch, ngroups, dstate), dtype=np.float32), dtype)
    out["D"] = rng.standard_normal(nheads, dtype=np.float32) if skip else None
    out["z"] = round_to(rng.standard_normal((batch, nheads, headdim), dtype=np.float32), dtype) if gate else None
    out["state"] = rng.standard_normal((batch, nheads, headdim, dstate), dtype=np.float32)
    out["meta"] = dict(kind="ssd_step", dtype=dtype, dt_dtype=dt_dtype, softplus=bool(dt_softplus))
    return out


def step_config_inputs(index: int, **overrides):
    """Inputs of decode workload `index` of STEP_CONFIGS (seed 142 + index)."""
    cfg = dict(STEP_CONFIGS[index])
    cfg.update(overrides)
    seed = 142 + index
    if cfg["kind"] == "step":
        return step_inputs(seed=seed, **cfg), cfg
    return ssd_step_inputs(seed=seed, **cfg), cfg


# Causal conv1d + SiLU feeding the scan, on the headline layer's shape (d_conv 4).
CONV_CONFIGS = [
    dict(name="conv1d_silu_bf16_b8_l2048_d1536_w4", kind="conv", batch=8, seqlen=2048, dim=1536, width=4,
         dtype="bf16"),
]


def conv_inputs(batch, seqlen, dim, width, dtype="bf16", seed=0, bias=True, state=False, **_):
    """Inputs of the causal depthwise conv1d: x ~ N(0,1) (batch, seqlen, dim); weight and bias
    ~ U(-1/sqrt(width), 1/sqrt(width)) (the Conv1d default range for one input channel per group);
    optional carried-in state (batch, dim, width-1) ~ N(0,1) in x's dtype."""
    rng = np.random.default_rng(seed)
    k = 1.0 / np.sqrt(width)
    out = {}
    out["x"] = round_to(rng.standard_normal((batch, seqlen, dim), dtype=np.float32), dtype)
    out["weight"] = rng.uniform(-k, k, (dim, width)).astype(np.float32)
    out["bias"] = rng.uniform(-k, k, dim).astype(np.float32) if bias else None
    out["state_in"] = (round_to(rng.standard_normal((batch, dim, width - 1), dtype=np.float32), dtype)
                       if state else None)
    out["meta"] = dict(kind="conv", dtype=dtype)
    return out


def config_inputs(index: int, **overrides):
    """Inputs of workload `index` (seed 42 + index), optionally with overridden sizes."""
    cfg = dict(CONFIGS[index])
    cfg.update(overrides)
    seed = 42 + index
    if cfg["kind"] == "scan":
        return scan_inputs(seed=seed, **cfg), cfg
    return ssd_inputs(seed=seed, **cfg), cfg


_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(inp: dict, device) -> dict:
    """Device tensors in their storage dtypes (exact: values are already rounded)."""
    meta = inp["meta"]
    act = _TORCH[meta["dtype"]]
    fp32_keys = {"A", "D", "delta_bias", "dt_bias", "h0", "state", "weight", "bias"}
    out = {}
    for k, v in inp.items():
        if k == "meta" or v is None:
            out[k] = None if k != "meta" else v
            continue
        if k in fp32_keys:
            dt = torch.float32
        elif k == "delta":
            dt = _TORCH[meta["delta_dtype"]]
        elif k == "dt":
            dt = _TORCH[meta["dt_dtype"]]
        else:
            dt = act
        out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device=device, dtype=dt)
    return out


def to_f64(inp: dict) -> dict:
    return {k: (None if v is None else (v if k == "meta" else np.asarray(v, dtype=np.float64)))
            for k, v in inp.items()}
