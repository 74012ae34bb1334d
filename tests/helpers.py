"""Shared test helpers: the parity metric and oracle calls on workload dicts."""
import numpy as np

import oracle
import workloads

# Parity bars: max relative error 1e-4 for fp32 activations, 2e-2 for bf16
# inputs (fp32 state).  Relative error of element i is |y_i - ref_i| / (|ref_i| + rms(ref)),
# so elements near zero are judged against the output's own scale.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + scale + 1e-300)))


def oracle_scan(inp, want_y=True, threads=None):
    f = workloads.to_f64(inp)
    return oracle.selective_scan(f["x"], f["delta"], f["A"], f["B"], f["C"], Dskip=f["D"], z=f["z"],
                                 delta_bias=f["delta_bias"], delta_softplus=inp["meta"]["softplus"], h0=f["h0"],
                                 want_y=want_y, threads=threads)


def oracle_scan_slices(inp, slices, threads=None):
    """Oracle outputs for a list of (b, d) slices: y (len, L) and h_final (len, N)."""
    f = workloads.to_f64(inp)
    ys, hs = [], []
    for b, d in slices:
        sl = lambda a: None if a is None else a[b:b + 1, :, d:d + 1]
        y, h = oracle.selective_scan(sl(f["x"]), sl(f["delta"]), f["A"][d:d + 1], f["B"][b:b + 1], f["C"][b:b + 1],
                                     Dskip=None if f["D"] is None else f["D"][d:d + 1], z=sl(f["z"]),
                                     delta_bias=None if f["delta_bias"] is None else f["delta_bias"][d:d + 1],
                                     delta_softplus=inp["meta"]["softplus"],
                                     h0=None if f["h0"] is None else f["h0"][b:b + 1, d:d + 1], threads=1)
        ys.append(y[0, :, 0])
        hs.append(h[0, 0])
    return np.stack(ys), np.stack(hs)


def oracle_ssd(inp, want_y=True, threads=None):
    f = workloads.to_f64(inp)
    return oracle.ssd_recurrent(f["x"], f["dt"], f["A"], f["B"], f["C"], Dskip=f["D"], z=f["z"],
                                dt_bias=f["dt_bias"], dt_softplus=inp["meta"]["softplus"], h0=f["h0"],
                                want_y=want_y, threads=threads)
