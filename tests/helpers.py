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


def err_report(got, ref, block=1 << 22) -> dict:
    """Three relative-error figures of `got` against `ref`, computed in blocks so that arrays of
    hundreds of millions of elements need no full-size temporaries:
      bar   max_i |d_i| / (|ref_i| + rms(ref))    (the parity metric, compared with TOL)
      inf   max_i |d_i| / max_i |ref_i|           (inf-norm relative error)
      floor max_i |d_i| / max(|ref_i|, 1e-3 rms)  (per-element relative error, 1e-3 rms floor)
    plus the element count and rms(ref).  NaN anywhere in `got` makes every figure NaN."""
    g = np.asarray(got).reshape(-1)
    r = np.asarray(ref).reshape(-1)
    if g.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (np.shape(got), np.shape(ref)))
    n = r.size
    if n == 0:
        return dict(bar=0.0, inf=0.0, floor=0.0, n=0, rms=0.0)
    ss, amax = 0.0, 0.0
    for i in range(0, n, block):
        rb = np.asarray(r[i:i + block], dtype=np.float64)
        ss += float(np.dot(rb, rb))
        amax = max(amax, float(np.max(np.abs(rb))))
    rms = (ss / n) ** 0.5
    bar = dmax = floor = 0.0
    for i in range(0, n, block):
        rb = np.asarray(r[i:i + block], dtype=np.float64)
        d = np.abs(np.asarray(g[i:i + block], dtype=np.float64) - rb)
        if np.isnan(d).any():
            return dict(bar=float("nan"), inf=float("nan"), floor=float("nan"), n=n, rms=rms)
        a = np.abs(rb)
        bar = max(bar, float(np.max(d / (a + rms + 1e-300))))
        floor = max(floor, float(np.max(d / np.maximum(a, 1e-3 * rms + 1e-300))))
        dmax = max(dmax, float(np.max(d)))
    return dict(bar=bar, inf=dmax / (amax + 1e-300), floor=floor, n=n, rms=rms)


def fmt_report(name, rep) -> str:
    return "%s: %d elements, bar %.3g, inf-norm %.3g, per-element (1e-3 rms floor) %.3g" % (
        name, rep["n"], rep["bar"], rep["inf"], rep["floor"])


def oracle_scan(inp, want_y=True, threads=None):
    f = workloads.to_f64(inp)
    return oracle.selective_scan(f["x"], f["delta"], f["A"], f["B"], f["C"], Dskip=f["D"], z=f["z"],
                                 delta_bias=f["delta_bias"], delta_softplus=inp["meta"]["softplus"], h0=f["h0"],
                                 want_y=want_y, threads=threads)


def oracle_ssd(inp, want_y=True, threads=None):
    f = workloads.to_f64(inp)
    return oracle.ssd_recurrent(f["x"], f["dt"], f["A"], f["B"], f["C"], Dskip=f["D"], z=f["z"],
                                dt_bias=f["dt_bias"], dt_softplus=inp["meta"]["softplus"], h0=f["h0"],
                                want_y=want_y, threads=threads)
