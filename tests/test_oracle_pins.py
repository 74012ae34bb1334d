"""Pins for the fp64 oracle, each against something other than the oracle itself.

What pins what (sources cited by page title and section):
  * N=1 closed form: a constant input held between samples gives the sampled
    continuous step response (ZOH assumption, "SSM & Mamba", Discretization/ZOH).
  * Convolution view: a time-invariant SSM equals the causal convolution with
    K_i = C Abar^i Bbar ("Mamba / SSM complete guide" sec. 2 and "SSM & Mamba",
    Equivalence with convolution); includes the page's own experiment parameters.
  * First output y_0 = C Bbar x_0 (complete guide sec. 2, expansion of y[0]).
  * Limits: a -> 0 gives a prefix sum; large dt forgets the past, small dt keeps
    it ("SSM & Mamba", intuition for dt).
  * Invariants: separability over the diagonal state, linearity in x,
    split/carry through h0/h_final, softplus/bias placement against numpy.
  * SSD: recurrent form == quadratic (matrix) form ("Mamba-2 / SSD", linear and
    quadratic forms), and SSD == selective scan with A and dt broadcast over a head.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_n1_closed_form_step_response(oracle_mod):
    # constant dt, a, B, C, x: h_t = -(B x / a) (1 - e^{a dt (t+1)})
    L = 300
    for a, dt, Bv, Cv, xv, Ds in [(-0.7, 0.05, 1.3, -0.4, 2.0, 0.3), (-3.0, 0.2, -0.5, 1.1, -1.5, 0.0),
                                  (-0.01, 1.0, 2.0, 0.5, 0.25, -1.0)]:
        x = np.full((1, L, 1), xv)
        y, hf = oracle_mod.selective_scan(x, np.full((1, L, 1), dt), np.array([[a]]), np.full((1, L, 1), Bv),
                                          np.full((1, L, 1), Cv), Dskip=np.array([Ds]))
        t = np.arange(L)
        h = -(Bv * xv / a) * (1.0 - np.exp(a * dt * (t + 1)))
        assert rel(y[0, :, 0], Cv * h + Ds * xv) < 1e-13
        assert abs(hf[0, 0, 0] - h[-1]) <= 1e-13 * abs(h[-1])


def test_page_mode_equivalence_experiment(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "p3_mode_equivalence.json")))
    n, L, dt = g["n"], g["seq_len"], g["delta"]
    rs = np.random.RandomState(42)
    A = -np.arange(1, n + 1, dtype=np.float64)
    B = np.ones(n) * g["B"]
    C = rs.randn(n) * 0.1
    t = np.linspace(0, 1, L)
    x = np.sin(2 * np.pi * 3 * t) + 0.5 * np.sin(2 * np.pi * 15 * t) + 0.2 * rs.randn(L)
    y_rec, _ = oracle_mod.selective_scan(x[None, :, None], np.full((1, L, 1), dt), A[None, :],
                                         np.broadcast_to(B, (1, L, n)), np.broadcast_to(C, (1, L, n)))
    y_conv = oracle_mod.lti_conv(x, A, B, C, dt)
    assert np.max(np.abs(y_rec[0, :, 0] - y_conv)) < g["max_abs_diff_bound"]


@pytest.mark.parametrize("n", [1, 3, 8, 16])
def test_lti_convolution_random(oracle_mod, n):
    rng = np.random.default_rng(100 + n)
    L, D = 400, 3
    for d in range(D):
        A = -rng.uniform(0.1, 5.0, n)
        B = rng.standard_normal(n)
        C = rng.standard_normal(n)
        dt = float(rng.uniform(0.01, 0.3))
        x = rng.standard_normal(L)
        Ds = float(rng.standard_normal())
        y, _ = oracle_mod.selective_scan(x[None, :, None], np.full((1, L, 1), dt), A[None, :],
                                         np.broadcast_to(B, (1, L, n)), np.broadcast_to(C, (1, L, n)),
                                         Dskip=np.array([Ds]))
        yc = oracle_mod.lti_conv(x, A, B, C, dt, Ds)
        assert rel(y[0, :, 0], yc) < 1e-12


def test_first_output(oracle_mod):
    rng = np.random.default_rng(7)
    b, L, D, N = 2, 5, 4, 6
    x = rng.standard_normal((b, L, D)); dt = rng.uniform(0.01, 0.5, (b, L, D))
    A = -rng.uniform(0.5, 4, (D, N)); B = rng.standard_normal((b, L, N)); C = rng.standard_normal((b, L, N))
    Ds = rng.standard_normal(D)
    y, _ = oracle_mod.selective_scan(x, dt, A, B, C, Dskip=Ds)
    g0 = np.expm1(dt[:, 0, :, None] * A[None]) / A[None]            # (b, D, N)
    y0 = np.einsum("bn,bdn->bd", C[:, 0], g0 * B[:, 0, None, :] * x[:, 0, :, None]) + Ds * x[:, 0]
    assert rel(y[:, 0], y0) < 1e-14


def test_a_zero_is_prefix_sum(oracle_mod):
    rng = np.random.default_rng(8)
    b, L, D, N = 2, 50, 3, 4
    x = rng.standard_normal((b, L, D)); dt = rng.uniform(0.01, 0.5, (b, L, D))
    B = rng.standard_normal((b, L, N)); C = rng.standard_normal((b, L, N))
    y, _ = oracle_mod.selective_scan(x, dt, np.zeros((D, N)), B, C)
    # h_t[n] = sum_{j<=t} dt_j B_j[n] x_j ; y_t = C_t . h_t   (B and C in distinct roles)
    h = np.cumsum(dt[..., None] * B[:, :, None, :] * x[..., None], axis=1)    # (b, L, D, N)
    assert rel(y, np.einsum("bln,bldn->bld", C, h)) < 1e-13
    # a tiny non-zero decay is within ~|a| * sum(dt) of the prefix sum
    y2, _ = oracle_mod.selective_scan(x, dt, np.full((D, N), -1e-9), B, C)
    assert rel(y2, y) < 1e-7


def test_large_dt_forgets_small_dt_keeps(oracle_mod):
    rng = np.random.default_rng(9)
    b, L, D, N = 1, 40, 3, 5
    x = rng.standard_normal((b, L, D)); z = rng.standard_normal((b, L, D))
    A = -rng.uniform(0.5, 4, (D, N)); B = rng.standard_normal((b, L, N)); C = rng.standard_normal((b, L, N))
    Ds = rng.standard_normal(D)
    # dt -> infinity: Abar = 0, Bbar -> -B/a : memoryless; skip added before the gate
    y, _ = oracle_mod.selective_scan(x, np.full((b, L, D), 1e3), A, B, C, Dskip=Ds, z=z)
    mem = np.einsum("bln,dn->bld", C * B, -1.0 / A) * x + Ds * x
    assert rel(y, mem * z * expit(z)) < 1e-13
    # dt -> 0: y/dt -> sum_{j<=t} (C_t . B_j) x_j  (first order in dt)
    eps = 1e-9
    y0, _ = oracle_mod.selective_scan(x, np.full((b, L, D), eps), A, B, C)
    cb = np.einsum("btn,bjn->btj", C, B)
    ref = np.einsum("btj,bjd->btd", np.tril(cb), x)
    assert rel(y0 / eps, ref) < 1e-6


def test_separable_linear_and_split(oracle_mod):
    rng = np.random.default_rng(10)
    b, L, D, N = 2, 64, 3, 5
    x = rng.standard_normal((b, L, D)); x2 = rng.standard_normal((b, L, D)); dt = rng.uniform(0.01, 0.4, (b, L, D))
    A = -rng.uniform(0.2, 4, (D, N)); B = rng.standard_normal((b, L, N)); C = rng.standard_normal((b, L, N))
    Ds = rng.standard_normal(D)
    h0 = rng.standard_normal((b, D, N))
    y, hf = oracle_mod.selective_scan(x, dt, A, B, C, Dskip=Ds, h0=h0)
    # separability over the diagonal state
    acc = np.zeros_like(y); hacc = np.zeros_like(hf)
    for n in range(N):
        yn, hn = oracle_mod.selective_scan(x, dt, A[:, n:n + 1], B[..., n:n + 1], C[..., n:n + 1], h0=h0[..., n:n + 1])
        acc += yn; hacc[..., n] = hn[..., 0]
    assert rel(y, acc + Ds * x) < 1e-13 and rel(hf, hacc) < 1e-14
    # linearity in x (h0 = 0)
    ya, _ = oracle_mod.selective_scan(x, dt, A, B, C, Dskip=Ds)
    yb, _ = oracle_mod.selective_scan(x2, dt, A, B, C, Dskip=Ds)
    yab, _ = oracle_mod.selective_scan(1.5 * x - 0.5 * x2, dt, A, B, C, Dskip=Ds)
    assert rel(yab, 1.5 * ya - 0.5 * yb) < 1e-13
    # split/carry: run(0:L) == run(0:m) then run(m:L) from its final state
    for m in (1, 17, 63):
        y1, h1 = oracle_mod.selective_scan(x[:, :m], dt[:, :m], A, B[:, :m], C[:, :m], Dskip=Ds, h0=h0)
        y2, h2 = oracle_mod.selective_scan(x[:, m:], dt[:, m:], A, B[:, m:], C[:, m:], Dskip=Ds, h0=h1)
        assert rel(np.concatenate([y1, y2], 1), y) < 1e-13 and rel(h2, hf) < 1e-13


def test_softplus_bias_gate(oracle_mod):
    rng = np.random.default_rng(11)
    b, L, D, N = 2, 30, 4, 3
    x = rng.standard_normal((b, L, D)); u = 3 * rng.standard_normal((b, L, D)); z = 4 * rng.standard_normal((b, L, D))
    u[0, 0, 0] = 60.0; u[0, 1, 0] = -60.0                    # far tails of softplus
    bias = rng.standard_normal(D)
    A = -rng.uniform(0.2, 4, (D, N)); B = rng.standard_normal((b, L, N)); C = rng.standard_normal((b, L, N))
    y, hf = oracle_mod.selective_scan(x, u, A, B, C, z=z, delta_bias=bias, delta_softplus=True)
    dt = np.logaddexp(0.0, u + bias)                          # numpy's softplus
    y_ref, hf_ref = oracle_mod.selective_scan(x, dt, A, B, C)
    assert rel(y, y_ref * z * expit(z)) < 1e-13 and rel(hf, hf_ref) < 1e-14
    # without softplus the bias is simply added to dt
    y2, _ = oracle_mod.selective_scan(x, np.abs(u), A, B, C, delta_bias=np.abs(bias))
    y2r, _ = oracle_mod.selective_scan(x, np.abs(u) + np.abs(bias), A, B, C)
    assert rel(y2, y2r) < 1e-14


def _ssd_inputs(rng, b, L, H, P, G, N):
    return dict(x=rng.standard_normal((b, L, H, P)), dt=rng.uniform(-2, 1, (b, L, H)),
                A=-rng.uniform(0.5, 6, H), B=rng.standard_normal((b, L, G, N)), C=rng.standard_normal((b, L, G, N)),
                Dskip=rng.standard_normal(H), z=rng.standard_normal((b, L, H, P)), dt_bias=rng.standard_normal(H),
                h0=rng.standard_normal((b, H, P, N)))


@pytest.mark.parametrize("G", [1, 2])
def test_ssd_recurrent_equals_quadratic(oracle_mod, G):
    rng = np.random.default_rng(20 + G)
    inp = _ssd_inputs(rng, 2, 37, 4, 3, G, 5)
    y_rec, _ = oracle_mod.ssd_recurrent(dt_softplus=True, **inp)
    y_quad = oracle_mod.ssd_quadratic(dt_softplus=True, **inp)
    assert rel(y_rec, y_quad) < 1e-12


@pytest.mark.parametrize("G", [1, 2])
def test_ssd_equals_selective_scan_broadcast(oracle_mod, G):
    rng = np.random.default_rng(30 + G)
    b, L, H, P, N = 2, 25, 4, 3, 6
    inp = _ssd_inputs(rng, b, L, H, P, G, N)
    y, hf = oracle_mod.ssd_recurrent(dt_softplus=True, **inp)
    hpg = H // G
    for h in range(H):
        g = h // hpg
        ys, hs = oracle_mod.selective_scan(
            inp["x"][:, :, h, :], np.repeat(inp["dt"][:, :, h:h + 1], P, axis=2),
            np.full((P, N), inp["A"][h]), inp["B"][:, :, g], inp["C"][:, :, g],
            Dskip=np.full(P, inp["Dskip"][h]), z=inp["z"][:, :, h, :],
            delta_bias=np.full(P, inp["dt_bias"][h]), delta_softplus=True, h0=inp["h0"][:, h])
        assert rel(y[:, :, h, :], ys) < 1e-13 and rel(hf[:, h], hs) < 1e-14


def test_empty_and_single_step(oracle_mod):
    rng = np.random.default_rng(40)
    D, N = 3, 4
    A = -rng.uniform(0.5, 2, (D, N))
    y, hf = oracle_mod.selective_scan(np.zeros((1, 0, D)), np.zeros((1, 0, D)), A, np.zeros((1, 0, N)),
                                      np.zeros((1, 0, N)), h0=np.ones((1, D, N)))
    assert y.shape == (1, 0, D) and np.all(hf == 1.0)     # no tokens: the state passes through
    # one token from a state h0: h = e^{dt a} h0 + g B x  (single-step decode)
    x = rng.standard_normal((1, 1, D)); dt = rng.uniform(0.1, 1, (1, 1, D))
    B = rng.standard_normal((1, 1, N)); C = rng.standard_normal((1, 1, N)); h0 = rng.standard_normal((1, D, N))
    y, hf = oracle_mod.selective_scan(x, dt, A, B, C, h0=h0)
    h = np.exp(dt[0, 0, :, None] * A) * h0[0] + np.expm1(dt[0, 0, :, None] * A) / A * B[0, 0] * x[0, 0, :, None]
    assert rel(hf[0], h) < 1e-14 and rel(y[0, 0], h @ C[0, 0]) < 1e-14


def test_state_update_step_closed_form_and_composition(oracle_mod):
    # one decode step written out: dt = softplus(u + bias); h = e^{dt a} h0 + expm1(dt a)/a B x;
    # y = (C.h + D x) silu(z)
    rng = np.random.default_rng(50)
    b, D, N, T = 3, 5, 6, 9
    A = -rng.uniform(0.3, 5, (D, N)); bias = rng.standard_normal(D); Ds = rng.standard_normal(D)
    x = rng.standard_normal((b, T, D)); u = rng.standard_normal((b, T, D)); z = rng.standard_normal((b, T, D))
    B = rng.standard_normal((b, T, N)); C = rng.standard_normal((b, T, N)); h0 = rng.standard_normal((b, D, N))
    y1, h1 = oracle_mod.state_update(x[:, 0], u[:, 0], A, B[:, 0], C[:, 0], h0, Dskip=Ds, z=z[:, 0],
                                     delta_bias=bias, delta_softplus=True)
    dt = np.logaddexp(0.0, u[:, 0] + bias)[:, :, None]
    h = np.exp(dt * A) * h0 + np.expm1(dt * A) / A * B[:, 0, None, :] * x[:, 0, :, None]
    yr = (np.einsum("bdn,bn->bd", h, C[:, 0]) + Ds * x[:, 0]) * z[:, 0] * expit(z[:, 0])
    assert rel(h1, h) < 1e-14 and rel(y1, yr) < 1e-13
    # T steps, each from the previous state, equal the scan over the T tokens
    y_seq, h_seq = oracle_mod.selective_scan(x, u, A, B, C, Dskip=Ds, z=z, delta_bias=bias, delta_softplus=True,
                                             h0=h0)
    st = h0
    for t in range(T):
        yt, st = oracle_mod.state_update(x[:, t], u[:, t], A, B[:, t], C[:, t], st, Dskip=Ds, z=z[:, t],
                                         delta_bias=bias, delta_softplus=True)
        assert rel(yt, y_seq[:, t]) < 1e-13
    assert rel(st, h_seq) < 1e-14


@pytest.mark.parametrize("G", [1, 2])
def test_ssd_state_update_steps_equal_quadratic_form(oracle_mod, G):
    # successive Mamba-2 decode steps reproduce the matrix (quadratic) form over the same tokens
    rng = np.random.default_rng(60 + G)
    inp = _ssd_inputs(rng, 2, 11, 4, 3, G, 5)
    y_quad = oracle_mod.ssd_quadratic(dt_softplus=True, **inp)
    st = inp["h0"]
    for t in range(11):
        yt, st = oracle_mod.ssd_state_update(inp["x"][:, t], inp["dt"][:, t], inp["A"], inp["B"][:, t],
                                             inp["C"][:, t], st, Dskip=inp["Dskip"], z=inp["z"][:, t],
                                             dt_bias=inp["dt_bias"], dt_softplus=True)
        assert rel(yt, y_quad[:, t]) < 1e-12


def test_causal_conv1d_against_numpy_and_torch(oracle_mod):
    # the block's depthwise causal conv: numpy's full convolution with the reversed taps, first L
    # outputs; and torch's Conv1d formulation (padding W-1, one group per channel, trimmed to L)
    import torch
    rng = np.random.default_rng(70)
    b, L, D, W = 2, 23, 5, 4
    x = rng.standard_normal((b, L, D)); w = rng.standard_normal((D, W)); bias = rng.standard_normal(D)
    out = oracle_mod.causal_conv1d(x, w, bias, silu=False)
    for bi in range(b):
        for d in range(D):
            ref = np.convolve(x[bi, :, d], w[d, ::-1])[:L] + bias[d]
            assert rel(out[bi, :, d], ref) < 1e-14
    conv = torch.nn.functional.conv1d(torch.from_numpy(x).transpose(1, 2), torch.from_numpy(w)[:, None, :],
                                      torch.from_numpy(bias), padding=W - 1, groups=D)[:, :, :L]
    ref = torch.nn.functional.silu(conv).transpose(1, 2).numpy()
    assert rel(oracle_mod.causal_conv1d(x, w, bias, silu=True), ref) < 1e-14


def test_causal_conv1d_impulse_and_state_handoff(oracle_mod):
    rng = np.random.default_rng(71)
    D, W, L = 3, 4, 17
    w = rng.standard_normal((D, W))
    x = np.zeros((1, L, D)); x[0, 0, :] = 1.0
    out = oracle_mod.causal_conv1d(x, w, silu=False)
    for t in range(L):                       # impulse response: the taps, newest first
        assert np.allclose(out[0, t], w[:, W - 1 - t] if t < W else 0.0, rtol=0, atol=1e-15)
    # a sequence split anywhere, the second part carrying the first part's state, equals the whole
    b = 2
    x = rng.standard_normal((b, L, D)); bias = rng.standard_normal(D); s0 = rng.standard_normal((b, D, W - 1))
    full, st_full = oracle_mod.causal_conv1d(x, w, bias, state_in=s0, want_state=True)
    for m in (0, 1, 2, 3, 9):
        o1, st1 = oracle_mod.causal_conv1d(x[:, :m], w, bias, state_in=s0, want_state=True)
        o2, st2 = oracle_mod.causal_conv1d(x[:, m:], w, bias, state_in=st1, want_state=True)
        assert rel(np.concatenate([o1, o2], 1), full) < 1e-14 and np.array_equal(st2, st_full)
    # the carried state is the last W-1 inputs, oldest first
    assert np.array_equal(st_full, np.transpose(x[:, L - (W - 1):, :], (0, 2, 1)))


def _scan_loss(oracle_mod, p, dout, dh_final, softplus, euler=False, reverse=False):
    y, hf = oracle_mod.selective_scan(p["x"], p["delta"], p["A"], p["B"], p["C"], Dskip=p.get("Dskip"), z=p.get("z"),
                                      delta_bias=p.get("delta_bias"), delta_softplus=softplus, h0=p.get("h0"),
                                      euler=euler, reverse=reverse)
    return float(np.sum(dout * y) + np.sum(dh_final * hf))


@pytest.mark.parametrize("softplus,full,euler,reverse,per_token",
                         [(True, True, False, False, False), (False, True, False, False, False),
                          (False, False, False, False, False), (True, True, True, False, False),
                          (False, True, False, True, False), (True, True, True, True, False),
                          (True, True, False, False, True), (False, False, True, True, True)])
def test_scan_backward_against_finite_differences(oracle_mod, softplus, full, euler, reverse, per_token):
    # every gradient of O5 (O5e for Euler, the flipped form for reverse, the channel-summed ddelta for one
    # step size per token) against central differences of the matching forward (O1 / O1e, pinned above)
    rng = np.random.default_rng(80 + 2 * softplus + full + 4 * euler + 8 * reverse + 16 * per_token)
    b, L, D, N = 2, 6, 3, 4
    dshape = (b, L) if per_token else (b, L, D)
    p = dict(x=rng.standard_normal((b, L, D)),
             delta=(rng.standard_normal(dshape) if softplus else rng.uniform(0.05, 0.8, dshape)),
             A=-rng.uniform(0.2, 3.0, (D, N)), B=rng.standard_normal((b, L, N)), C=rng.standard_normal((b, L, N)))
    p["A"][0, 0] = 0.0                       # the a = 0 limit of the gain and its derivative
    p["A"][1, 1] = -1e-7                     # |dt a| far below the series threshold
    if full:
        p.update(Dskip=rng.standard_normal(D), z=rng.standard_normal((b, L, D)), delta_bias=rng.standard_normal(D) * 0.3,
                 h0=rng.standard_normal((b, D, N)))
    dout = rng.standard_normal((b, L, D))
    dh_final = rng.standard_normal((b, D, N))
    g = oracle_mod.selective_scan_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], dout, Dskip=p.get("Dskip"),
                                      z=p.get("z"), delta_bias=p.get("delta_bias"), delta_softplus=softplus,
                                      h0=p.get("h0"), dh_final=dh_final, threads=1, euler=euler, reverse=reverse)
    names = dict(x="dx", delta="ddelta", A="dA", B="dB", C="dC", Dskip="dDskip", z="dz", delta_bias="ddelta_bias",
                 h0="dh0")
    for k, gk in names.items():
        if k not in p:
            continue
        num = np.zeros_like(p[k])
        for idx in np.ndindex(p[k].shape):
            v0 = p[k][idx]
            eps = 1e-6 * max(1.0, abs(v0))
            p[k][idx] = v0 + eps
            lp = _scan_loss(oracle_mod, p, dout, dh_final, softplus, euler, reverse)
            p[k][idx] = v0 - eps
            lm = _scan_loss(oracle_mod, p, dout, dh_final, softplus, euler, reverse)
            p[k][idx] = v0
            num[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(g[gk] - num)) / max(np.max(np.abs(num)), 1e-12)
        assert err < 2e-7, (k, err)


def test_euler_closed_form(oracle_mod):
    # constant dt, a, B, C, x with Bbar = dt B: h_t = dt B x (1 - e^{a dt (t+1)}) / (1 - e^{a dt})
    L = 200
    for a, dt, Bv, Cv, xv in [(-0.7, 0.05, 1.3, -0.4, 2.0), (-3.0, 0.2, -0.5, 1.1, -1.5)]:
        y, hf = oracle_mod.selective_scan(np.full((1, L, 1), xv), np.full((1, L, 1), dt), np.array([[a]]),
                                          np.full((1, L, 1), Bv), np.full((1, L, 1), Cv), euler=True)
        E = np.exp(a * dt)
        h = dt * Bv * xv * (1.0 - E ** (np.arange(L) + 1)) / (1.0 - E)
        assert rel(y[0, :, 0], Cv * h) < 1e-13 and abs(hf[0, 0, 0] - h[-1]) <= 1e-13 * abs(h[-1])
    # a = 0: Euler and ZOH coincide (both gains are dt)
    rng = np.random.default_rng(90)
    x = rng.standard_normal((1, 20, 2)); dt = rng.uniform(0.1, 0.5, (1, 20, 2))
    B = rng.standard_normal((1, 20, 3)); C = rng.standard_normal((1, 20, 3))
    A = np.zeros((2, 3))
    assert rel(oracle_mod.selective_scan(x, dt, A, B, C, euler=True)[0], oracle_mod.selective_scan(x, dt, A, B, C)[0]) < 1e-15


def test_reverse_scan_is_anticausal_convolution(oracle_mod):
    # time-invariant parameters: the reverse scan is y_t = sum_{j >= t} K_{j-t} x_j with the same kernel
    rng = np.random.default_rng(91)
    L, N = 40, 5
    A = -rng.uniform(0.2, 2.0, N); B = rng.standard_normal(N); C = rng.standard_normal(N); dt = 0.07
    x = rng.standard_normal(L)
    y, _ = oracle_mod.selective_scan(x[None, :, None], np.full((1, L, 1), dt), A[None, :],
                                     np.broadcast_to(B, (1, L, N)), np.broadcast_to(C, (1, L, N)), reverse=True)
    K = oracle_mod.lti_conv(np.eye(L)[0], A, B, C, dt)     # impulse response = the kernel K_0 .. K_{L-1}
    ref = np.array([sum(K[j - t] * x[j] for j in range(t, L)) for t in range(L)])
    assert rel(y[0, :, 0], ref) < 1e-13
