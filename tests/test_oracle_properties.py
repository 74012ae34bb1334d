"""Property sweeps of the fp64 oracle over small random shapes (CPU only).

Each property holds for the selective scan as a map, whatever the shapes and
values: splitting the sequence and carrying the state through h0/h_final, the
independence of the diagonal states, linearity in x for fixed (dt, B, C, z),
and the associativity of the step composition that the chunked GPU path uses
to carry state across time chunks (each token is the affine map
h -> Abar_t h + b_t; two of them compose as (Abar2 Abar1, Abar2 b1 + b2),
"SSM & Mamba", Mamba: selective SSM; "Mamba / SSM complete guide" sec. 5,
parallel scan).  Shapes are drawn up to (batch, seqlen, dim, dstate) =
(2, 64, 8, 8).
"""
import functools

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True)


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def draw_inputs(seed, b, L, D, N, softplus, gate, skip, bias, h0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, L, D))
    if softplus:
        delta = rng.standard_normal((b, L, D))
    else:
        delta = rng.uniform(0.005, 0.5, (b, L, D))
    A = -rng.uniform(0.1, 5.0, (D, N))
    B = rng.standard_normal((b, L, N))
    C = rng.standard_normal((b, L, N))
    kw = dict(Dskip=rng.standard_normal(D) if skip else None, z=rng.standard_normal((b, L, D)) if gate else None,
              delta_bias=rng.uniform(-3, 0, D) if bias else None, delta_softplus=softplus,
              h0=rng.standard_normal((b, D, N)) if h0 else None)
    return x, delta, A, B, C, kw


shapes = st.tuples(st.integers(1, 2), st.integers(2, 64), st.integers(1, 8), st.integers(1, 8))
flags = st.tuples(st.booleans(), st.booleans(), st.booleans(), st.booleans(), st.booleans())


@SETTINGS
@given(shape=shapes, fl=flags, seed=st.integers(0, 2**31 - 1), frac=st.floats(0.0, 1.0))
def test_split_carry_any_point(oracle_mod, shape, fl, seed, frac):
    b, L, D, N = shape
    x, delta, A, B, C, kw = draw_inputs(seed, b, L, D, N, *fl)
    y, hf = oracle_mod.selective_scan(x, delta, A, B, C, **kw)
    m = min(L - 1, max(1, int(frac * L)))
    cut = lambda a, s: None if a is None else a[:, s]
    kw1 = dict(kw, z=cut(kw["z"], slice(0, m)))
    y1, h1 = oracle_mod.selective_scan(x[:, :m], delta[:, :m], A, B[:, :m], C[:, :m], **kw1)
    kw2 = dict(kw, z=cut(kw["z"], slice(m, L)), h0=h1)
    y2, h2 = oracle_mod.selective_scan(x[:, m:], delta[:, m:], A, B[:, m:], C[:, m:], **kw2)
    assert rel(np.concatenate([y1, y2], 1), y) < 1e-12
    assert rel(h2, hf) < 1e-12


@SETTINGS
@given(shape=shapes, fl=flags, seed=st.integers(0, 2**31 - 1))
def test_states_are_independent(oracle_mod, shape, fl, seed):
    b, L, D, N = shape
    x, delta, A, B, C, kw = draw_inputs(seed, b, L, D, N, *fl)
    y, hf = oracle_mod.selective_scan(x, delta, A, B, C, **kw)
    # the readout before skip and gate is a sum over states of independent one-state scans
    kw0 = dict(kw, Dskip=None, z=None)
    acc = np.zeros_like(y)
    for n in range(N):
        h0n = None if kw["h0"] is None else kw["h0"][..., n:n + 1]
        yn, hn = oracle_mod.selective_scan(x, delta, A[:, n:n + 1], B[..., n:n + 1], C[..., n:n + 1],
                                           **dict(kw0, h0=h0n))
        acc += yn
        assert rel(hn[..., 0], hf[..., n]) < 1e-13 or np.max(np.abs(hf[..., n])) < 1e-300
    pre = acc + (0.0 if kw["Dskip"] is None else kw["Dskip"] * x)
    gate = 1.0 if kw["z"] is None else kw["z"] / (1.0 + np.exp(-kw["z"]))
    assert rel(pre * gate, y) < 1e-12


@SETTINGS
@given(shape=shapes, fl=flags, seed=st.integers(0, 2**31 - 1), c1=st.floats(-3, 3), c2=st.floats(-3, 3))
def test_linear_in_x(oracle_mod, shape, fl, seed, c1, c2):
    b, L, D, N = shape
    x, delta, A, B, C, kw = draw_inputs(seed, b, L, D, N, *fl)
    kw["h0"] = None
    x2 = np.random.default_rng(seed + 1).standard_normal(x.shape)
    y1, h1 = oracle_mod.selective_scan(x, delta, A, B, C, **kw)
    y2, h2 = oracle_mod.selective_scan(x2, delta, A, B, C, **kw)
    y3, h3 = oracle_mod.selective_scan(c1 * x + c2 * x2, delta, A, B, C, **kw)
    scale = max(np.max(np.abs(y1)), np.max(np.abs(y2)), 1e-300)
    assert np.max(np.abs(y3 - (c1 * y1 + c2 * y2))) <= 1e-12 * scale * (abs(c1) + abs(c2) + 1)
    hs = max(np.max(np.abs(h1)), np.max(np.abs(h2)), 1e-300)
    assert np.max(np.abs(h3 - (c1 * h1 + c2 * h2))) <= 1e-12 * hs * (abs(c1) + abs(c2) + 1)


def all_trees(lo, hi):
    """Every full binary bracketing of the items lo .. hi-1 (Catalan many)."""
    if hi - lo == 1:
        return [lo]
    out = []
    for m in range(lo + 1, hi):
        for left in all_trees(lo, m):
            for right in all_trees(m, hi):
                out.append((left, right))
    return out


def compose(tree, elems):
    """Evaluate a bracketing with (A2, b2) o (A1, b1) = (A2 A1, A2 b1 + b2), earlier items on the left."""
    if isinstance(tree, int):
        return elems[tree]
    a1, b1 = compose(tree[0], elems)
    a2, b2 = compose(tree[1], elems)
    return a2 * a1, a2 * b1 + b2


@settings(max_examples=25, deadline=None, derandomize=True)
@given(L=st.integers(1, 7), seed=st.integers(0, 2**31 - 1))
def test_every_bracketing_of_the_step_composition(oracle_mod, L, seed):
    # one (batch, channel, state) slice: token t is the affine map h -> E_t h + g_t B_t x_t with
    # E_t = exp(dt_t a) and the ZOH gain g_t = expm1(dt_t a) / a; every bracketing of their composition,
    # applied to h0, must give the oracle's final state
    rng = np.random.default_rng(seed)
    a = -rng.uniform(0.1, 5.0)
    dt = rng.uniform(0.005, 0.8, L)
    x = rng.standard_normal(L); Bv = rng.standard_normal(L); h0 = rng.standard_normal()
    _, hf = oracle_mod.selective_scan(x[None, :, None], dt[None, :, None], np.array([[a]]), Bv[None, :, None],
                                      np.ones((1, L, 1)), h0=np.array([[[h0]]]))
    elems = [(np.exp(dt[t] * a), np.expm1(dt[t] * a) / a * Bv[t] * x[t]) for t in range(L)]
    trees = all_trees(0, L)
    assert len(trees) == [1, 1, 2, 5, 14, 42, 132][L - 1]   # Catalan(L - 1)
    for tree in trees:
        At, bt = compose(tree, elems)
        assert abs(At * h0 + bt - hf[0, 0, 0]) <= 1e-13 * max(1.0, abs(hf[0, 0, 0]))


@functools.lru_cache(maxsize=None)
def _catalan(n):
    return 1 if n <= 1 else sum(_catalan(i) * _catalan(n - 1 - i) for i in range(n))


def test_bracketing_counts_are_catalan():
    for n in range(1, 8):
        assert len(all_trees(0, n)) == _catalan(n - 1)
