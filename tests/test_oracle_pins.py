"""Pins for the oracle: printed page values, closed forms, brute force, limits.

Every test here runs on the CPU.  None of them compares the oracle with a
retyped copy of its own formula: each expected value is either printed in a
page (tests/golden/page_examples.json, cited there), a closed form derived from
the mathematics, a library routine, or a structurally different evaluation
(unrolled sum, semiseparable matrix, convolution, reordered combine scans).
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import forms


def _scan1(x, delta, A, B, C, bbar, h0=None, last=False):
    """One chain (batch = 1, D = 1) through the oracle; A, B, C broadcast over t."""
    x = np.asarray(x, dtype=np.float64)
    L = len(x)
    A = np.atleast_1d(np.asarray(A, dtype=np.float64))
    N = A.shape[0]
    delta = np.broadcast_to(np.asarray(delta, dtype=np.float64), (L,))
    B = np.broadcast_to(np.asarray(B, dtype=np.float64), (L, N))
    C = np.broadcast_to(np.asarray(C, dtype=np.float64), (L, N))
    res = oracle.selective_scan(
        x.reshape(1, L, 1), delta.reshape(1, L, 1), A.reshape(1, N),
        B.reshape(1, L, N), C.reshape(1, L, N), bbar=bbar,
        h0=None if h0 is None else np.asarray(h0, dtype=np.float64).reshape(1, 1, N),
        return_last_state=last)
    if last:
        return res[0][0, :, 0], res[1][0, 0]
    return res[0, :, 0]


def _states(x, delta, A, B, C, bbar):
    """h after every step, read back from the oracle's final-state output."""
    return np.array([_scan1(x[:t + 1], np.broadcast_to(delta, (len(x),))[:t + 1], A,
                            np.broadcast_to(B, (len(x), len(np.atleast_1d(A))))[:t + 1],
                            np.broadcast_to(C, (len(x), len(np.atleast_1d(A))))[:t + 1],
                            bbar, last=True)[1] for t in range(len(x))])


def _discretized_by_oracle(delta, A, B, bbar):
    """(Abar, Bbar) as the oracle applies them: one step from h = 1 with x = 0
    reads Abar; one step from h = 0 with x = 1 reads Bbar (C = 1)."""
    N = len(A)
    ones = np.ones(N)
    _, abar = _scan1([0.0], delta, A, B, ones, bbar, h0=ones, last=True)
    _, bbar_v = _scan1([1.0], delta, A, B, ones, bbar, h0=np.zeros(N), last=True)
    return abar, bbar_v


# --- printed worked examples ------------------------------------------------------------

def test_lti_zoh_four_tokens(golden):
    g = golden["lti_zoh_four_tokens"]
    p, dec = g["printed"], g["decimals"]
    abar, bbar = _discretized_by_oracle(g["Delta"], g["A"], g["B"], "zoh")
    np.testing.assert_array_equal(np.round(abar, dec), p["Abar"])
    np.testing.assert_array_equal(np.round(bbar, dec), p["Bbar"])
    y = _scan1(g["x"], g["Delta"], g["A"], g["B"], g["C"], "zoh")
    np.testing.assert_array_equal(np.round(y, dec) + 0.0, np.array(p["y"]) + 0.0)
    h = _states(g["x"], g["Delta"], g["A"], g["B"], g["C"], "zoh")
    np.testing.assert_array_equal(np.round(h, dec), p["h"])
    # forms.discretize agrees with the printed values as well
    fa, fb = forms.discretize(g["Delta"], g["A"], g["B"], "zoh")
    np.testing.assert_array_equal(np.round(fa, dec), p["Abar"])
    np.testing.assert_array_equal(np.round(fb, dec), p["Bbar"])


def test_lti_convolution_taps(golden):
    g0 = golden["lti_zoh_four_tokens"]
    g = golden["lti_convolution_taps"]
    abar, bbar = _discretized_by_oracle(g0["Delta"], g0["A"], g0["B"], "zoh")
    K = forms.convolution_kernel(abar, bbar, g0["C"], 4)
    np.testing.assert_array_equal(np.round(K, 3), g["printed"]["K"])
    y_conv = forms.convolution_output(g0["x"], K)
    np.testing.assert_array_equal(np.round(y_conv, 3) + 0.0, np.array(g["printed"]["y"]) + 0.0)
    y_rec = _scan1(g0["x"], g0["Delta"], g0["A"], g0["B"], g0["C"], "zoh")
    np.testing.assert_allclose(y_rec, y_conv, rtol=0, atol=1e-15)


def _selective_example_via_fused(g, bbar):
    """The one-channel selective example as the fused path: D = 1, R = 1, the
    x_proj row is [w_delta | w_B | w_C], dt_proj is the 1x1 identity, bias b_delta."""
    x = np.asarray(g["x"], dtype=np.float64).reshape(1, -1, 1)
    W_x = np.array([[g["w_delta"], *g["w_B"], *g["w_C"]]])
    W_dt = np.array([[1.0]])
    bias = np.array([g["b_delta"]])
    A = np.array([g["A"]])
    delta, B, C = oracle.selection.fused_projections(x, W_x, W_dt, bias, R=1, N=2)
    y = oracle.selective_ssm_fused(x, W_x, W_dt, bias, A, R=1, bbar=bbar)
    return x, delta, A, B, C, y


def test_selective_zoh_four_tokens(golden):
    g = golden["selective_zoh_four_tokens"]
    p, dec = g["printed"], g["decimals"]
    x, delta, A, B, C, y = _selective_example_via_fused(g, "zoh")
    np.testing.assert_array_equal(np.round(delta[0, :, 0], dec), p["Delta"])
    np.testing.assert_array_equal(np.round(y[0, :, 0], dec), p["y"])
    L = x.shape[1]
    h = np.array([oracle.selective_scan(x[:, :t + 1], delta[:, :t + 1], A, B[:, :t + 1],
                                        C[:, :t + 1], bbar="zoh", return_last_state=True)[1][0, 0]
                  for t in range(L)])
    np.testing.assert_array_equal(np.round(h, dec), p["h"])
    abar = np.array([_discretized_by_oracle(delta[0, t, 0], A[0], B[0, t], "zoh")[0]
                     for t in range(L)])
    np.testing.assert_array_equal(np.round(abar, dec), p["Abar"])


def test_pairwise_combine_tree(golden):
    g = golden["pairwise_combine_tree"]
    p, dec = g["printed"], g["decimals"]
    s = [tuple(v) for v in g["steps"]]
    P12 = forms.combine(s[0], s[1])
    P34 = forms.combine(s[2], s[3])
    P14 = forms.combine(P12, P34)
    np.testing.assert_array_equal(np.round(P12, dec), p["P12"])
    np.testing.assert_array_equal(np.round(P34, dec), p["P34"])
    np.testing.assert_array_equal(np.round(P14, dec), p["P14"])
    assert round(P14[0] * 0.0 + P14[1], dec) == p["h4"]


def test_tree_of_exact_steps_equals_oracle_state(golden):
    """Channel 0 of the selective example: the pairwise tree over the exact
    (Abar_t, Bbar_t x_t) pairs lands on the oracle's final state."""
    g = golden["selective_zoh_four_tokens"]
    x, delta, A, B, C, _ = _selective_example_via_fused(g, "zoh")
    pairs = []
    for t in range(x.shape[1]):
        abar, bbar = _discretized_by_oracle(delta[0, t, 0], A[0], B[0, t], "zoh")
        pairs.append((abar[0], bbar[0] * x[0, t, 0]))
    tree = forms.combine(forms.combine(pairs[0], pairs[1]), forms.combine(pairs[2], pairs[3]))
    _, h_last = oracle.selective_scan(x, delta, A, B, C, bbar="zoh", return_last_state=True)
    assert abs(tree[1] - h_last[0, 0, 0]) < 1e-15


def test_small_delta_limit(golden):
    g = golden["small_delta_limit"]
    p, dec = g["printed"], g["decimals"]
    abar, bbar = _discretized_by_oracle(g["Delta"], g["A"], g["B"], "zoh")
    np.testing.assert_array_equal(np.round(abar, dec), p["Abar"])
    np.testing.assert_array_equal(np.round(bbar, dec), p["Bbar"])
    np.testing.assert_array_equal(np.round(g["Delta"] * np.array(g["B"]), dec), p["DeltaB"])
    # the first-order input term is exactly Delta*B
    _, bbar_e = _discretized_by_oracle(g["Delta"], g["A"], g["B"], "euler")
    np.testing.assert_array_equal(bbar_e, g["Delta"] * np.array(g["B"]))


@pytest.mark.parametrize("key", ["scalar_selective_first_order", "scalar_selective_q3",
                                 "scalar_selective_q4"])
def test_scalar_first_order_examples(golden, key):
    g = golden[key]
    p, tol = g["printed"], g["abs_tol"]
    x = np.array(g["x"])
    delta = oracle.softplus(g["w_delta"] * x + g["b_delta"])
    np.testing.assert_allclose(delta, p["Delta"], rtol=0, atol=tol["Delta"])
    abar, _ = zip(*[_discretized_by_oracle(d, [g["A"]], [g["B"]], "euler") for d in delta])
    abar = np.ravel(abar)
    keep = [i for i in range(len(abar)) if i not in g.get("page_slips", {}).get("Abar", [])]
    np.testing.assert_allclose(abar[keep], np.array(p["Abar"])[keep], rtol=0, atol=tol["Abar"])
    for i in g.get("page_slips", {}).get("Abar", []):        # documented slips on the page
        assert abs(abar[i] - p["Abar"][i]) > tol["Abar"]
    h = _scan1(x, delta, [g["A"]], g["B"], g["C"], "euler")      # C = 1, so y = h
    assert np.all(np.abs(h - np.array(p["h"])) <= np.array(tol["h"])), (h, p["h"])


def test_leaky_bucket_zoh(golden):
    g = golden["leaky_bucket"]
    p = g["printed"]
    y = _scan1(g["x"], g["Delta"], [g["A"]], g["B"], g["C"], "zoh")
    t = np.arange(1, 5)
    np.testing.assert_allclose(y, 1.0 - np.exp(-t), rtol=0, atol=1e-15)   # h(t) = 1 - e^-t
    np.testing.assert_array_equal(np.round(y, 3), p["continuous_h"])
    abar, bbar = _discretized_by_oracle(g["Delta"], [g["A"]], [g["B"]], "zoh")
    assert round(abar[0], 3) == p["Abar"] and round(bbar[0], 3) == p["Bbar"]


@pytest.mark.parametrize("delta", [1e-4, 0.1, 1.0, 7.5])
def test_zoh_convex_combination_identity(delta):
    """A = -1, B = 1: the zero-order-hold pair sums to one (Prerequisites, section 5)."""
    abar, bbar = _discretized_by_oracle(delta, [-1.0], [1.0], "zoh")
    assert abs(abar[0] + bbar[0] - 1.0) < 1e-15


def test_unrolled_and_semiseparable(golden):
    g = golden["unrolled_and_semiseparable"]
    p, dec, tol = g["printed"], g["decimals"], g["abs_tol"]
    T = len(g["x"])
    Abar = np.full((T, 1), g["Abar"])
    Bbar = np.full((T, 1), g["Bbar"])
    terms = [g["Abar"] ** (T - 1 - j) * g["Bbar"] for j in range(T)]
    np.testing.assert_array_equal(np.round(terms, dec["h4_terms"]), p["h4_terms"])
    h_unrolled = forms.unrolled_states(Abar, Bbar, g["x"])[:, 0]
    assert round(h_unrolled[-1], dec["h4"]) == p["h4"]
    Lm = forms.semiseparable(Abar[:, 0])
    np.testing.assert_array_equal(np.round(Lm, dec["L"]), p["L"])
    h_ss = forms.semiseparable_states(Abar, Bbar, g["x"])[:, 0]
    np.testing.assert_allclose(h_ss, p["h"], rtol=0, atol=tol["h"])
    np.testing.assert_allclose(h_unrolled, p["h"], rtol=0, atol=tol["h"])


def test_unit_input_gain_toy(golden):
    """Abar = e^-Delta, Bbar = 1: with the first-order term, B_t = 1/Delta_t gives Bbar = 1."""
    g = golden["unit_input_gain_toy"]
    p, tol = g["printed"], g["abs_tol"]
    d = np.array(g["Delta"])
    y = _scan1(g["u"], d, [-1.0], (1.0 / d)[:, None], 1.0, "euler")
    np.testing.assert_allclose(y, p["x"], rtol=0, atol=tol["x"])
    np.testing.assert_allclose(np.exp(-d), p["Abar"], rtol=0, atol=tol["Abar"])


# --- closed forms and limits ------------------------------------------------------------

@pytest.mark.parametrize("delta", [1e-2, 1e-3, 1e-4])
def test_fine_step_leaky_bucket_first_order(delta):
    """A = -1, B = C = 1, x = 1 with constant Delta: the geometric series gives
    h_n = Delta (1 - e^{-n Delta}) / (1 - e^{-Delta}); as Delta -> 0 this tends to
    the leaky-bucket curve 1 - e^{-t} at t = n Delta (Prerequisites, running example)."""
    steps = int(round(4 / delta))
    y = _scan1(np.ones(steps), delta, [-1.0], 1.0, 1.0, "euler")
    n = np.arange(1, steps + 1)
    closed = delta * (1 - np.exp(-n * delta)) / (1 - np.exp(-delta))
    np.testing.assert_allclose(y, closed, rtol=1e-11, atol=0)
    at_t = y[np.array([1, 2, 3, 4]) * int(round(1 / delta)) - 1]
    exact = 1 - np.exp(-np.arange(1, 5))
    assert np.all(np.abs(at_t - exact) <= delta)          # gap ~ Delta/2 * (1 - e^-t)
    if delta <= 1e-4:
        np.testing.assert_array_equal(np.round(at_t, 3), [0.632, 0.865, 0.950, 0.982])


def test_impulse_response_closed_form():
    """x = impulse at t = 0, constant Delta: y_t = sum_n C_n B_n Delta e^{A_n Delta t}."""
    L, delta = 5000, 1e-3
    A = np.array([-1.0, -2.5, -0.3])
    B = np.array([0.7, -1.2, 0.4])
    C = np.array([1.1, 0.5, -2.0])
    x = np.zeros(L)
    x[0] = 1.0
    y = _scan1(x, delta, A, B, C, "euler")
    t = np.arange(L)[:, None]
    closed = (C * B * delta * np.exp(A * delta * t)).sum(axis=1)
    np.testing.assert_allclose(y, closed, rtol=1e-11, atol=1e-18)


def test_tiny_delta_skips_token():
    rng = np.random.default_rng(0)
    N = 4
    A = -np.arange(1.0, N + 1)
    h0 = rng.standard_normal(N)
    x = rng.standard_normal(6)
    B = rng.standard_normal((6, N))
    _, h = _scan1(x, 1e-18, A, B, np.ones((6, N)), "euler", h0=h0, last=True)
    np.testing.assert_allclose(h, h0, rtol=0, atol=1e-16)


def test_large_delta_forgets_history():
    """Delta |A| >= 800: Abar underflows to 0, so h_t is this step's input term only
    (Delta B x under the first-order term) whatever came before."""
    rng = np.random.default_rng(1)
    N = 3
    A = -np.array([1.0, 2.0, 3.0])
    B = rng.standard_normal((1, N))
    for h0 in (np.zeros(N), 1e6 * rng.standard_normal(N)):
        _, h = _scan1([0.37], 900.0, A, B, np.ones((1, N)), "euler", h0=h0, last=True)
        np.testing.assert_array_equal(h, 900.0 * B[0] * 0.37)


def test_zoh_limit_as_A_goes_to_zero():
    abar0, bbar0 = _discretized_by_oracle(0.3, [0.0], [2.0], "zoh")
    assert abar0[0] == 1.0 and bbar0[0] == pytest.approx(0.6, abs=1e-15)
    _, bbar_small = _discretized_by_oracle(0.3, [-1e-9], [2.0], "zoh")
    assert bbar_small[0] == pytest.approx(0.6, rel=1e-6)


# --- brute-force reformulations ------------------------------------------------------------

def _random_chain(seed, L, N):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(L)
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(1.0), L))
    A = -np.exp(rng.uniform(-1, 1.5, N))
    B = rng.standard_normal((L, N))
    C = rng.standard_normal((L, N))
    return x, delta, A, B, C


@pytest.mark.parametrize("bbar", ["euler", "zoh"])
def test_oracle_matches_unrolled_and_semiseparable(bbar):
    x, delta, A, B, C = _random_chain(2, 7, 3)
    Abar, Bbar = zip(*[forms.discretize(delta[t], A, B[t], bbar) for t in range(len(x))])
    Abar, Bbar = np.array(Abar), np.array(Bbar)
    h_oracle = _states(x, delta, A, B, C, bbar)
    np.testing.assert_allclose(forms.unrolled_states(Abar, Bbar, x), h_oracle, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(forms.semiseparable_states(Abar, Bbar, x), h_oracle, rtol=1e-13, atol=1e-15)
    y = _scan1(x, delta, A, B, C, bbar)
    np.testing.assert_allclose((C * h_oracle).sum(axis=1), y, rtol=1e-13, atol=1e-15)


def test_oracle_matches_convolution_when_time_invariant():
    rng = np.random.default_rng(3)
    N, L = 4, 12
    A = -np.exp(rng.uniform(-1, 1, N))
    B = rng.standard_normal(N)
    C = rng.standard_normal(N)
    x = rng.standard_normal(L)
    for bbar in ("euler", "zoh"):
        abar, bb = forms.discretize(0.2, A, B, bbar)
        K = forms.convolution_kernel(abar, bb, C, L)
        y = _scan1(x, 0.2, A, B, C, bbar)
        np.testing.assert_allclose(y, forms.convolution_output(x, K), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 7])
def test_every_bracketing_equals_sequential(L):
    x, delta, A, B, C = _random_chain(10 + L, L, 3)
    pairs = []
    for t in range(L):
        abar, bbar = forms.discretize(delta[t], A, B[t], "euler")
        pairs.append((abar, bbar * x[t]))
    ref = forms.fold_left(pairs)[-1]
    _, h_last = _scan1(x, delta, A, B, C, "euler", last=True)
    np.testing.assert_allclose(ref[1], h_last, rtol=1e-14, atol=1e-16)
    count = 0
    for tree in forms.bracketings(0, L):
        got = forms.reduce_tree(pairs, tree)
        np.testing.assert_allclose(got[0], ref[0], rtol=1e-14)
        np.testing.assert_allclose(got[1], ref[1], rtol=1e-13, atol=1e-16)
        count += 1
    assert count == math.comb(2 * (L - 1), L - 1) // L        # Catalan number


def test_chunked_and_doubling_scans_equal_sequential():
    L = 9
    x, delta, A, B, C = _random_chain(20, L, 3)
    pairs = [(forms.discretize(delta[t], A, B[t], "euler")[0],
              forms.discretize(delta[t], A, B[t], "euler")[1] * x[t]) for t in range(L)]
    h = _states(x, delta, A, B, C, "euler")
    seq = forms.fold_left(pairs)
    np.testing.assert_allclose(np.array([p[1] for p in seq]), h, rtol=1e-13, atol=1e-16)
    dbl = forms.doubling_scan(pairs)
    np.testing.assert_allclose(np.array([p[1] for p in dbl]), h, rtol=1e-13, atol=1e-16)
    n = 0
    for lengths in forms.all_chunkings(L):
        got = forms.chunked_scan(pairs, lengths)
        np.testing.assert_allclose(np.array([p[1] for p in got]), h, rtol=1e-13, atol=1e-16)
        n += 1
    assert n == 2 ** (L - 1)


# --- structural invariants ------------------------------------------------------------

def _random_batch(seed, batch=2, L=33, D=5, N=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, L, D))
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), (batch, L, D)))
    A = -np.exp(rng.uniform(-1, 1, (D, N)))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    return x, delta, A, B, C


def test_linearity_causality_channel_permutation():
    x, delta, A, B, C = _random_batch(4)
    rng = np.random.default_rng(5)
    x2 = rng.standard_normal(x.shape)
    y1 = oracle.selective_scan(x, delta, A, B, C)
    y2 = oracle.selective_scan(x2, delta, A, B, C)
    y12 = oracle.selective_scan(2.5 * x - 0.75 * x2, delta, A, B, C)
    np.testing.assert_allclose(y12, 2.5 * y1 - 0.75 * y2, rtol=1e-12, atol=1e-13)
    t0 = 17
    xp = x.copy()
    xp[:, t0, :] += 3.0
    yp = oracle.selective_scan(xp, delta, A, B, C)
    np.testing.assert_array_equal(yp[:, :t0], y1[:, :t0])
    assert np.all(np.abs(yp[:, t0] - y1[:, t0]) > 0)
    perm = np.array([3, 0, 4, 1, 2])
    yperm = oracle.selective_scan(x[:, :, perm], delta[:, :, perm], A[perm], B, C)
    np.testing.assert_array_equal(yperm, y1[:, :, perm])


def test_state_continuation_and_decode_steps():
    x, delta, A, B, C = _random_batch(6, L=20)
    y, h = oracle.selective_scan(x, delta, A, B, C, return_last_state=True)
    k = 8
    ya, ha = oracle.selective_scan(x[:, :k], delta[:, :k], A, B[:, :k], C[:, :k],
                                   return_last_state=True)
    yb, hb = oracle.selective_scan(x[:, k:], delta[:, k:], A, B[:, k:], C[:, k:], h0=ha,
                                   return_last_state=True)
    np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
    np.testing.assert_array_equal(hb, h)
    hs = np.zeros(h.shape)
    for t in range(x.shape[1]):
        yt, hs = oracle.selective_scan_step(hs, x[:, t], delta[:, t], A, B[:, t], C[:, t])
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(hs, h)


def test_feedthrough_and_gate():
    x, delta, A, B, C = _random_batch(7)
    rng = np.random.default_rng(8)
    Dk = rng.standard_normal(x.shape[2])
    z = 4 * rng.standard_normal(x.shape)
    y = oracle.selective_scan(x, delta, A, B, C)
    yD = oracle.selective_scan(x, delta, A, B, C, Dskip=Dk)
    np.testing.assert_allclose(yD - y, Dk * x, rtol=1e-12, atol=1e-14)
    yg = oracle.selective_scan(x, delta, A, B, C, Dskip=Dk, z=z)
    np.testing.assert_allclose(yg, yD * z * expit(z), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)


def test_zero_sizes():
    for shape in [(0, 5, 3), (2, 0, 3), (2, 5, 0)]:
        b, L, D = shape
        y, h = oracle.selective_scan(np.zeros(shape), np.zeros(shape), -np.ones((D, 4)),
                                     np.zeros((b, L, 4)), np.zeros((b, L, 4)),
                                     return_last_state=True)
        assert y.shape == shape and h.shape == (b, D, 4)
        assert not np.any(h)


# --- selection and the fused projection path -------------------------------------------

def test_softplus_values_and_identities():
    z = np.linspace(-50, 50, 2001)
    np.testing.assert_allclose(oracle.softplus(z) - oracle.softplus(-z), z, rtol=0, atol=1e-12)
    assert oracle.softplus(800.0) == 800.0                      # no overflow
    assert oracle.softplus(-800.0) == 0.0
    assert oracle.softplus(0.0) == math.log(2.0)
    mid = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(oracle.softplus(mid), np.log1p(np.exp(mid)), rtol=1e-15)


def test_fused_projection_matches_brute_force_matmul():
    rng = np.random.default_rng(9)
    batch, L, D, R, N = 2, 3, 5, 2, 3
    x = rng.standard_normal((batch, L, D))
    W_x = rng.standard_normal((D, R + 2 * N))
    W_dt = rng.standard_normal((R, D))
    bias = rng.standard_normal(D)
    delta, B, C = oracle.selection.fused_projections(x, W_x, W_dt, bias, R=R, N=N)
    for b in range(batch):
        for t in range(L):
            p = [sum(x[b, t, i] * W_x[i, j] for i in range(D)) for j in range(R + 2 * N)]
            for n in range(N):
                assert B[b, t, n] == pytest.approx(p[R + n], abs=1e-13)
                assert C[b, t, n] == pytest.approx(p[R + N + n], abs=1e-13)
            for d in range(D):
                pre = sum(p[r] * W_dt[r, d] for r in range(R)) + bias[d]
                assert delta[b, t, d] == pytest.approx(math.log1p(math.exp(pre)), rel=1e-13)


def test_fused_with_zero_dt_proj_reduces_to_plain_scan():
    rng = np.random.default_rng(11)
    batch, L, D, R, N = 2, 9, 4, 3, 4
    x = rng.standard_normal((batch, L, D))
    W_x = rng.standard_normal((D, R + 2 * N))
    W_dt = np.zeros((R, D))
    bias = rng.standard_normal(D)
    A = -np.arange(1.0, N + 1) * np.ones((D, 1))
    y = oracle.selective_ssm_fused(x, W_x, W_dt, bias, A, R=R)
    proj = x.reshape(-1, D) @ W_x
    delta = np.broadcast_to(np.log1p(np.exp(bias)), x.shape)
    y_ref = oracle.selective_scan(x, delta, A, proj[:, R:R + N].reshape(batch, L, N),
                                  proj[:, R + N:].reshape(batch, L, N))
    np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-15)


def test_round_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    v32 = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                          [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 0.0]]
                         ).astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(v32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert oracle.round_to_bf16(1 + 2 ** -8) == 1.0                 # tie to even
    assert oracle.round_to_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
