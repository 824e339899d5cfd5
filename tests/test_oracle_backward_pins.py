"""Pins for the backward oracle (oracle/backward.py): every gradient against
central finite differences of the forward oracle (float64, tiny inputs), plus
closed forms of the single-step case."""
import numpy as np
import pytest

import oracle
from oracle.backward import selective_scan_backward


def _case(seed, batch=2, L=7, D=3, N=4, parts=True):
    rng = np.random.default_rng(seed)
    c = dict(x=rng.standard_normal((batch, L, D)),
             delta=np.exp(rng.uniform(np.log(0.01), np.log(0.5), (batch, L, D))),
             A=-np.exp(rng.uniform(0.0, 1.5, (D, N))),
             B=rng.standard_normal((batch, L, N)), C=rng.standard_normal((batch, L, N)))
    extra = dict(Dskip=rng.standard_normal(D), z=rng.standard_normal((batch, L, D)),
                 h0=0.5 * rng.standard_normal((batch, D, N))) if parts else {}
    dout = rng.standard_normal((batch, L, D))
    return c, extra, dout


def _loss(c, extra, dout):
    return float(np.sum(dout * oracle.selective_scan(c["x"], c["delta"], c["A"], c["B"], c["C"],
                                                     **extra)))


def _fd(c, extra, dout, group, name, eps=1e-6):
    src = c if group == "c" else extra
    base = src[name]
    g = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = base[i]
        base[i] = old + eps
        lp = _loss(c, extra, dout)
        base[i] = old - eps
        lm = _loss(c, extra, dout)
        base[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


NAMES = [("c", "x", "dx"), ("c", "delta", "ddelta"), ("c", "A", "dA"), ("c", "B", "dB"),
         ("c", "C", "dC"), ("e", "Dskip", "dD"), ("e", "z", "dz"), ("e", "h0", "dh0")]


@pytest.mark.parametrize("group,name,key", NAMES, ids=[n[2] for n in NAMES])
def test_gradients_match_finite_differences(group, name, key):
    c, extra, dout = _case(1)
    grads = selective_scan_backward(c["x"], c["delta"], c["A"], c["B"], c["C"], dout, **extra)
    fd = _fd(c, extra, dout, group, name)
    np.testing.assert_allclose(grads[key], fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("group,name,key", NAMES[:5], ids=[n[2] for n in NAMES[:5]])
def test_gradients_without_optional_parts(group, name, key):
    c, extra, dout = _case(2, parts=False)
    grads = selective_scan_backward(c["x"], c["delta"], c["A"], c["B"], c["C"], dout)
    assert set(grads) == {"dx", "ddelta", "dA", "dB", "dC"}
    np.testing.assert_allclose(grads[key], _fd(c, extra, dout, group, name), rtol=1e-6,
                               atol=1e-7)


def test_single_step_closed_forms():
    """L = 1 from h = 0: out = (delta (B . C) x + D x) SiLU(z), so e.g.
    dC_n = g delta B_n x and dx = g (delta B . C + D), with g = dout SiLU(z)."""
    c, extra, dout = _case(3, batch=1, L=1, D=1, N=3)
    extra.pop("h0")
    gr = selective_scan_backward(c["x"], c["delta"], c["A"], c["B"], c["C"], dout, **extra)
    x, d, B, C = c["x"][0, 0, 0], c["delta"][0, 0, 0], c["B"][0, 0], c["C"][0, 0]
    zz, Dk, g0 = extra["z"][0, 0, 0], extra["Dskip"][0], dout[0, 0, 0]
    g = g0 * zz / (1 + np.exp(-zz))
    np.testing.assert_allclose(gr["dC"][0, 0], g * d * B * x, rtol=1e-13)
    np.testing.assert_allclose(gr["dx"][0, 0, 0], g * (d * B @ C + Dk), rtol=1e-13)
    np.testing.assert_allclose(gr["ddelta"][0, 0, 0], g * (B @ C) * x, rtol=1e-13)
    np.testing.assert_allclose(gr["dA"], 0.0, atol=0)          # h_{-1} = 0
    np.testing.assert_allclose(gr["dD"][0], g * x, rtol=1e-13)
