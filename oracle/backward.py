"""Gradients of the selective scan -- oracle, TEST INFRASTRUCTURE ONLY.

The backward pass of the recurrence of "Understanding Mamba" section 2.3
eq. (3) with the first-order input term ("Selective State Space Models",
section "Selection"), the optional feedthrough D x (eq. (1)/(3)), the optional
SiLU(z) gate (section 8.1 eq. (9)) and an optional initial state.  The pages
only say the backward recomputes the states rather than storing them ("State
Space Models and Mamba", hardware-aware scan); the gradients themselves are
the plain chain rule through the forward loop, written out here:

    forward   a_t = exp(delta_t A),  h_t = a_t h_{t-1} + delta_t B_t x_t,
              y_t = C_t . h_t + D x_t,  out_t = y_t SiLU(z_t)
    given     dout_t = dL/dout_t
    gate      g_t = dout_t SiLU(z_t),  dz_t = dout_t y_t SiLU'(z_t)
    adjoint   lam_t = C_t g_t + a_{t+1} lam_{t+1}          (lam_L = 0)
    then      dC_t = g_t h_t                   (summed over channels d)
              dB_t = lam_t delta_t x_t         (summed over channels d)
              dx_t = g_t D + sum_n lam_t delta_t B_t
              ddelta_t = sum_n lam_t (B_t x_t + A a_t h_{t-1})
              dA = sum_t lam_t delta_t a_t h_{t-1}    (summed over batch too)
              dD = sum_t g_t x_t                      (summed over batch too)
              dh0 = a_0 lam_0

Evaluated in float64, vectorised over (channel, state) and sequential in time,
one batch row at a time (the row's states [L, D, N] are kept).  Pinned by
central finite differences of the forward oracle (tests/test_oracle_backward_pins.py).
"""
from __future__ import annotations

import numpy as np


def _silu_and_slope(v):
    s = 1.0 / (1.0 + np.exp(-v))
    return v * s, s * (1.0 + v * (1.0 - s))


def selective_scan_backward(x, delta, A, B, C, dout, *, Dskip=None, z=None, h0=None):
    """Gradients of L = sum(dout * out) for out = selective_scan(x, delta, A, B,
    C, Dskip=Dskip, z=z, h0=h0) (first-order input term), float64.

    Returns a dict with dx, ddelta [batch, L, D]; dA [D, N]; dB, dC [batch, L, N];
    and dD [D], dz [batch, L, D], dh0 [batch, D, N] for the parts given.
    """
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    x, delta, A, B, C, dout = map(f, (x, delta, A, B, C, dout))
    Dk, z, h0 = f(Dskip), f(z), f(h0)
    batch, L, D = x.shape
    N = A.shape[1]
    out = {"dx": np.zeros((batch, L, D)), "ddelta": np.zeros((batch, L, D)),
           "dA": np.zeros((D, N)), "dB": np.zeros((batch, L, N)), "dC": np.zeros((batch, L, N))}
    if Dk is not None:
        out["dD"] = np.zeros(D)
    if z is not None:
        out["dz"] = np.zeros((batch, L, D))
    if h0 is not None:
        out["dh0"] = np.zeros((batch, D, N))
    for b in range(batch):
        xb, db, Bb, Cb, gb = x[b], delta[b], B[b], C[b], dout[b]
        hist = np.empty((L + 1, D, N))
        hist[0] = h0[b] if h0 is not None else 0.0
        for t in range(L):                                   # forward, states kept
            a = np.exp(db[t][:, None] * A)
            hist[t + 1] = a * hist[t] + (db[t] * xb[t])[:, None] * Bb[t][None, :]
        y = np.einsum("tdn,tn->td", hist[1:], Cb)
        if Dk is not None:
            y = y + Dk * xb
        if z is not None:
            sz, slope = _silu_and_slope(z[b])
            g = gb * sz
            out["dz"][b] = gb * y * slope
        else:
            g = gb
        if Dk is not None:
            out["dD"] += np.sum(g * xb, axis=0)
            out["dx"][b] += g * Dk
        lam_next = np.zeros((D, N))                          # a_{t+1} lam_{t+1}
        for t in range(L - 1, -1, -1):                       # reverse
            a = np.exp(db[t][:, None] * A)
            lam = Cb[t][None, :] * g[t][:, None] + lam_next
            hprev = hist[t]
            out["dC"][b, t] = g[t] @ hist[t + 1]
            out["dB"][b, t] = (db[t] * xb[t]) @ lam
            out["dx"][b, t] += db[t] * (lam @ Bb[t])
            out["ddelta"][b, t] = np.sum(lam * (Bb[t][None, :] * xb[t][:, None] + A * a * hprev),
                                         axis=1)
            out["dA"] += lam * db[t][:, None] * a * hprev
            lam_next = a * lam
        if h0 is not None:
            out["dh0"][b] = lam_next
    return out
