"""The Mamba block around the scan -- oracle, TEST INFRASTRUCTURE ONLY.

* causal_conv1d: the depthwise causal convolution of the block listing in
  "Understanding Mamba" (section 10.2): each channel's sequence is left-padded
  with k - 1 zeros and output t is the dot product of padded[t : t + k] with
  the channel's k taps, so tap k - 1 weighs the current token and tap 0 the
  token k - 1 steps back.  An optional per-channel bias is added afterwards.
* mamba_block: eq. (9) of "Understanding Mamba" (section 8.1):
      [u | z] = u0 @ W_in,   x = SiLU(conv(u)),   y = SSM(x),
      out = (y * SiLU(z)) @ W_out,
  with the selective SSM of section 5.1 (Delta, B, C selected from x through
  the low-rank x_proj / dt_proj of ``selection.fused_projections``) and the
  feedthrough D x added to y before the gate (section 2.1: D x is a separate
  term added after everything else).  No normalisation or residual: they sit
  outside the block (section 8.2).

``gemm_inputs_bf16`` (off by default) rounds the inputs of x_proj and W_out
to bfloat16; the GPU path carries them as bf16 hi + lo pairs (about 16
significant bits), so parity runs without rounding.
"""
from __future__ import annotations

import numpy as np

from .scan import selective_scan
from .selection import fused_projections, round_to_bf16, silu


def causal_conv1d(u, w, b=None):
    """Depthwise causal convolution, float64.

    u: [batch, L, D]; w: [D, k] (taps per channel); b: [D] or None.
    out[b, t, d] = sum_i w[d, i] * u[b, t - (k - 1) + i, d] (+ b[d]), with u
    taken as zero before t = 0.
    """
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    batch, L, D = u.shape
    if w.ndim != 2 or w.shape[0] != D:
        raise ValueError("w must be [D, k]")
    k = w.shape[1]
    padded = np.concatenate([np.zeros((batch, k - 1, D)), u], axis=1)
    out = np.zeros((batch, L, D))
    for i in range(k):
        out += w[:, i] * padded[:, i:i + L, :]
    if b is not None:
        out += np.asarray(b, dtype=np.float64)
    return out


def mamba_block(u0, W_in, conv_w, conv_b, W_x, W_dt, dt_bias, A, Dskip, W_out, *, R: int,
                gemm_inputs_bf16: bool = False, bbar: str = "euler", nthreads=None,
                return_parts: bool = False):
    """The block forward of eq. (9), float64 (see the module docstring).

    u0: [batch, L, Dm]; W_in: [Dm, 2 Di] (columns [u | z]); conv_w: [Di, k];
    conv_b: [Di] or None; W_x: [Di, R + 2N]; W_dt: [R, Di]; dt_bias: [Di];
    A: [Di, N]; Dskip: [Di] or None; W_out: [Di, Dm].  Returns out
    [batch, L, Dm] (and the intermediates when ``return_parts``).
    """
    u0 = np.asarray(u0, dtype=np.float64)
    W_in = np.asarray(W_in, dtype=np.float64)
    Di = W_in.shape[1] // 2
    proj = u0 @ W_in
    u, z = proj[..., :Di], proj[..., Di:]
    x = silu(causal_conv1d(u, conv_w, conv_b))
    xq = round_to_bf16(x) if gemm_inputs_bf16 else x
    A = np.asarray(A, dtype=np.float64)
    delta, B, C = fused_projections(xq, W_x, W_dt, dt_bias, R=R, N=A.shape[1])
    # (C . h + D x) * SiLU(z): the scan oracle applies the feedthrough and the gate
    gated = selective_scan(x, delta, A, B, C, bbar=bbar, Dskip=Dskip, z=z, nthreads=nthreads)
    g = round_to_bf16(gated) if gemm_inputs_bf16 else gated
    out = g @ np.asarray(W_out, dtype=np.float64)
    if return_parts:
        return out, {"u": u, "z": z, "x": x, "delta": delta, "B": B, "C": C, "gated": gated}
    return out
