"""Selection and the fused projection path -- oracle, TEST INFRASTRUCTURE ONLY.

* softplus(z) = ln(1 + e^z)  ("Understanding Mamba", section 5.1; the traced
  example of "State Space Models and Mamba").  Evaluated in the overflow-free
  form max(z, 0) + log1p(exp(-|z|)), which is the same function.
* SiLU(v) = v * sigmoid(v)  ("Understanding Mamba", section 8.1).
* The fused selective SSM: the selection projections of eq. (6) in the low-rank
  Mamba shape -- x_proj maps each token x_t (length D) to R + 2N values split,
  in this order, into dt_low (R), B_t (N) and C_t (N); dt_proj maps dt_low back
  to D channels, a per-channel bias is added and softplus gives Delta_t.  The
  scan then runs on (x, Delta, A, B, C).  Weights are [in, out] (y = x @ W).
"""
from __future__ import annotations

import numpy as np

from .scan import selective_scan


def softplus(z):
    """ln(1 + e^z) in float64, overflow-free form."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def silu(v):
    """v / (1 + e^-v) in float64."""
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def round_to_bf16(v):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range; values below
    2^-126 are quantised to multiples of 2^-133 (bfloat16 subnormals).  Returned
    as float64.  Used only where the GPU path rounds an intermediate to bf16.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    normal = np.ldexp(np.rint(m * 256.0), e - 8)   # 8 significant bits, RNE
    sub = np.ldexp(np.rint(np.ldexp(v, 133)), -133)
    return np.where(np.abs(v) < 2.0 ** -126, sub, normal)


def fused_projections(x, W_x, W_dt, dt_bias, *, R: int, N: int, dt_low_bf16: bool = False):
    """Return (delta, B, C) from the token projections, all float64.

    x: [batch, L, D]; W_x: [D, R + 2N]; W_dt: [R, D]; dt_bias: [D].
    ``dt_low_bf16`` rounds dt_low to bfloat16 before dt_proj (kept as an option;
    the GPU path carries dt_low to about 16 significant bits, so parity runs
    with it off); B, C and the pre-softplus value are kept unrounded.
    """
    x = np.asarray(x, dtype=np.float64)
    batch, L, D = x.shape
    W_x = np.asarray(W_x, dtype=np.float64)
    W_dt = np.asarray(W_dt, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    if W_x.shape != (D, R + 2 * N):
        raise ValueError(f"W_x must be [D, R+2N] = {(D, R + 2 * N)}, got {W_x.shape}")
    if W_dt.shape != (R, D):
        raise ValueError(f"W_dt must be [R, D] = {(R, D)}, got {W_dt.shape}")
    if dt_bias.shape != (D,):
        raise ValueError("dt_bias must be [D]")
    tokens = x.reshape(batch * L, D)
    proj = tokens @ W_x                          # x_proj
    dt_low = proj[:, :R]
    B = proj[:, R:R + N]
    C = proj[:, R + N:R + 2 * N]
    if dt_low_bf16:
        dt_low = round_to_bf16(dt_low)
    pre = dt_low @ W_dt + dt_bias                # dt_proj plus bias
    delta = softplus(pre)
    return (delta.reshape(batch, L, D), B.reshape(batch, L, N), C.reshape(batch, L, N))


def selective_ssm_fused(x, W_x, W_dt, dt_bias, A, *, R: int, bbar: str = "euler",
                        dt_low_bf16: bool = False, Dskip=None, z=None, h0=None,
                        return_last_state: bool = False, nthreads=None):
    """Projections then the sequential scan, float64.

    Pinned by the selective worked example of "Understanding Mamba" section 5.3
    (one channel, R = 1: Delta_t = softplus(2 x_t), B_t = C_t = 0.4 x_t) and by
    the reduction to the plain scan when W_dt = 0 (Delta = softplus(bias)).
    """
    A = np.asarray(A)
    N = A.shape[1]
    delta, B, C = fused_projections(x, W_x, W_dt, dt_bias, R=R, N=N, dt_low_bf16=dt_low_bf16)
    return selective_scan(x, delta, A, B, C, bbar=bbar, Dskip=Dskip, z=z, h0=h0,
                          return_last_state=return_last_state, nthreads=nthreads)
