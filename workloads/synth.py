"""Seeded input generation for the five synthetic selective-scan workloads.

Draws are made in float64 with numpy's PCG64 (``default_rng(seed)``), in chunks
of at most 2^24 values (a chunked draw equals one large draw), then cast to
float32 with round-to-nearest-even and, for bfloat16 workloads, to bfloat16
bits with round-to-nearest-even.  Arrays are returned in their storage form:
``np.float32`` for float32 data, ``np.uint16`` holding bfloat16 bits for
bfloat16 data.  A and dt_bias are always float32.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

_CHUNK = 1 << 24


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    L: int
    D: int
    N: int
    dtype: str                 # "fp32" or "bf16": storage type of x, delta, B, C, y, weights
    seed: int
    R: int | None = None       # dt rank of the fused projection workload
    description: str = ""
    Dm: int | None = None      # model width of the Mamba-block workload (D is the inner width)
    conv_k: int | None = None  # causal conv width of the Mamba-block workload

    @property
    def fused(self) -> bool:
        return self.R is not None


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_fp32", 1, 64, 4, 4, "fp32", 5401,
                 description="tiny fp32 scan; x,B,C ~ N(0,1); Delta = softplus(u), "
                             "u ~ N(-2,1); A[d,n] = -(n+1)"),
        Workload("mamba130m_layer_fp32", 8, 2048, 1536, 16, "fp32", 5402,
                 description="Mamba-130M-layer-shaped fp32 scan; x,B,C ~ N(0,1); "
                             "Delta log-uniform in [1e-3, 1e-1]; A[d,n] = -(n+1)"),
        Workload("mid_bf16", 4, 8192, 2048, 16, "bf16", 5403,
                 description="mid-size bf16 scan, fp32 state; x,B,C ~ N(0,1); Delta "
                             "log-uniform in [1e-3, 1e-1]; A = -exp(A_log), "
                             "A_log[d,n] = log(n+1) in fp32"),
        Workload("long_seq_bf16", 1, 131072, 2560, 16, "bf16", 5404,
                 description="long-sequence bf16 scan, fp32 state; x ~ N(0,1); "
                             "B,C ~ N(0, 1/N); Delta log-uniform in [1e-4, 1e-1]; "
                             "A[d,n] = -(n+1)"),
        Workload("fused_proj_bf16", 16, 2048, 5120, 16, "bf16", 5405, R=160,
                 description="fused projection + scan, bf16 weights/activations, fp32 "
                             "state; x ~ N(0,1); x_proj W [D, R+2N] ~ N(0, 1/D); "
                             "dt_proj W [R, D] ~ N(0, 1/R); softplus(dt_bias) "
                             "log-uniform in [1e-3, 1e-1]; A[d,n] = -(n+1)"),
        Workload("decode_step_bf16", 256, 1, 5120, 16, "bf16", 5406,
                 description="one recurrent (decode) step for 256 sequences of a "
                             "D = 5120, N = 16 layer; bf16 token inputs, fp32 state "
                             "[batch, D, N] ~ N(0, 1/4); x, z, B, C ~ N(0,1); Delta "
                             "log-uniform in [1e-3, 1e-1]; Dskip ~ N(0,1); "
                             "A[d,n] = -(n+1)"),
    )
}

WORKLOADS["mamba_block_bf16"] = Workload(
    "mamba_block_bf16", 16, 2048, 5120, 16, "bf16", 5407, R=160, Dm=2560, conv_k=4,
    description="Mamba block forward (in_proj, causal conv1d + SiLU, selective SSM with "
                "x_proj/dt_proj, D x, SiLU(z) gate, out_proj) at the fused workload's inner "
                "shape: model width 2560, inner width 5120, conv width 4; bf16 u0 ~ N(0,1) "
                "and weights W_in ~ N(0, 1/2560), W_x ~ N(0, 1/5120), W_dt ~ N(0, 1/160), "
                "W_out ~ N(0, 1/5120); float32 conv taps ~ N(0, 1/4), conv bias ~ "
                "N(0, 0.01), Dskip ~ N(0,1); softplus(dt_bias) log-uniform in [1e-3, 1e-1]; "
                "A[d,n] = -(n+1)")

# Workloads that are one full-sequence scan (the others: the decode step, the block).
SCAN_WORKLOADS = ("tiny_fp32", "mamba130m_layer_fp32", "mid_bf16", "long_seq_bf16",
                  "fused_proj_bf16")


def workload(name: str, **overrides) -> Workload:
    """The named workload, optionally with other sizes (batch, L, D, N, R, seed)."""
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def bf16_bits_from_float32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round to nearest, ties to even."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits (uint16) -> the float32 values they encode (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float64(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of a storage-form array (float32, or uint16 bf16 bits)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_float32(a).astype(np.float64)
    return a.astype(np.float64)


def _encode(v64: np.ndarray, dtype: str) -> np.ndarray:
    v32 = v64.astype(np.float32)
    return bf16_bits_from_float32(v32) if dtype == "bf16" else v32


def _draw(rng, n: int, dtype: str, kind: str, p0: float, p1: float) -> np.ndarray:
    """n values, chunked: kind "normal" (mean p0, std p1) or "loguniform" [p0, p1]."""
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if kind == "loguniform":
        lo, hi = np.log(p0), np.log(p1)
    for s in range(0, n, _CHUNK):
        k = min(_CHUNK, n - s)
        if kind == "normal":
            v = rng.standard_normal(k) * p1 + p0
        elif kind == "loguniform":
            v = np.exp(lo + (hi - lo) * rng.random(k))
        elif kind == "softplus_normal":
            v = np.logaddexp(0.0, rng.standard_normal(k) * p1 + p0)
        else:
            raise ValueError(kind)
        out[s:s + k] = _encode(v, dtype)
    return out


def _a_matrix(w: Workload) -> np.ndarray:
    n1 = np.arange(1, w.N + 1, dtype=np.float64)
    if w.name == "mid_bf16":
        a_log = np.log(n1).astype(np.float32)                  # A_log in fp32
        row = (-np.exp(a_log.astype(np.float64))).astype(np.float32)
    else:
        row = (-n1).astype(np.float32)
    return np.ascontiguousarray(np.broadcast_to(row, (w.D, w.N)))


def generate(w: Workload | str, **overrides) -> dict:
    """Draw the inputs of workload ``w`` (a Workload or its name).

    Plain scan workloads return x, delta, A, B, C; the fused workload returns
    x, W_x, W_dt, dt_bias, A.  Also returned: "workload" (the Workload).
    """
    if isinstance(w, str):
        w = workload(w, **overrides)
    elif overrides:
        w = replace(w, **overrides)
    rng = np.random.default_rng(w.seed)
    BLD = w.batch * w.L * w.D
    BLN = w.batch * w.L * w.N
    out = {"workload": w}
    if w.name == "fused_proj_bf16":
        R = w.R
        out["x"] = _draw(rng, BLD, w.dtype, "normal", 0.0, 1.0).reshape(w.batch, w.L, w.D)
        out["W_x"] = _draw(rng, w.D * (R + 2 * w.N), w.dtype, "normal", 0.0,
                           1.0 / np.sqrt(w.D)).reshape(w.D, R + 2 * w.N)
        out["W_dt"] = _draw(rng, R * w.D, w.dtype, "normal", 0.0,
                            1.0 / np.sqrt(R)).reshape(R, w.D)
        d0 = _draw(rng, w.D, "fp32", "loguniform", 1e-3, 1e-1).astype(np.float64)
        out["dt_bias"] = np.log(np.expm1(d0)).astype(np.float32)
        out["A"] = _a_matrix(w)
        return out
    bc_std = 1.0 / np.sqrt(w.N) if w.name == "long_seq_bf16" else 1.0
    out["x"] = _draw(rng, BLD, w.dtype, "normal", 0.0, 1.0).reshape(w.batch, w.L, w.D)
    if w.name == "tiny_fp32":
        delta = _draw(rng, BLD, w.dtype, "softplus_normal", -2.0, 1.0)
    elif w.name == "long_seq_bf16":
        delta = _draw(rng, BLD, w.dtype, "loguniform", 1e-4, 1e-1)
    else:
        delta = _draw(rng, BLD, w.dtype, "loguniform", 1e-3, 1e-1)
    out["delta"] = delta.reshape(w.batch, w.L, w.D)
    out["B"] = _draw(rng, BLN, w.dtype, "normal", 0.0, bc_std).reshape(w.batch, w.L, w.N)
    out["C"] = _draw(rng, BLN, w.dtype, "normal", 0.0, bc_std).reshape(w.batch, w.L, w.N)
    out["A"] = _a_matrix(w)
    return out


def generate_extras(w: Workload | str, seed_offset: int = 1000, **overrides) -> dict:
    """Inputs for the scan's optional parts, for workload ``w``'s shape.

    Dskip [D] ~ N(0,1) float32, z [batch, L, D] ~ N(0,1) in the workload's
    storage type, h0 [batch, D, N] ~ N(0, 1/4) float32; drawn in that order
    from default_rng(seed + seed_offset).
    """
    if isinstance(w, str):
        w = workload(w, **overrides)
    elif overrides:
        w = replace(w, **overrides)
    rng = np.random.default_rng(w.seed + seed_offset)
    return {
        "Dskip": _draw(rng, w.D, "fp32", "normal", 0.0, 1.0),
        "z": _draw(rng, w.batch * w.L * w.D, w.dtype, "normal", 0.0, 1.0).reshape(
            w.batch, w.L, w.D),
        "h0": _draw(rng, w.batch * w.D * w.N, "fp32", "normal", 0.0, 0.5).reshape(
            w.batch, w.D, w.N),
    }


def generate_step(w: Workload | str = "decode_step_bf16", **overrides) -> dict:
    """Inputs of one decode step: x, delta, z [batch, D]; B, C [batch, N];
    A [D, N]; Dskip [D]; h [batch, D, N] float32 (the state before the step).
    Draw order: x, delta, B, C, z, Dskip, h."""
    if isinstance(w, str):
        w = workload(w, **overrides)
    elif overrides:
        w = replace(w, **overrides)
    rng = np.random.default_rng(w.seed)
    BD, BN = w.batch * w.D, w.batch * w.N
    out = {"workload": w}
    out["x"] = _draw(rng, BD, w.dtype, "normal", 0.0, 1.0).reshape(w.batch, w.D)
    out["delta"] = _draw(rng, BD, w.dtype, "loguniform", 1e-3, 1e-1).reshape(w.batch, w.D)
    out["B"] = _draw(rng, BN, w.dtype, "normal", 0.0, 1.0).reshape(w.batch, w.N)
    out["C"] = _draw(rng, BN, w.dtype, "normal", 0.0, 1.0).reshape(w.batch, w.N)
    out["z"] = _draw(rng, BD, w.dtype, "normal", 0.0, 1.0).reshape(w.batch, w.D)
    out["Dskip"] = _draw(rng, w.D, "fp32", "normal", 0.0, 1.0)
    out["h"] = _draw(rng, BD * w.N, "fp32", "normal", 0.0, 0.5).reshape(w.batch, w.D, w.N)
    out["A"] = _a_matrix(w)
    return out


def generate_block(w: Workload | str = "mamba_block_bf16", **overrides) -> dict:
    """Inputs of the Mamba-block workload: u0 [batch, L, Dm], W_in [Dm, 2 Di],
    conv_w [Di, k], conv_b [Di], W_x [Di, R + 2N], W_dt [R, Di], dt_bias [Di],
    A [Di, N], Dskip [Di], W_out [Di, Dm] (Di = D).  Draw order as listed."""
    if isinstance(w, str):
        w = workload(w, **overrides)
    elif overrides:
        w = replace(w, **overrides)
    rng = np.random.default_rng(w.seed)
    Dm, Di, R, N, k = w.Dm, w.D, w.R, w.N, w.conv_k
    out = {"workload": w}
    out["u0"] = _draw(rng, w.batch * w.L * Dm, w.dtype, "normal", 0.0, 1.0).reshape(
        w.batch, w.L, Dm)
    out["W_in"] = _draw(rng, Dm * 2 * Di, w.dtype, "normal", 0.0, 1.0 / np.sqrt(Dm)).reshape(
        Dm, 2 * Di)
    out["conv_w"] = _draw(rng, Di * k, "fp32", "normal", 0.0, 1.0 / np.sqrt(k)).reshape(Di, k)
    out["conv_b"] = _draw(rng, Di, "fp32", "normal", 0.0, 0.1)
    out["W_x"] = _draw(rng, Di * (R + 2 * N), w.dtype, "normal", 0.0,
                       1.0 / np.sqrt(Di)).reshape(Di, R + 2 * N)
    out["W_dt"] = _draw(rng, R * Di, w.dtype, "normal", 0.0, 1.0 / np.sqrt(R)).reshape(R, Di)
    d0 = _draw(rng, Di, "fp32", "loguniform", 1e-3, 1e-1).astype(np.float64)
    out["dt_bias"] = np.log(np.expm1(d0)).astype(np.float32)
    out["A"] = _a_matrix(w)
    out["Dskip"] = _draw(rng, Di, "fp32", "normal", 0.0, 1.0)
    out["W_out"] = _draw(rng, Di * Dm, w.dtype, "normal", 0.0, 1.0 / np.sqrt(Di)).reshape(Di, Dm)
    return out
