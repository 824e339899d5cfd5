"""Helpers for the GPU parity tests: device transfer, oracle calls, tolerances.

The tolerance is the one the method is held to: for float32 data
|y - y_ref| <= 1e-4 (1 + |y_ref|); for bfloat16 data with a float32 state,
|y - y_ref| <= 2e-3 (1 + |y_ref|), where y_ref is the float64 oracle on the same
(rounded) inputs.
"""
import os

import numpy as np

import oracle
import workloads

TOL = {"fp32": 1e-4, "bf16": 2e-3}
ORACLE_THREADS = min(os.cpu_count() or 1, 16)


def torch_mod():
    import torch
    return torch


def dev(a):
    """Storage-form numpy array (float32, or uint16 bf16 bits) -> GPU tensor."""
    torch = torch_mod()
    a = np.array(a, copy=True, order="C")
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def inputs_on_device(g):
    return {k: dev(g[k]) for k in ("x", "delta", "A", "B", "C") if k in g}


def oracle_scan(g, channels=None, **kw):
    """float64 oracle on the generator's exact values; optionally only some channels."""
    x = workloads.to_float64(g["x"])
    delta = workloads.to_float64(g["delta"])
    A = g["A"].astype(np.float64)
    if channels is not None:
        x = x[:, :, channels]
        delta = delta[:, :, channels]
        A = A[channels]
    return oracle.selective_scan(x, delta, A, workloads.to_float64(g["B"]),
                                 workloads.to_float64(g["C"]), nthreads=ORACLE_THREADS, **kw)


def parity_report(y_gpu, y_ref, dtype):
    err = np.abs(y_gpu - y_ref)
    bound = TOL[dtype] * (1.0 + np.abs(y_ref))
    ratio = float((err / bound).max()) if err.size else 0.0
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    return {"max_err_over_bound": ratio, "max_abs_err": float(err.max()) if err.size else 0.0,
            "max_err_over_rms": float(err.max() / rms) if rms > 0 else 0.0,
            "finite": bool(np.isfinite(y_gpu).all())}


def assert_parity(y_gpu, y_ref, dtype, what=""):
    r = parity_report(y_gpu, y_ref, dtype)
    assert r["finite"], f"{what}: non-finite GPU output"
    assert r["max_err_over_bound"] <= 1.0, f"{what}: {r}"
    return r
