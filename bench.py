#!/usr/bin/env python3
"""Selective-scan benchmark on one MI355X; prints ONE JSON line.

A step is one full pass of the hot path (discretise, recurrence, read-out,
store) over one batch of the workload, inputs already in HBM.  With at least
8192 channels (batch * D) and N = 16 the library runs the single-pass kernel
(one lane per channel and state); otherwise the chunked kernels (summaries,
carries, output).  The headline workload is the Mamba-130M-layer-shaped float32 scan
(batch 8, L 2048, D 1536, N 16); the other synthetic workloads are measured
the same way with fewer steps and reported under "workloads".

value    = algorithmic bytes per step * steps / wall time of the timed region
           (bytes = (x + delta + y) over batch*L*D plus (B + C) over batch*L*N)
roofline = the scan kernel against its binding roof.  The scan is bound by
           vector-ALU issue: each (b, t, d, n) element needs 4 single-rate fp32
           VALU operations and one half-rate v_exp_f32 = 6 lane-issue slots; the
           chip issues 256 CU * 4 SIMD * 16 lanes * 2.4 GHz = 39.32e12 slots/s,
           so the element roof is 6553.6 Gelem/s.  Kernel time comes from HIP
           events recorded on the stream the kernels are launched on.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
VALU_LANE_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
SLOTS_PER_ELEMENT = 6
ELEM_PEAK_GPS = VALU_LANE_SLOTS_PER_S / SLOTS_PER_ELEMENT / 1e9
HEADLINE = "mamba130m_layer_fp32"
OTHERS = ["tiny_fp32", "mid_bf16", "long_seq_bf16", "fused_proj_bf16"]


def algorithmic_bytes(w) -> int:
    e = 4 if w.dtype == "fp32" else 2
    return (3 * w.batch * w.L * w.D + 2 * w.batch * w.L * w.N) * e


def elements(w) -> int:
    return w.batch * w.L * w.D * w.N


# The sources the headline scan's kernel (the single pass: first-order input
# term, no optional parts) is built from; the traffic record is tied to their
# hash.
HEADLINE_SOURCES = ("scan_device.h", "chain_scan.h", "chain_scan.hip", "chain_euler_plain.hip",
                    "scan_kernels.hip", "mssm_internal.h")


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    for name in HEADLINE_SOURCES:
        with open(os.path.join(ROOT, "selective_state_space_54_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str):
    """HBM bytes per step measured with rocprofv3 counters, if they were taken
    on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel_sources_sha256") != kernel_sources_digest():
        return None
    return rec.get("hbm_bytes_per_step")


def device_inputs(g, torch):
    import numpy as np
    out = {}
    for k in ("x", "delta", "A", "B", "C"):
        a = np.ascontiguousarray(g[k])
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a)
        out[k] = t.cuda()
    return out


def time_workload(name, steps, warmup, rotate, torch, mssm, workloads):
    w = workloads.workload(name)
    sets = []
    for r in range(rotate):
        g = workloads.generate(name, seed=w.seed + 1000 * r)
        d = device_inputs(g, torch)
        d["y"] = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")
        sets.append(d)
        del g
    nbytes = mssm.mssm_selective_scan_workspace_size(w.batch, w.L, w.D, w.N, sets[0]["x"].dtype)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    # validated once; each step issues the C call directly
    calls = [mssm.prepare_selective_scan_fwd_ws(d["x"], d["delta"], d["A"], d["B"], d["C"],
                                                d["y"], ws) for d in sets]

    def step(i):
        calls[i % rotate]()

    for i in range(warmup):
        step(i)
    # One event pair around the whole timed region, on the stream the library
    # launches on: the average launch duration is its elapsed time / steps
    # (launches queue back to back, so this is kernel time plus the gaps
    # between launches, not the cost of per-step event records).
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = start.elapsed_time(end) / steps
    del sets, ws, calls
    torch.cuda.empty_cache()
    return w, wall, kernel_ms


def time_fused(name, steps, warmup, torch, mssm, workloads):
    """The fused path per step: W_x transpose, x_proj GEMM, dt_low split, W_dt
    transpose, then (>= 8192 channels) the Delta kernel and the single-pass
    scan, or the chunked fused summary / carry / output kernels."""
    import numpy as np
    w = workloads.workload(name)
    g = workloads.generate(name)
    d = {}
    for k in ("x", "W_x", "W_dt", "dt_bias", "A"):
        a = np.ascontiguousarray(g[k])
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a)
        d[k] = t.cuda()
    del g
    y = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")
    nb = mssm.mssm_selective_ssm_fused_workspace_size(w.batch, w.L, w.D, w.N, w.R, torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def step():
        mssm.mssm_selective_ssm_fused_fwd(d["x"], d["W_x"], d["W_dt"], d["dt_bias"], d["A"], y, ws)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s_ev.record(stream)
    for _ in range(steps):
        step()
    e_ev.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = s_ev.elapsed_time(e_ev) / steps
    del d, y, ws
    torch.cuda.empty_cache()
    return w, wall, kernel_ms


def _to_device(a, torch):
    import numpy as np
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
        else torch.from_numpy(a)
    return t.cuda()


def time_scan_ex(name, steps, warmup, torch, mssm, workloads):
    """The scan with every optional part on: exact zero-order hold, feedthrough,
    SiLU(z) gate, initial state in and final state out."""
    w = workloads.workload(name)
    g = workloads.generate(name)
    e = workloads.generate_extras(w)
    d = device_inputs(g, torch)
    for k in ("Dskip", "z", "h0"):
        d[k] = _to_device(e[k], torch)
    del g, e
    d["y"] = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")
    d["h_last"] = torch.empty(d["h0"].shape, dtype=torch.float32, device="cuda")
    nbytes = mssm.mssm_selective_scan_workspace_size(w.batch, w.L, w.D, w.N, d["x"].dtype)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        mssm.mssm_selective_scan_fwd_ex(d["x"], d["delta"], d["A"], d["B"], d["C"], d["y"], ws,
                                        Dskip=d["Dskip"], z=d["z"], h0=d["h0"],
                                        h_last=d["h_last"], bbar="zoh")

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for _ in range(steps):
        step()
    e_ev.record(stream)
    torch.cuda.synchronize()
    kernel_ms = s_ev.elapsed_time(e_ev) / steps
    el = 4 if w.dtype == "fp32" else 2
    nb = (4 * w.batch * w.L * w.D * el + 2 * w.batch * w.L * w.N * el
          + 2 * w.batch * w.D * w.N * 4 + w.D * 4)
    del d, ws
    torch.cuda.empty_cache()
    return {"kernel_ms": round(kernel_ms, 4),
            "GB/s": round(nb / (kernel_ms * 1e-3) / 1e9, 1),
            "Gelem/s": round(elements(w) / (kernel_ms * 1e-3) / 1e9, 1),
            "note": "bbar zoh, Dskip, z gate, h0 in, h_last out; bytes = x + Delta + z + y, "
                    "B + C, h0 + h_last, Dskip"}


def decode_bytes(w) -> int:
    el = 4 if w.dtype == "fp32" else 2
    return (2 * w.batch * w.D * w.N * 4            # state read and written
            + 3 * w.batch * w.D * el + w.batch * w.D * 4   # x, delta, z in; y out
            + 2 * w.batch * w.N * el                # B, C
            + w.D * w.N * 4 + w.D * 4)              # A, Dskip


def time_decode(name, steps, warmup, torch, mssm, workloads, states=4):
    """One decode step per call over `states` rotating state buffers (their
    total exceeds the 256 MB last-level cache, so the state comes from HBM)."""
    w = workloads.workload(name)
    s = workloads.generate_step(name)
    d = {k: _to_device(s[k], torch) for k in ("x", "delta", "A", "B", "C", "z", "Dskip")}
    hs = [_to_device(s["h"], torch) for _ in range(states)]
    del s
    y = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")

    def step(i):
        mssm.mssm_selective_scan_step(d["x"], d["delta"], d["A"], d["B"], d["C"], hs[i % states],
                                      y, Dskip=d["Dskip"], z=d["z"])

    for i in range(warmup):
        step(i)
    stream = torch.cuda.current_stream()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for i in range(steps):
        step(i)
    e_ev.record(stream)
    torch.cuda.synchronize()
    kernel_ms = s_ev.elapsed_time(e_ev) / steps
    nb = decode_bytes(w)
    del d, hs, y
    torch.cuda.empty_cache()
    gbs = nb / (kernel_ms * 1e-3) / 1e9
    return {"kernel_ms": round(kernel_ms, 5), "GB/s": round(gbs, 1),
            "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
            "tokens_channels_per_s": round(w.batch * w.D / (kernel_ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "bytes_per_launch": nb},
            "note": f"selective_step_kernel, batch {w.batch}, D {w.D}, N {w.N}, bf16 token "
                    f"inputs, fp32 state; Dskip and z gate on; {states} rotating states"}


def time_block(name, steps, warmup, torch, mssm, workloads):
    """The Mamba block forward: in_proj (2 GEMMs), conv1d + SiLU, x_proj (hi and
    lo GEMMs), dt_low split, the fused scan with feedthrough and gate, out_proj
    (hi and lo GEMMs)."""
    w = workloads.workload(name)
    g = workloads.generate_block(name)
    keys = ("u0", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "dt_bias", "A", "Dskip", "W_out")
    d = {k: _to_device(g[k], torch) for k in keys}
    del g
    M, Dm, Di, N, R = w.batch * w.L, w.Dm, w.D, w.N, w.R
    out = torch.empty((w.batch, w.L, Dm), dtype=torch.float32, device="cuda")
    nb = mssm.mssm_mamba_block_workspace_size(w.batch, w.L, Dm, Di, N, R, w.conv_k,
                                              torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def step():
        mssm.mssm_mamba_block_fwd(*(d[k] for k in keys), out, ws)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for _ in range(steps):
        step()
    e_ev.record(stream)
    torch.cuda.synchronize()
    kernel_ms = s_ev.elapsed_time(e_ev) / steps
    gemm_flops = 2 * M * Dm * 2 * Di + 2 * 2 * M * Di * (R + 2 * N) + 2 * 2 * M * Di * Dm
    del d, out, ws
    torch.cuda.empty_cache()
    return {"kernel_ms": round(kernel_ms, 4),
            "tokens_per_s": round(M / (kernel_ms * 1e-3), 1),
            "Gelem/s": round(M * Di * N / (kernel_ms * 1e-3) / 1e9, 1),
            "gemm_TFLOP": round(gemm_flops / 1e12, 3),
            "note": f"batch {w.batch}, L {w.L}, Dm {Dm}, Di {Di}, N {N}, R {R}, conv {w.conv_k}; "
                    f"in_proj, conv1d+SiLU, x_proj (hi+lo), fused scan (dt_proj on MFMA, D x, "
                    f"SiLU(z) gate), out_proj (hi+lo)"}


def time_conv(torch, mssm, steps=20, warmup=3, batch=16, L=2048, D=5120, k=4):
    """The causal depthwise conv1d + SiLU alone on float32 [batch, L, D]: HBM-bound,
    4 bytes read and 4 written per element."""
    u = [torch.randn((batch, L, D), device="cuda") for _ in range(2)]
    w = torch.randn((D, k), device="cuda") * 0.5
    b = torch.randn((D,), device="cuda") * 0.1
    out = torch.empty((batch, L, D), device="cuda")
    for i in range(warmup):
        mssm.mssm_causal_conv1d_silu(u[i % 2], w, b, out)
    stream = torch.cuda.current_stream()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for i in range(steps):
        mssm.mssm_causal_conv1d_silu(u[i % 2], w, b, out)
    e_ev.record(stream)
    torch.cuda.synchronize()
    kernel_ms = s_ev.elapsed_time(e_ev) / steps
    nb = 8 * batch * L * D + 4 * D * (k + 1)
    del u, w, b, out
    torch.cuda.empty_cache()
    gbs = nb / (kernel_ms * 1e-3) / 1e9
    return {"kernel_ms": round(kernel_ms, 4), "GB/s": round(gbs, 1),
            "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "bytes_per_launch": nb},
            "note": f"conv1d_silu_kernel, float32 [{batch}, {L}, {D}], width {k}, bias; "
                    f"2 rotated inputs"}


def time_backward(name, steps, warmup, torch, mssm, workloads, parts=True):
    """The scan's backward pass (forward and reverse chunk summaries, recompute,
    partial sums) with feedthrough, gate and initial state."""
    w = workloads.workload(name)
    g = workloads.generate(name)
    d = device_inputs(g, torch)
    e = workloads.generate_extras(w)
    opt = {k: _to_device(e[k], torch) for k in ("Dskip", "z", "h0")} if parts else {}
    del g, e
    dout = torch.randn((w.batch, w.L, w.D), device="cuda")
    opts = dict(device="cuda", dtype=torch.float32)
    grads = {"dx": torch.empty((w.batch, w.L, w.D), **opts),
             "ddelta": torch.empty((w.batch, w.L, w.D), **opts),
             "dA": torch.empty((w.D, w.N), **opts), "dB": torch.empty((w.batch, w.L, w.N), **opts),
             "dC": torch.empty((w.batch, w.L, w.N), **opts)}
    if parts:
        grads.update(dD=torch.empty((w.D,), **opts), dz=torch.empty((w.batch, w.L, w.D), **opts),
                     dh0=torch.empty((w.batch, w.D, w.N), **opts))
    nb = mssm.mssm_selective_scan_bwd_workspace_size(w.batch, w.L, w.D, w.N, d["x"].dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def step():
        mssm.mssm_selective_scan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], dout, grads, ws,
                                     Dskip=opt.get("Dskip"), z=opt.get("z"), h0=opt.get("h0"))

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for _ in range(steps):
        step()
    e_ev.record(stream)
    torch.cuda.synchronize()
    kernel_ms = s_ev.elapsed_time(e_ev) / steps
    del d, opt, dout, grads, ws
    torch.cuda.empty_cache()
    return {"kernel_ms": round(kernel_ms, 4),
            "Gelem/s": round(elements(w) / (kernel_ms * 1e-3) / 1e9, 1),
            "note": "backward of the scan with Dskip, z gate and h0; at this shape the single-"
                    "pass order: a forward pass storing the state after every 16-step tile, "
                    "one reverse kernel recomputing each tile from its checkpoint, and the "
                    "fixed-order partial-sum reductions"}


def time_train_pair(name, steps, warmup, torch, mssm, workloads):
    """One training pair on the workload with feedthrough, gate and initial
    state: forward then backward, timed (a) as mssm_selective_scan_fwd_ex +
    mssm_selective_scan_bwd (the backward recomputes its checkpoints and the
    pre-gate output) and (b) as mssm_selective_scan_fwd_save +
    mssm_selective_scan_bwd_saved (the forward saves them)."""
    w = workloads.workload(name)
    g = workloads.generate(name)
    d = device_inputs(g, torch)
    e = workloads.generate_extras(w)
    opt = {k: _to_device(e[k], torch) for k in ("Dskip", "z", "h0")}
    del g, e
    dout = torch.randn((w.batch, w.L, w.D), device="cuda")
    opts = dict(device="cuda", dtype=torch.float32)
    y = torch.empty((w.batch, w.L, w.D), **opts)
    grads = {"dx": torch.empty((w.batch, w.L, w.D), **opts),
             "ddelta": torch.empty((w.batch, w.L, w.D), **opts),
             "dA": torch.empty((w.D, w.N), **opts), "dB": torch.empty((w.batch, w.L, w.N), **opts),
             "dC": torch.empty((w.batch, w.L, w.N), **opts), "dD": torch.empty((w.D,), **opts),
             "dz": torch.empty((w.batch, w.L, w.D), **opts),
             "dh0": torch.empty((w.batch, w.D, w.N), **opts)}
    nb = mssm.mssm_selective_scan_bwd_workspace_size(w.batch, w.L, w.D, w.N, d["x"].dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    nf = mssm.mssm_selective_scan_workspace_size(w.batch, w.L, w.D, w.N, d["x"].dtype)
    wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device="cuda")
    ns = mssm.mssm_selective_scan_saved_size(w.batch, w.L, w.D, w.N, True)
    saved = torch.empty(ns, dtype=torch.uint8, device="cuda")
    args = (d["x"], d["delta"], d["A"], d["B"], d["C"])

    def recompute():
        mssm.mssm_selective_scan_fwd_ex(*args, y, wsf, **opt)
        mssm.mssm_selective_scan_bwd(*args, dout, grads, ws, **opt)

    def with_saved():
        mssm.mssm_selective_scan_fwd_save(*args, y, saved, **opt)
        mssm.mssm_selective_scan_bwd_saved(*args, saved, dout, grads, ws, **opt)

    def timed(fn):
        for _ in range(warmup):
            fn()
        stream = torch.cuda.current_stream()
        s_ev = torch.cuda.Event(enable_timing=True)
        e_ev = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s_ev.record(stream)
        for _ in range(steps):
            fn()
        e_ev.record(stream)
        torch.cuda.synchronize()
        return s_ev.elapsed_time(e_ev) / steps

    ms_re = timed(recompute)
    ms_saved = timed(with_saved)
    fwd_save_ms = timed(lambda: mssm.mssm_selective_scan_fwd_save(*args, y, saved, **opt))
    del d, opt, dout, grads, ws, wsf, saved, y
    torch.cuda.empty_cache()
    return {"recompute_ms": round(ms_re, 4), "saved_ms": round(ms_saved, 4),
            "fwd_save_ms": round(fwd_save_ms, 4),
            "Gelem/s (saved)": round(elements(w) / (ms_saved * 1e-3) / 1e9, 1),
            "note": "forward + backward with Dskip, z gate and h0; saved: the forward also "
                    "writes the state after every 16-step tile and the output before the "
                    "gate, which the backward reads instead of recomputing"}


def cpu_baseline(name, workloads, oracle, threads):
    """The float64 oracle on the host cores, on the whole headline workload."""
    g = workloads.generate(name)
    w = g["workload"]
    x = workloads.to_float64(g["x"])
    dl = workloads.to_float64(g["delta"])
    A = g["A"].astype("float64")
    B = workloads.to_float64(g["B"])
    C = workloads.to_float64(g["C"])
    oracle.selective_scan(x[:, :64], dl[:, :64], A, B[:, :64], C[:, :64], nthreads=threads)
    # repeat whole passes until about 10 s of wall time (bounded to 1000 passes)
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.selective_scan(x, dl, A, B, C, nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 1000:
            break
    return {"value": round(algorithmic_bytes(w) * passes / dt / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{passes} pass(es) over the whole {name} workload "
                      f"({w.batch}x{w.L}x{w.D}x{w.N}), float64, {threads} threads over "
                      f"independent (batch, channel) chains"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    choices=["fused_proj_bf16", "scan_ex", "decode_step_bf16", "conv1d_silu_fp32",
                             "mamba_block_bf16", "backward", "train_pair"],
                    help="time only this extra workload and print its record (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) and exit; "
                         "used to scale rocprofv3 FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the scan does not shard across GPUs in this build "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch

    import workloads
    from selective_state_space_54_amd import mssm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "bytes_written": n * 4}))
        return 0
    mssm.load()
    if args.only:
        if args.only == "fused_proj_bf16":
            wo, _, kms = time_fused(args.only, args.steps, args.warmup, torch, mssm, workloads)
            rec = {"kernel_ms": round(kms, 4)}
        elif args.only == "scan_ex":
            rec = time_scan_ex(HEADLINE, args.steps, args.warmup, torch, mssm, workloads)
        elif args.only == "decode_step_bf16":
            rec = time_decode(args.only, args.steps, args.warmup, torch, mssm, workloads)
        elif args.only == "conv1d_silu_fp32":
            rec = time_conv(torch, mssm, steps=args.steps, warmup=args.warmup)
        elif args.only == "backward":
            rec = time_backward(HEADLINE, args.steps, args.warmup, torch, mssm, workloads)
        elif args.only == "train_pair":
            rec = time_train_pair(HEADLINE, args.steps, args.warmup, torch, mssm, workloads)
        else:
            rec = time_block(args.only, args.steps, args.warmup, torch, mssm, workloads)
        print(json.dumps({"only": args.only, **rec}), flush=True)
        return 0

    w, wall, kernel_ms = time_workload(args.workload, args.steps, args.warmup, 2, torch, mssm,
                                       workloads)
    nb = algorithmic_bytes(w)
    gbs = nb * args.steps / wall / 1e9
    elem_rate = elements(w) / (kernel_ms * 1e-3) / 1e9
    line = {
        "metric": "selective-scan GB/s achieved (% of HBM peak) and B·L·D tokens-channels/sec",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "L": w.L, "D": w.D, "N": w.N,
                   "storage": w.dtype, "parallelism": "single GPU"},
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_channels_per_s": round(w.batch * w.L * w.D * args.steps / wall, 1),
        "roofline": {
            "bound": "alu",
            "kernel": "chain_scan_kernel (the whole scan call is this one kernel)",
            "achieved": round(elem_rate, 1),
            "peak": round(ELEM_PEAK_GPS, 1),
            "unit": "Gelem/s",
            "frac": round(elem_rate / ELEM_PEAK_GPS, 4),
            "kernel_ms": round(kernel_ms, 4),
            "hbm_GBps_at_kernel_time": round(nb / (kernel_ms * 1e-3) / 1e9, 1),
            "traffic": load_traffic(w.name),
        },
    }
    if not args.headline_only:
        others = {}

        def extra(name, fn):
            """Measure one further workload; a failure is recorded in the line
            (with its message) instead of losing the headline record."""
            try:
                others[name] = fn()
            except Exception as e:   # noqa: BLE001 - reported, not hidden
                others[name] = {"error": f"{type(e).__name__}: {e}"[:300]}

        def config_record(name):
            if workloads.workload(name).fused:
                wo, wall_o, kms_o = time_fused(name, 5, 2, torch, mssm, workloads)
            else:
                wo, wall_o, kms_o = time_workload(name, 5, 2, 1, torch, mssm, workloads)
            nbo = algorithmic_bytes(wo)
            rec = {
                "ms_per_step": round(wall_o * 1e3 / 5, 4),
                "kernel_ms": round(kms_o, 4),
                "GB/s": round(nbo / (kms_o * 1e-3) / 1e9, 1),
                "hbm_peak_frac": round(nbo / (kms_o * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tokens_channels_per_s": round(wo.batch * wo.L * wo.D / (kms_o * 1e-3), 1),
                "Gelem/s": round(elements(wo) / (kms_o * 1e-3) / 1e9, 1),
                "alu_frac": round(elements(wo) / (kms_o * 1e-3) / 1e9 / ELEM_PEAK_GPS, 4),
            }
            if wo.fused:
                flops = 2 * wo.batch * wo.L * (wo.D * (wo.R + 2 * wo.N) + wo.R * wo.D)
                rec["projection_TFLOPs"] = round(flops / 1e12, 2)
                rec["note"] = ("bytes by the scan formula (x + Delta + y, B + C); Delta, B, "
                               "C are formed on chip from x and the weights")
            return rec

        for name in OTHERS:
            if name != w.name:
                extra(name, lambda name=name: config_record(name))
        extra("mamba130m_layer_fp32 zoh+skip+gate+state",
              lambda: time_scan_ex(HEADLINE, 10, 2, torch, mssm, workloads))
        extra("decode_step_bf16",
              lambda: time_decode("decode_step_bf16", 200, 10, torch, mssm, workloads))
        extra("conv1d_silu_fp32", lambda: time_conv(torch, mssm))
        extra("mamba_block_bf16",
              lambda: time_block("mamba_block_bf16", 5, 2, torch, mssm, workloads))
        extra("backward mamba130m_layer_fp32",
              lambda: time_backward(HEADLINE, 5, 2, torch, mssm, workloads))
        extra("forward + backward mamba130m_layer_fp32",
              lambda: time_train_pair(HEADLINE, 5, 2, torch, mssm, workloads))
        line["workloads"] = others
    if not args.no_cpu_baseline:
        import oracle
        threads = min(os.cpu_count() or 1, 16)
        line["cpu_baseline"] = cpu_baseline(w.name, workloads, oracle, threads)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
