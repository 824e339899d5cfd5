#!/usr/bin/env python3
"""Selective-scan benchmark on one MI355X; prints ONE JSON line.

A step is one full pass of the hot path (discretise, recurrence, read-out,
store; for the fused workload also the selection projections) over one batch
of the workload, inputs already in HBM.  The headline workload is the largest
single-GPU configuration, the long-sequence bfloat16 scan (batch 1, L 131072,
D 2560, N 16): with 2560 channels it takes the chunked order (chunk summaries,
carries, output).  The other synthetic workloads are measured the same way and
reported under "workloads"; every scan workload rotates two input sets so no
step finds its inputs in the 256 MB last-level cache left by the step before.

value    = algorithmic bytes per step * steps / wall time of the timed region
           (bytes = (x + delta + y) over batch*L*D plus (B + C) over batch*L*N,
           input element size for all five, as the metric defines them)
roofline = the scan call against the roof that binds it.  Each (b, t, d, n)
           element needs 4 fp32 VALU operations (exponent multiply, input-term
           multiply, state fma, read-out fma) and one v_exp_f32.  MI355X's
           published fp32 vector peak, 157.3 TFLOP/s, is 256 CU * 128 fma
           lanes * 2.4 GHz = 78.64e12 fma lane-operations/s; a transcendental
           issues at a quarter of that rate, so an element costs 4 + 4 = 8
           lane-operation slots and the element roof is 9830.4 Gelem/s
           ("alu").  (The issue-rate probes measure what the chip sustains
           against it.)  The same call is also reported against HBM
           (algorithmic bytes / call time vs 8 TB/s and vs a device copy
           measured in the same run), with the HBM bytes the rocprofv3 counters
           measured for the current kernel sources ("traffic").  Call time
           comes from HIP events recorded on the stream the kernels run on.
cpu_baseline = the float64 oracle on the host cores: passes over the headline
           workload for about 10 s, plus one oracle pass per workload (and one
           on a single thread for the two smallest), with the core count and
           CPU model.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_FMA_LANE_OPS_PER_S = 256 * 128 * 2.4e9   # 157.3 TFLOP/s / 2 flops per fma
SLOTS_PER_ELEMENT = 4 + 4                     # 4 single-rate VALU + one quarter-rate exp
ELEM_PEAK_GPS = FP32_FMA_LANE_OPS_PER_S / SLOTS_PER_ELEMENT / 1e9
# probe reports: a wave64 instruction issued every 4 clocks on each of the
# 1024 SIMDs, the unit the probes express their rates in
VALU_LANE_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
MFMA_BF16_PEAK_TFLOPS = 2500.0
HEADLINE = "long_seq_bf16"
CONFIGS = ("tiny_fp32", "mamba130m_layer_fp32", "mid_bf16", "long_seq_bf16", "fused_proj_bf16")
TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "selective_state_space_54_amd", "csrc")


def algorithmic_bytes(w) -> int:
    e = 4 if w.dtype == "fp32" else 2
    return (3 * w.batch * w.L * w.D + 2 * w.batch * w.L * w.N) * e


def elements(w) -> int:
    return w.batch * w.L * w.D * w.N


def projection_flops(w) -> int:
    return 2 * w.batch * w.L * (w.D * (w.R + 2 * w.N) + w.R * w.D)


def kernel_sources_digest() -> str:
    """Hash of every kernel source: a traffic record taken on other sources is stale."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str):
    """The counter record of this workload if it was taken on the current
    kernel sources, else None."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    with open(TRAFFIC_PATH) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel_sources_sha256") != kernel_sources_digest():
        return None
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ---- rocprofv3 counter ingestion (CPU only) ----------------------------------------------

def _counter_rows(directory):
    import csv
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    return rows


def _per_kernel(directory, counter):
    """{kernel name: (dispatches, total counter value)} for one counter."""
    out = {}
    for r in _counter_rows(directory):
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "")
        n, v = out.get(name, (0, 0.0))
        disp = r.get("Dispatch_Id")
        out[name] = (n, v + float(r["Counter_Value"]))
        out.setdefault("__dispatches__", {}).setdefault(name, set()).add(disp)
    disp = out.pop("__dispatches__", {})
    return {k: (len(disp.get(k, ())), v) for k, (_, v) in out.items()}


def ingest_counters(args):
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs of `--only-config WORKLOAD`
    and of `--calibrate-copy MIB` into the workload's traffic record."""
    copy_bytes = args.calibrate_mib * (1 << 20)
    scales = {}
    for counter, d in (("FETCH_SIZE", args.copy_fetch_dir), ("WRITE_SIZE", args.copy_write_dir)):
        per = _per_kernel(d, counter)
        # the copy kernel is the dispatch with the largest count per launch
        best = max(v / n for n, v in per.values() if n)
        scales[counter] = copy_bytes / (best * 1024.0)
    fetch = _per_kernel(args.fetch_dir, "FETCH_SIZE")
    write = _per_kernel(args.write_dir, "WRITE_SIZE")
    kernels = {}
    read_b = write_b = 0.0
    for name in sorted(set(fetch) | set(write)):
        if "mssm" not in name:
            continue
        nf, vf = fetch.get(name, (0, 0.0))
        nw, vw = write.get(name, (0, 0.0))
        rb = vf * 1024.0 * scales["FETCH_SIZE"] / args.calls
        wb = vw * 1024.0 * scales["WRITE_SIZE"] / args.calls
        kernels[name] = {"dispatches_per_call": round(max(nf, nw) / args.calls, 3),
                         "fetch_KiB_per_dispatch": round(vf / max(nf, 1), 1),
                         "write_KiB_per_dispatch": round(vw / max(nw, 1), 1),
                         "read_bytes_per_call": int(rb), "write_bytes_per_call": int(wb)}
        read_b += rb
        write_b += wb
    db = {}
    if os.path.exists(TRAFFIC_PATH):
        with open(TRAFFIC_PATH) as f:
            db = json.load(f)
    db[args.workload] = {
        "kernel_sources_sha256": kernel_sources_digest(),
        "hbm_bytes_per_step": int(read_b + write_b),
        "read_bytes": int(read_b), "write_bytes": int(write_b),
        "fetch_scale": round(scales["FETCH_SIZE"], 4),
        "write_scale": round(scales["WRITE_SIZE"], 4),
        "calls": args.calls, "kernels": kernels,
        "summary": args.summary,
    }
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(db[args.workload], indent=1))
    return 0


# ---- GPU timing -----------------------------------------------------------------------------

def _to_dev_array(a, torch):
    import numpy as np
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
        else torch.from_numpy(a)
    return t.cuda()


def measure_copy_bandwidth(torch, mib=1024, reps=10):
    """GB/s (bytes read + bytes written) of a plain device-to-device copy."""
    n = mib * (1 << 20) // 4
    src = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    dst = torch.empty_like(src[0])
    for i in range(3):
        dst.copy_(src[i % 2])
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for i in range(reps):
        dst.copy_(src[i % 2])
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def _timed(fn, steps, warmup, torch):
    """Warm up, then time `steps` calls: one event pair around the region on the
    stream the library launches on (launches queue back to back, so this is
    call time plus the gaps between calls), and the host wall clock."""
    for i in range(warmup):
        fn(i)
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


def time_scan(name, steps, warmup, rotate, torch, mssm, workloads, keep_host=False):
    """The plain scan (mssm_selective_scan_fwd_ws) on `rotate` input sets drawn
    with seeds seed + 1000 r, used in turn.  Returns (workload, wall s, call ms,
    host arrays of set 0 when keep_host)."""
    w = workloads.workload(name)
    sets, host0 = [], None
    for r in range(rotate):
        g = workloads.generate(name, seed=w.seed + 1000 * r)
        d = {k: _to_dev_array(g[k], torch) for k in ("x", "delta", "A", "B", "C")}
        d["y"] = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")
        sets.append(d)
        if r == 0 and keep_host:
            host0 = g
        del g
    nbytes = mssm.mssm_selective_scan_workspace_size(w.batch, w.L, w.D, w.N, sets[0]["x"].dtype)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    # validated once; each step issues the C call directly
    calls = [mssm.prepare_selective_scan_fwd_ws(d["x"], d["delta"], d["A"], d["B"], d["C"],
                                                d["y"], ws) for d in sets]
    wall, call_ms = _timed(lambda i: calls[i % rotate](), steps, warmup, torch)
    del sets, ws, calls
    torch.cuda.empty_cache()
    return w, wall, call_ms, host0


def time_fused(name, steps, warmup, rotate, torch, mssm, workloads, keep_host=False):
    """The fused selective SSM per step (W_x transpose, x_proj GEMM with the
    dt_low split in its epilogue, W_dt transpose, the Delta kernel and the
    single-pass scan at this shape) on `rotate` input sets used in turn."""
    w = workloads.workload(name)
    sets, host0 = [], None
    for r in range(rotate):
        g = workloads.generate(name, seed=w.seed + 1000 * r)
        sets.append({k: _to_dev_array(g[k], torch) for k in ("x", "W_x", "W_dt", "dt_bias", "A")})
        if r == 0 and keep_host:
            host0 = g
        del g
    y = torch.empty(sets[0]["x"].shape, dtype=torch.float32, device="cuda")
    nb = mssm.mssm_selective_ssm_fused_workspace_size(w.batch, w.L, w.D, w.N, w.R, torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def step(i):
        d = sets[i % rotate]
        mssm.mssm_selective_ssm_fused_fwd(d["x"], d["W_x"], d["W_dt"], d["dt_bias"], d["A"], y, ws)

    wall, call_ms = _timed(step, steps, warmup, torch)
    del sets, y, ws
    torch.cuda.empty_cache()
    return w, wall, call_ms, host0


def config_record(w, wall, call_ms, steps, rotate, copy_gbs):
    """Throughput and roofline figures of one workload."""
    nb = algorithmic_bytes(w)
    gbs_call = nb / (call_ms * 1e-3) / 1e9
    elem_rate = elements(w) / (call_ms * 1e-3) / 1e9
    tr = load_traffic(w.name)
    rec = {
        "steps": steps, "input_sets_rotated": rotate,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "kernel_ms": round(call_ms, 4),
        "GB/s": round(nb * steps / wall / 1e9, 2),
        "tokens_channels_per_s": round(w.batch * w.L * w.D / (call_ms * 1e-3), 1),
        "roofline": {
            "bound": "alu", "achieved": round(elem_rate, 1), "peak": round(ELEM_PEAK_GPS, 1),
            "unit": "Gelem/s", "frac": round(elem_rate / ELEM_PEAK_GPS, 4),
            "traffic": tr["hbm_bytes_per_step"] if tr else None,
            "hbm": {"achieved": round(gbs_call, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs_call / HBM_PEAK_GBS, 4),
                    "measured_copy_GBps": round(copy_gbs, 1),
                    "frac_of_measured_copy": round(gbs_call / copy_gbs, 4),
                    "algorithmic_bytes": nb,
                    "traffic_over_algorithmic": (round(tr["hbm_bytes_per_step"] / nb, 3)
                                                 if tr else None)},
        },
    }
    if w.fused:
        fl = projection_flops(w)
        rec["roofline"]["projection_mfma"] = {
            "flops": fl, "achieved_TFLOPs_over_call": round(fl / (call_ms * 1e-3) / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        rec["note"] = ("bytes by the scan formula (x + Delta + y, B + C); Delta, B, C are formed "
                       "from x and the weights inside the call")
    return rec


def device_inputs(g, torch):
    return {k: _to_dev_array(g[k], torch) for k in ("x", "delta", "A", "B", "C")}


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


def probe_rates(torch, iters=4000, blocks=2048, reps=5):
    """Issue rates of the VALU instructions the scan is made of, the scan's
    per-element sequence as a whole, and plain read and copy bandwidth, from
    the probes in libmssm_probe.so (built next to libmssm.so)."""
    import ctypes
    from selective_state_space_54_amd import build as hb
    lib = ctypes.CDLL(hb.PROBE_LIB_PATH)
    lib.mssm_probe_launch.restype = ctypes.c_int
    lib.mssm_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    out = torch.empty(4096 * 256, dtype=torch.float32, device="cuda")
    bc = torch.linspace(-1.0, 1.0, 32, device="cuda", dtype=torch.float32)
    n16 = (2 << 30) // 16
    buf = torch.ones(n16 * 4, dtype=torch.int32, device="cuda")

    def timed(which, nblk, it, arg=None, n=0):
        def go():
            rc = lib.mssm_probe_launch(which, nblk, it, ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(arg) if arg else None, n, sh)
            if rc != 0:
                raise RuntimeError(f"probe {which} launch failed: {rc}")
        go()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record(stream)
        for _ in range(reps):
            go()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e-3

    res = {"published_fp32_fma_lane_ops_per_s": FP32_FMA_LANE_OPS_PER_S,
           "wave_issue_lane_slots_per_s": VALU_LANE_SLOTS_PER_S, "blocks": blocks,
           "threads_per_block": 256, "iterations": iters}
    lanes = blocks * 256
    for which, name in ((0, "v_exp_f32"), (1, "v_fma_f32"), (2, "v_mul_f32"),
                        (3, "v_mul_f32 with DPP row_newbcast operand")):
        t = timed(which, blocks, iters)
        rate = lanes * iters * 16 / t
        res[name] = {"lane_instructions_per_s": rate,
                     "frac_of_published_fp32_lane_rate": round(rate / FP32_FMA_LANE_OPS_PER_S, 4),
                     "lane_slots_per_instruction": round(VALU_LANE_SLOTS_PER_S / rate, 3),
                     "seconds": t}
    t = timed(4, blocks, iters, bc.data_ptr())
    rate = lanes * iters * 16 / t
    res["scan element (mul, v_exp_f32, mul, fma, fma)"] = {
        "Gelem_per_s": round(rate / 1e9, 1),
        "frac_of_element_roof": round(rate / 1e9 / ELEM_PEAK_GPS, 4),
        "lane_slots_per_element": round(VALU_LANE_SLOTS_PER_S / rate, 3), "seconds": t}
    t = timed(5, 4096, 0, buf.data_ptr(), n16)
    res["read_GBps"] = round(n16 * 16 / t / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    res["copy_GBps (read + write)"] = round(measure_copy_bandwidth(torch), 1)
    return res


def _oracle_pass(g, oracle, workloads, threads):
    """One float64 oracle pass over the workload's inputs (the fused workload:
    its projections, then the scan); returns the seconds it took."""
    import numpy as np
    w = g["workload"]
    f64 = workloads.to_float64
    t0 = time.perf_counter()
    if w.fused:
        oracle.selective_ssm_fused(f64(g["x"]), f64(g["W_x"]), f64(g["W_dt"]),
                                   g["dt_bias"].astype(np.float64), g["A"].astype(np.float64),
                                   R=w.R, nthreads=threads)
    else:
        oracle.selective_scan(f64(g["x"]), f64(g["delta"]), g["A"].astype(np.float64),
                              f64(g["B"]), f64(g["C"]), nthreads=threads)
    return time.perf_counter() - t0


def cpu_baseline(hosts, oracle, workloads, threads, seconds=10.0):
    """The oracle on the host: whole passes over the headline workload until
    about `seconds` have passed (at least one), one pass over every other
    workload, and single-thread passes over the two smallest."""
    import numpy as np  # noqa: F401
    g = hosts[HEADLINE]
    w = g["workload"]
    passes, spent = 0, 0.0
    while passes == 0 or spent < seconds:
        spent += _oracle_pass(g, oracle, workloads, threads)
        passes += 1
        if passes >= 100:
            break
    per = {}
    for name, gg in hosts.items():
        if name == HEADLINE:
            per[name] = {"threads": threads, "seconds_per_pass": round(spent / passes, 3)}
            continue
        ww = gg["workload"]
        s = _oracle_pass(gg, oracle, workloads, threads)
        per[name] = {"threads": threads, "seconds_per_pass": round(s, 6),
                     "GB/s": round(algorithmic_bytes(ww) / s / 1e9, 4)}
        if name in ("tiny_fp32", "mamba130m_layer_fp32"):
            s1 = _oracle_pass(gg, oracle, workloads, 1)
            per[name]["one_thread"] = {"seconds_per_pass": round(s1, 6),
                                       "GB/s": round(algorithmic_bytes(ww) / s1 / 1e9, 4)}
    return {"value": round(algorithmic_bytes(w) * passes / spent / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle", "seconds": round(spent, 3),
            "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{passes} whole pass(es) over {HEADLINE} ({w.batch}x{w.L}x{w.D}x{w.N}), "
                      f"float64, {threads} threads over independent (batch, channel) chains",
            "per_workload": per}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-config", default=None, choices=list(CONFIGS),
                    help="time only this workload (two rotated input sets) and print its "
                         "record; used for profiling")
    ap.add_argument("--only", default=None,
                    choices=["scan_ex", "decode_step_bf16", "conv1d_silu_fp32",
                             "mamba_block_bf16", "backward", "train_pair"],
                    help="time only this extra workload and print its record (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) and exit; "
                         "used to scale rocprofv3 FETCH_SIZE/WRITE_SIZE counters")
    ap.add_argument("--probe-rates", action="store_true",
                    help="only run the VALU issue-rate and bandwidth probes and print them")
    ap.add_argument("--ingest-counters", action="store_true",
                    help="(CPU only) turn rocprofv3 counter runs into profiles/traffic.json: "
                         "needs --workload, --calls, --fetch-dir, --write-dir, --copy-fetch-dir, "
                         "--copy-write-dir, --calibrate-mib, --summary")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--calls", type=int, default=0)
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    ap.add_argument("--calibrate-mib", type=int, default=1024)
    ap.add_argument("--summary", default="")
    args = ap.parse_args(argv)
    if args.ingest_counters:
        if not (args.workload and args.calls > 0 and args.fetch_dir and args.write_dir
                and args.copy_fetch_dir and args.copy_write_dir):
            ap.error("--ingest-counters needs --workload, --calls and the four run directories")
        return ingest_counters(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs each call on a single GPU and "
              f"does not shard across GPUs (asked for --gpus {args.gpus}).", file=sys.stderr)
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
    if args.probe_rates:
        print(json.dumps({"probe_rates": probe_rates(torch)}), flush=True)
        return 0
    mssm.load()
    if args.only:
        HL = "mamba130m_layer_fp32"
        if args.only == "scan_ex":
            rec = time_scan_ex(HL, args.steps, args.warmup, torch, mssm, workloads)
        elif args.only == "decode_step_bf16":
            rec = time_decode(args.only, args.steps, args.warmup, torch, mssm, workloads)
        elif args.only == "conv1d_silu_fp32":
            rec = time_conv(torch, mssm, steps=args.steps, warmup=args.warmup)
        elif args.only == "backward":
            rec = time_backward(HL, args.steps, args.warmup, torch, mssm, workloads)
        elif args.only == "train_pair":
            rec = time_train_pair(HL, args.steps, args.warmup, torch, mssm, workloads)
        else:
            rec = time_block(args.only, args.steps, args.warmup, torch, mssm, workloads)
        print(json.dumps({"only": args.only, **rec}), flush=True)
        return 0

    copy_gbs = measure_copy_bandwidth(torch)
    timer = lambda name, keep: (time_fused if workloads.workload(name).fused else time_scan)(
        name, args.steps, args.warmup, 2, torch, mssm, workloads, keep_host=keep)
    if args.only_config:
        w, wall, call_ms, _ = timer(args.only_config, False)
        print(json.dumps({"only_config": w.name,
                          **config_record(w, wall, call_ms, args.steps, 2, copy_gbs)}), flush=True)
        return 0

    want_cpu = not args.no_cpu_baseline
    hosts = {}
    w, wall, call_ms, h0 = timer(HEADLINE, want_cpu)
    if want_cpu:
        hosts[HEADLINE] = h0
    head = config_record(w, wall, call_ms, args.steps, 2, copy_gbs)
    nb = algorithmic_bytes(w)
    gbs = nb * args.steps / wall / 1e9
    roof = dict(head["roofline"])
    roof["kernel"] = ("one scan call: chunk_summary_kernel, chunk_carry_kernel, "
                      "chunk_output_kernel launched back to back (2560 channels: the chunked "
                      "order)")
    roof["kernel_ms"] = head["kernel_ms"]
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
                   "storage": w.dtype, "parallelism": "single GPU",
                   "input_sets_rotated": 2},
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "measured_copy_GBps": round(copy_gbs, 1),
        "tokens_channels_per_s": round(w.batch * w.L * w.D * args.steps / wall, 1),
        "roofline": roof,
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

        def scan_config(name):
            wo, wall_o, ms_o, g0 = timer(name, want_cpu)
            if want_cpu:
                hosts[name] = g0
            return config_record(wo, wall_o, ms_o, args.steps, 2, copy_gbs)

        for name in CONFIGS:
            if name != HEADLINE:
                extra(name, lambda name=name: scan_config(name))
        HL = "mamba130m_layer_fp32"
        extra("mamba130m_layer_fp32 zoh+skip+gate+state",
              lambda: time_scan_ex(HL, 10, 2, torch, mssm, workloads))
        extra("decode_step_bf16",
              lambda: time_decode("decode_step_bf16", 200, 10, torch, mssm, workloads))
        extra("conv1d_silu_fp32", lambda: time_conv(torch, mssm))
        extra("mamba_block_bf16",
              lambda: time_block("mamba_block_bf16", 5, 2, torch, mssm, workloads))
        extra("backward mamba130m_layer_fp32",
              lambda: time_backward(HL, 5, 2, torch, mssm, workloads))
        extra("forward + backward mamba130m_layer_fp32",
              lambda: time_train_pair(HL, 5, 2, torch, mssm, workloads))
        line["workloads"] = others
    if want_cpu:
        import oracle
        threads = min(os.cpu_count() or 1, 16)
        line["cpu_baseline"] = cpu_baseline(hosts, oracle, workloads, threads)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
