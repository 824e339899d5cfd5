"""GPU parity of the scan's optional parts (mssm_selective_scan_fwd_ex through
the C ABI) against the float64 oracle: the exact zero-order-hold input term,
the feedthrough D x, the SiLU(z) gate, an initial state h0 and the final state
h_last, across chunk boundaries, both chains-per-lane layouts, the workloads'
full sizes, and a long sequence processed in pieces."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_support import ORACLE_THREADS, TOL, assert_parity, dev, host64, inputs_on_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_54_amd import mssm  # noqa: E402


def _opts(extras, skip, gate, init):
    return {"Dskip": extras["Dskip"] if skip else None, "z": extras["z"] if gate else None,
            "h0": extras["h0"] if init else None}


def run_ex(g, opts, bbar, last=True):
    t = inputs_on_device(g)
    kw = {k: (dev(v) if v is not None else None) for k, v in opts.items()}
    out = mssm.selective_scan_ex(t["x"], t["delta"], t["A"], t["B"], t["C"], bbar=bbar,
                                 return_last_state=last, **kw)
    torch.cuda.synchronize()
    return (host64(out[0]), host64(out[1])) if last else host64(out)


def oracle_ex(g, opts, bbar, channels=None):
    x = workloads.to_float64(g["x"])
    delta = workloads.to_float64(g["delta"])
    A = g["A"].astype(np.float64)
    B = workloads.to_float64(g["B"])
    C = workloads.to_float64(g["C"])
    Dk = opts["Dskip"].astype(np.float64) if opts["Dskip"] is not None else None
    z = workloads.to_float64(opts["z"]) if opts["z"] is not None else None
    h0 = opts["h0"].astype(np.float64) if opts["h0"] is not None else None
    if channels is not None:
        x, delta, A = x[:, :, channels], delta[:, :, channels], A[channels]
        Dk = Dk[channels] if Dk is not None else None
        z = z[:, :, channels] if z is not None else None
        h0 = h0[:, channels] if h0 is not None else None
    return oracle.selective_scan(x, delta, A, B, C, bbar=bbar, Dskip=Dk, z=z, h0=h0,
                                 return_last_state=True, nthreads=ORACLE_THREADS)


def check(g, opts, bbar, what, channels=None):
    y, h = run_ex(g, opts, bbar)
    if channels is not None:
        y, h = y[:, :, channels], h[:, channels]
    y_ref, h_ref = oracle_ex(g, opts, bbar, channels)
    dtype = g["workload"].dtype
    ry = assert_parity(y, y_ref, dtype, f"{what} y")
    rh = assert_parity(h, h_ref, dtype, f"{what} h_last")
    return ry, rh


SMALL = [  # (batch, L, D, N)
    (1, 1, 1, 1), (2, 63, 5, 4), (3, 65, 100, 16), (2, 200, 300, 16), (1, 1000, 70, 32),
    (2, 129, 257, 8),
]


@pytest.mark.parametrize("chunk_len", [None, 7, 64], indirect=True)
@pytest.mark.parametrize("bbar", ["euler", "zoh"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("kind", ["mamba130m_layer_fp32", "mid_bf16"])
def test_all_parts_small_shapes(kind, shape, bbar, chunk_len):
    batch, L, D, N = shape
    print(f"case ex {kind} {shape} {bbar} chunk={chunk_len}", flush=True)
    g = workloads.generate(kind, batch=batch, L=L, D=D, N=N, seed=300 + L + D)
    extras = workloads.generate_extras(g["workload"])
    check(g, _opts(extras, True, True, True), bbar, f"{kind} {shape} {bbar}")


@pytest.mark.parametrize("init", [False, True], ids=["h0=0", "h0"])
@pytest.mark.parametrize("gate", [False, True], ids=["nogate", "gate"])
@pytest.mark.parametrize("skip", [False, True], ids=["noskip", "skip"])
@pytest.mark.parametrize("bbar", ["euler", "zoh"])
@pytest.mark.parametrize("kind", ["mamba130m_layer_fp32", "mid_bf16"])
def test_each_combination_of_parts(kind, bbar, skip, gate, init):
    print(f"case ex parts {kind} {bbar} skip={skip} gate={gate} h0={init}", flush=True)
    g = workloads.generate(kind, batch=2, L=777, D=130, N=16, seed=17)
    extras = workloads.generate_extras(g["workload"])
    check(g, _opts(extras, skip, gate, init), bbar, f"{kind} {bbar} {skip} {gate} {init}")


@pytest.mark.parametrize("cpl", ["1", "2"])
def test_both_chain_per_lane_variants(cpl):
    with mssm.tuning(chains_per_lane=int(cpl)):
        g = workloads.generate("mid_bf16", batch=2, L=900, D=320, N=16, seed=23)
        extras = workloads.generate_extras(g["workload"])
        check(g, _opts(extras, True, True, True), "zoh", f"cpl={cpl}")


def test_zoh_on_small_steps_of_the_long_sequence_workload():
    """Delta down to 1e-4: the zero-order-hold term (Abar - 1) / A is formed
    from Abar close to 1."""
    g = workloads.generate("long_seq_bf16", batch=1, L=5000, D=256, N=16, seed=29)
    extras = workloads.generate_extras(g["workload"])
    check(g, _opts(extras, False, False, False), "zoh", "long_seq zoh")


def test_sequence_in_pieces_equals_one_call():
    """h_last of one call as h0 of the next continues the sequence."""
    g = workloads.generate("mamba130m_layer_fp32", batch=2, L=1000, D=192, N=16, seed=37)
    extras = workloads.generate_extras(g["workload"])
    t = inputs_on_device(g)
    h = dev(extras["h0"])
    pieces = []
    for a, b in ((0, 300), (300, 301), (301, 301), (301, 1000)):
        sl = {k: t[k][:, a:b].contiguous() for k in ("x", "delta", "B", "C")}
        y, h = mssm.selective_scan_ex(sl["x"], sl["delta"], t["A"], sl["B"], sl["C"], h0=h,
                                      bbar="zoh", return_last_state=True)
        pieces.append(y)
    torch.cuda.synchronize()
    y = host64(torch.cat(pieces, dim=1))
    y_ref, h_ref = oracle_ex(g, _opts(extras, False, False, True), "zoh")
    assert_parity(y, y_ref, "fp32", "pieces y")
    assert_parity(host64(h), h_ref, "fp32", "pieces h_last")


def test_empty_sequence_passes_the_state_through():
    g = workloads.generate("mid_bf16", batch=2, L=4, D=64, N=8, seed=41)
    extras = workloads.generate_extras(g["workload"])
    t = inputs_on_device(g)
    x0 = t["x"][:, :0].contiguous()
    B0 = t["B"][:, :0].contiguous()
    h0 = dev(extras["h0"])
    y, h = mssm.selective_scan_ex(x0, x0, t["A"], B0, B0, h0=h0, return_last_state=True)
    _, hz = mssm.selective_scan_ex(x0, x0, t["A"], B0, B0, return_last_state=True)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 64)
    assert torch.equal(h, h0)
    assert not torch.any(hz)


def test_plain_entry_point_equals_ex_without_parts():
    g = workloads.generate("mid_bf16", batch=2, L=3000, D=256, N=16, seed=43)
    t = inputs_on_device(g)
    y1 = mssm.selective_scan(t["x"], t["delta"], t["A"], t["B"], t["C"])
    y2, _ = mssm.selective_scan_ex(t["x"], t["delta"], t["A"], t["B"], t["C"],
                                   return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("name", ["mamba130m_layer_fp32", "mid_bf16"])
def test_full_size_workloads_all_parts_sampled_channels(name):
    print(f"case ex full size {name}", flush=True)
    g = workloads.generate(name)
    extras = workloads.generate_extras(g["workload"])
    ch = np.arange(0, g["workload"].D, 10)
    ry, rh = check(g, _opts(extras, True, True, True), "zoh", f"{name} full", channels=ch)
    print(name, ry, rh, flush=True)


def test_h_last_must_be_float32_and_shaped():
    g = workloads.generate("mid_bf16", batch=1, L=8, D=64, N=16)
    t = inputs_on_device(g)
    y = torch.empty((1, 8, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        mssm.mssm_selective_scan_fwd_ex(t["x"], t["delta"], t["A"], t["B"], t["C"], y, None,
                                        h_last=torch.empty((1, 16, 64), device="cuda"))
    with pytest.raises(ValueError):
        mssm.selective_scan_ex(t["x"], t["delta"], t["A"], t["B"], t["C"], bbar="rk4")
    assert TOL["bf16"] > 0
