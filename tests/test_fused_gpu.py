"""GPU parity of the fused selective SSM (x_proj, dt_proj + bias + softplus,
scan) through the C ABI against the float64 oracle on the same bf16 inputs.
The GPU keeps dt_low to about 16 significant bits (a bf16 hi + lo pair on the
matrix cores); the oracle keeps it in float64."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_support import ORACLE_THREADS, assert_parity, dev, host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_54_amd import mssm  # noqa: E402


def fused_inputs_device(g):
    return {k: dev(g[k]) for k in ("x", "W_x", "W_dt", "dt_bias", "A")}


def run_fused(g):
    t = fused_inputs_device(g)
    y = mssm.selective_ssm_fused(t["x"], t["W_x"], t["W_dt"], t["dt_bias"], t["A"])
    torch.cuda.synchronize()
    return host64(y)


def oracle_fused(g, channels=None):
    w = g["workload"]
    x = workloads.to_float64(g["x"])
    delta, B, C = oracle.selection.fused_projections(
        x, workloads.to_float64(g["W_x"]), workloads.to_float64(g["W_dt"]),
        g["dt_bias"].astype(np.float64), R=w.R, N=w.N)
    A = g["A"].astype(np.float64)
    if channels is not None:
        x, delta, A = x[:, :, channels], delta[:, :, channels], A[channels]
    return oracle.selective_scan(x, delta, A, B, C, nthreads=ORACLE_THREADS)


SHAPES = [  # batch, L, D, N, R
    (1, 1, 64, 16, 16), (1, 31, 64, 16, 32), (2, 33, 100, 16, 16), (1, 100, 130, 4, 48),
    (2, 300, 257, 16, 160), (1, 257, 512, 8, 160), (3, 129, 96, 16, 64),
    # x_proj over whole 64-wide k tiles with 192 columns: 15 and 30 tiles (the
    # copy-to-LDS form's unrolled period, once and twice), 5 tiles (period
    # remainder only), ragged rows
    (1, 100, 960, 16, 160), (3, 70, 1920, 16, 160), (2, 61, 320, 16, 160),
]


@pytest.mark.parametrize("chunk_len", [None, 40, 64], indirect=True)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_small_shapes(shape, chunk_len):
    batch, L, D, N, R = shape
    print(f"case fused {shape} chunk={chunk_len}", flush=True)
    g = workloads.generate("fused_proj_bf16", batch=batch, L=L, D=D, N=N, R=R, seed=900 + L + D)
    assert_parity(run_fused(g), oracle_fused(g), "bf16", f"fused {shape}")


CHAIN_SHAPES = [  # batch, L, D, N = 16, R from 16 to 256: one step, ragged tails
    (1, 1, 16, 16, 16), (2, 17, 32, 16, 48), (1, 100, 64, 16, 64), (2, 33, 48, 16, 128),
    (1, 257, 96, 16, 160), (2, 64, 32, 16, 208), (1, 31, 128, 16, 256),
]


@pytest.mark.parametrize("design", ["chain"], indirect=True)
@pytest.mark.parametrize("shape", CHAIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_single_pass_shapes(shape, design):
    """The single pass (delta from the dt_proj + softplus kernel) at small sizes."""
    batch, L, D, N, R = shape
    print(f"case fused single pass {shape}", flush=True)
    g = workloads.generate("fused_proj_bf16", batch=batch, L=L, D=D, N=N, R=R, seed=950 + L + R)
    assert_parity(run_fused(g), oracle_fused(g), "bf16", f"fused single pass {shape}")


SPLIT_SHAPES = [  # batch, L, D, N = 16, R: batch * D >= 32768 channels, D % 64 == 0
    (1, 1, 32768, 16, 16), (1, 33, 32768, 16, 32), (2, 17, 16384, 16, 160), (4, 41, 8192, 16, 64),
]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_split_state_shapes(shape):
    """The single pass with the state split over a block's wavefronts (chosen
    from 32768 channels on): one step, ragged 8-step tiles, several batch rows."""
    batch, L, D, N, R = shape
    print(f"case fused split {shape}", flush=True)
    g = workloads.generate("fused_proj_bf16", batch=batch, L=L, D=D, N=N, R=R, seed=970 + L + R)
    assert_parity(run_fused(g), oracle_fused(g), "bf16", f"fused split {shape}")


@pytest.mark.parametrize("cpl", ["1", "2"])
def test_fused_both_chain_per_lane_variants(cpl):
    with mssm.tuning(chains_per_lane=int(cpl)):
        g = workloads.generate("fused_proj_bf16", batch=2, L=200, D=320, N=16, R=160, seed=31)
        y = run_fused(g)
    assert_parity(y, oracle_fused(g), "bf16", f"fused cpl={cpl}")


@pytest.mark.parametrize("design", ["auto", "chain"], indirect=True)
def test_fused_zero_dt_proj_matches_plain_scan_on_gpu(design):
    """W_dt = 0: Delta = softplus(bias) for every token; the fused result must
    equal the plain scan run on that Delta and on B, C taken from x @ W_x."""
    g = workloads.generate("fused_proj_bf16", batch=2, L=150, D=128, N=16, R=32, seed=41)
    g["W_dt"] = np.zeros_like(g["W_dt"])
    y = run_fused(g)
    assert_parity(y, oracle_fused(g), "bf16", "fused with W_dt = 0")


@pytest.mark.parametrize("design", ["auto", "chunked"], indirect=True)
def test_fused_full_size_workload_every_output(design):
    """batch 16, L 2048, D 5120, N 16, R 160: every output against the oracle;
    by default this shape takes the single-pass scan over a written-out delta,
    pinned "chunked" the chunked kernels with delta on the matrix cores."""
    print(f"case fused_proj_bf16 full size design={design}", flush=True)
    g = workloads.generate("fused_proj_bf16")
    y = run_fused(g)
    r = assert_parity(y, oracle_fused(g), "bf16", "fused_proj_bf16")
    print("fused_proj_bf16", r, flush=True)


def test_fused_rejects_float32():
    g = workloads.generate("fused_proj_bf16", batch=1, L=8, D=64, N=16, R=16)
    t = fused_inputs_device(g)
    with pytest.raises(mssm.MssmError) as e:
        mssm.selective_ssm_fused(t["x"].float(), t["W_x"].float(), t["W_dt"].float(),
                                 t["dt_bias"], t["A"])
    assert e.value.status == 2
