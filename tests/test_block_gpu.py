"""GPU parity of the Mamba block forward and its conv1d + SiLU prologue
(through the C ABI) against the float64 block oracle.  The GPU carries the
float32 inputs of x_proj and W_out as bf16 hi + lo pairs (about 16 significant
bits); the oracle keeps them in float64."""
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

BLOCK_KEYS = ("u0", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "dt_bias", "A", "Dskip", "W_out")


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 70, 5), (3, 200, 300), (1, 1000, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_conv1d_silu_matches_oracle(shape, dtype, k, bias):
    batch, L, D = shape
    print(f"case conv {shape} {dtype} k={k} bias={bias}", flush=True)
    g = workloads.generate("mid_bf16" if dtype == "bf16" else "mamba130m_layer_fp32",
                           batch=batch, L=L, D=D, N=4, seed=40 + L + k)
    rng = np.random.default_rng(L + D + k)
    w = (rng.standard_normal((D, k)) / np.sqrt(k)).astype(np.float32)
    b = (0.1 * rng.standard_normal(D)).astype(np.float32) if bias else None
    out = mssm.causal_conv1d_silu(dev(g["x"]), dev(w), dev(b) if bias else None)
    torch.cuda.synchronize()
    ref = oracle.silu(oracle.block.causal_conv1d(workloads.to_float64(g["x"]),
                                                 w.astype(np.float64),
                                                 None if b is None else b.astype(np.float64)))
    assert_parity(host64(out), ref, dtype, f"conv {shape} k={k}")


def run_block(g, drop=()):
    t = {k: (dev(g[k]) if k not in drop else None) for k in BLOCK_KEYS}
    out = mssm.mamba_block(*(t[k] for k in BLOCK_KEYS))
    torch.cuda.synchronize()
    return host64(out)


def oracle_block(g, drop=(), rows=None):
    w = g["workload"]
    f = workloads.to_float64
    args = {}
    for k in BLOCK_KEYS:
        v = g[k]
        args[k] = None if k in drop else (f(v) if v.dtype == np.uint16 else v.astype(np.float64))
    if rows is not None:
        args["u0"] = args["u0"][rows]
    return oracle.block.mamba_block(**args, R=w.R, nthreads=ORACLE_THREADS)


SHAPES = [  # batch, L, Dm, Di, N, R, k
    (1, 1, 32, 64, 16, 16, 4), (2, 100, 48, 96, 16, 32, 4), (2, 300, 64, 130, 8, 16, 3),
    (1, 257, 128, 256, 16, 160, 4), (3, 129, 40, 80, 4, 16, 2), (1, 65, 16, 32, 16, 16, 1),
    # x_proj's copy-to-LDS form with the hi + lo pair (192 columns, whole k
    # tiles): 15 and 30 tiles (its unrolled period once and twice), ragged rows
    (1, 65, 32, 960, 16, 160, 4), (2, 70, 32, 1920, 16, 160, 2),
]


@pytest.mark.parametrize("chunk_len", [None, 40], indirect=True)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_block_small_shapes(shape, chunk_len):
    batch, L, Dm, Di, N, R, k = shape
    print(f"case block {shape} chunk={chunk_len}", flush=True)
    g = workloads.generate_block(batch=batch, L=L, Dm=Dm, D=Di, N=N, R=R, conv_k=k,
                                 seed=700 + L + Di)
    assert_parity(run_block(g), oracle_block(g), "bf16", f"block {shape}")


CHAIN_SHAPES = [  # batch, L, Dm, Di (a multiple of 16), N = 16, R, k
    (1, 1, 32, 64, 16, 16, 4), (2, 100, 48, 96, 16, 48, 4), (1, 257, 128, 256, 16, 160, 4),
    (1, 65, 16, 32, 16, 256, 1),
]


@pytest.mark.parametrize("design", ["chain"], indirect=True)
@pytest.mark.parametrize("shape", CHAIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_block_single_pass_shapes(shape, design):
    batch, L, Dm, Di, N, R, k = shape
    print(f"case block single pass {shape}", flush=True)
    g = workloads.generate_block(batch=batch, L=L, Dm=Dm, D=Di, N=N, R=R, conv_k=k,
                                 seed=750 + L + R)
    assert_parity(run_block(g), oracle_block(g), "bf16", f"block single pass {shape}")


SPLIT_SHAPES = [  # batch, L, Dm, Di, N = 16, R, k: batch * Di >= 32768 channels
    (1, 33, 64, 32768, 16, 16, 4), (2, 17, 32, 16384, 16, 32, 2),
]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_block_split_state_shapes(shape):
    """The block's scan with the state split over a block's wavefronts
    (feedthrough, gate, the bf16 hi + lo output), ragged 8-step tiles."""
    batch, L, Dm, Di, N, R, k = shape
    print(f"case block split {shape}", flush=True)
    g = workloads.generate_block(batch=batch, L=L, Dm=Dm, D=Di, N=N, R=R, conv_k=k,
                                 seed=780 + L + R)
    assert_parity(run_block(g), oracle_block(g), "bf16", f"block split {shape}")
    drop = ("Dskip",)
    assert_parity(run_block(g, drop), oracle_block(g, drop), "bf16", f"block split {shape} no D")


@pytest.mark.parametrize("design", ["auto", "chain"], indirect=True)
@pytest.mark.parametrize("drop", [("conv_b",), ("Dskip",), ("conv_b", "Dskip")],
                         ids=lambda d: "-".join(d))
def test_block_optional_parts_absent(drop, design):
    g = workloads.generate_block(batch=2, L=150, Dm=64, D=128, N=16, R=32, seed=77)
    assert_parity(run_block(g, drop), oracle_block(g, drop), "bf16", f"block without {drop}")


def test_block_is_deterministic():
    g = workloads.generate_block(batch=2, L=300, Dm=64, D=256, N=16, R=32, seed=78)
    a, b = run_block(g), run_block(g)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("design", ["auto", "chunked"], indirect=True)
def test_block_full_size_sampled_rows(design):
    """batch 16, L 2048, Dm 2560, Di 5120, N 16, R 160, k 4: rows 0 and 15
    (batch rows are independent) against the oracle, with either scan order."""
    print(f"case mamba_block_bf16 full size design={design}", flush=True)
    g = workloads.generate_block()
    out = run_block(g)
    assert np.isfinite(out).all()
    rows = [0, 15]
    r = assert_parity(out[rows], oracle_block(g, rows=rows), "bf16", "mamba_block_bf16")
    print("mamba_block_bf16", r, flush=True)


def test_block_from_two_host_threads_on_two_streams():
    """The library shares one rocBLAS handle per device; two host threads
    calling the block at once on their own streams must each get their own
    result (the handle and its stream are held for a whole call)."""
    import threading
    gs = [workloads.generate_block(batch=2, L=200, Dm=64, D=128, N=16, R=32, seed=s)
          for s in (81, 82)]
    ts = [{k: dev(g[k]) for k in BLOCK_KEYS} for g in gs]
    refs = [mssm.mamba_block(*(t[k] for k in BLOCK_KEYS)) for t in ts]
    torch.cuda.synchronize()
    outs = [[None] * 6, [None] * 6]
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(6):
                    outs[i][r] = mssm.mamba_block(*(ts[i][k] for k in BLOCK_KEYS), stream=s)
            s.synchronize()
        except Exception as e:   # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in (0, 1)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i in (0, 1):
        for r in range(6):
            assert torch.equal(outs[i][r], refs[i]), f"thread {i} call {r}"
