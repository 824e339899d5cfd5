"""GPU: mssm_selective_scan_fwd_noalloc (chunk summaries in the library's fixed
per-GPU scratch array, no allocation in the call) against
mssm_selective_scan_fwd on the same inputs, twice in a row, the second call
with a smaller input (the array keeps the first call's contents).  The
tolerance is the oracle bar; the two calls run the same kernels with the same
chunking, so they also agree bit for bit."""
import numpy as np
import pytest

import workloads
from gpu_support import assert_parity, host64, inputs_on_device, oracle_scan

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_54_amd import mssm  # noqa: E402


def _both(g):
    t = inputs_on_device(g)
    w = g["workload"]
    y_ref = torch.empty((w.batch, w.L, w.D), dtype=torch.float32, device="cuda")
    y_new = torch.full((w.batch, w.L, w.D), float("nan"), dtype=torch.float32, device="cuda")
    mssm.mssm_selective_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], y_ref)
    mssm.mssm_selective_scan_fwd_noalloc(t["x"], t["delta"], t["A"], t["B"], t["C"], y_new)
    torch.cuda.synchronize()
    return y_ref, y_new


@pytest.mark.parametrize("kind", ["mid_bf16", "mamba130m_layer_fp32"])
def test_noalloc_matches_the_allocating_call_twice(kind):
    """Two calls in a row: a long chunked scan, then a smaller one (fewer
    chunks, fewer channels) that finds the first call's summaries in the
    array."""
    nbytes_big = mssm.mssm_selective_scan_workspace_size(2, 9000, 320, 16,
                                                         torch.bfloat16 if kind == "mid_bf16"
                                                         else torch.float32)
    assert 0 < nbytes_big <= mssm.NOALLOC_SCRATCH_BYTES
    for shape, seed in (((2, 9000, 320, 16), 61), ((1, 1500, 96, 8), 62)):
        print(f"case noalloc {kind} {shape}", flush=True)
        batch, L, D, N = shape
        g = workloads.generate(kind, batch=batch, L=L, D=D, N=N, seed=seed)
        y_ref, y_new = _both(g)
        assert torch.equal(y_new, y_ref)
        assert_parity(host64(y_new), oracle_scan(g), g["workload"].dtype, f"noalloc {shape}")


def test_noalloc_long_sequence_workload():
    """The long-sequence workload at its full size (its chunk summaries fit the
    array), then a small call."""
    print("case noalloc long_seq_bf16", flush=True)
    g = workloads.generate("long_seq_bf16")
    y_ref, y_new = _both(g)
    assert torch.equal(y_new, y_ref)
    del y_ref
    ch = np.arange(5, g["workload"].D, 64)
    y = host64(y_new)[:, :, ch]
    assert_parity(y, oracle_scan(g, channels=ch), "bf16", "noalloc long_seq_bf16")
    g = workloads.generate("mid_bf16", batch=1, L=700, D=64, N=16, seed=63)
    y_ref, y_new = _both(g)
    assert torch.equal(y_new, y_ref)


def test_noalloc_single_pass_shape_needs_no_scratch():
    g = workloads.generate("mamba130m_layer_fp32", batch=1, L=300, D=8192, N=16, seed=64)
    y_ref, y_new = _both(g)
    assert torch.equal(y_new, y_ref)


def test_noalloc_refuses_summaries_larger_than_the_array():
    with mssm.tuning(scan_order="chunked", chunk_len=64):
        need = mssm.mssm_selective_scan_workspace_size(1, 64 * 2100, 1024, 16, torch.float32)
        assert need > mssm.NOALLOC_SCRATCH_BYTES
        x = torch.zeros((1, 64 * 2100, 1024), dtype=torch.float32, device="cuda")
        A = -torch.ones((1024, 16), dtype=torch.float32, device="cuda")
        B = torch.zeros((1, 64 * 2100, 16), dtype=torch.float32, device="cuda")
        with pytest.raises(mssm.MssmError) as e:
            mssm.mssm_selective_scan_fwd_noalloc(x, x, A, B, B, torch.empty_like(x))
        assert e.value.status == mssm.MSSM_ERROR_WORKSPACE
        text = mssm.load().mssm_last_error_string().decode()
        assert "scratch" in text and str(mssm.NOALLOC_SCRATCH_BYTES) in text, text
