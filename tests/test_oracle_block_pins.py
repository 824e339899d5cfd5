"""Pins for the block oracle (oracle/block.py): the causal depthwise
convolution against numpy's convolution routine and its impulse response, the
block's single-token closed form, its causality, and the gate branch."""
import numpy as np
import pytest

import oracle
from oracle import block as blk


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 7])
def test_conv_equals_numpy_convolution(k):
    """np.convolve(u, taps reversed) truncated to L is the causal filter in which
    tap k-1 weighs the current token (the listing's left padding by k-1 zeros)."""
    rng = _rng(k)
    u = rng.standard_normal((2, 23, 5))
    w = rng.standard_normal((5, k))
    b = rng.standard_normal(5)
    out = blk.causal_conv1d(u, w, b)
    for bb in range(2):
        for d in range(5):
            ref = np.convolve(u[bb, :, d], w[d, ::-1])[:23] + b[d]
            np.testing.assert_allclose(out[bb, :, d], ref, rtol=1e-13, atol=1e-13)


def test_conv_impulse_response_reads_the_taps_backwards():
    w = np.array([[0.5, -2.0, 3.0, 7.0]])
    u = np.zeros((1, 6, 1))
    u[0, 1, 0] = 1.0                      # impulse at t = 1
    out = blk.causal_conv1d(u, w)[0, :, 0]
    np.testing.assert_array_equal(out, [0.0, 7.0, 3.0, -2.0, 0.5, 0.0])


def _block_inputs(seed, batch=2, L=9, Dm=6, Di=8, N=4, R=3, k=4, conv_bias=True):
    rng = _rng(seed)
    return dict(
        u0=rng.standard_normal((batch, L, Dm)),
        W_in=rng.standard_normal((Dm, 2 * Di)) / np.sqrt(Dm),
        conv_w=rng.standard_normal((Di, k)) / np.sqrt(k),
        conv_b=0.3 * rng.standard_normal(Di) if conv_bias else None,
        W_x=rng.standard_normal((Di, R + 2 * N)) / np.sqrt(Di),
        W_dt=rng.standard_normal((R, Di)) / np.sqrt(R),
        dt_bias=np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), Di)))),
        A=-np.broadcast_to(np.arange(1.0, N + 1), (Di, N)).copy(),
        Dskip=rng.standard_normal(Di),
        W_out=rng.standard_normal((Di, Dm)) / np.sqrt(Di),
    ), R


def test_single_token_closed_form():
    """L = 1 from h = 0: h = Delta B x, so y = (Delta sum_n B_n C_n + D) x, and
    the block is out = (y SiLU(z)) W_out with x = SiLU(w[:, k-1] u + b) (only the
    current-token tap sees a nonzero input) and [u | z] = u0 W_in."""
    p, R = _block_inputs(3, L=1)
    out = blk.mamba_block(**p, R=R, gemm_inputs_bf16=False)
    Di = p["W_in"].shape[1] // 2
    N = p["A"].shape[1]
    uz = np.einsum("blm,mj->blj", p["u0"], p["W_in"])
    u, z = uz[..., :Di], uz[..., Di:]
    pre = u * p["conv_w"][:, -1] + p["conv_b"]
    x = pre / (1.0 + np.exp(-pre))
    proj = np.einsum("bld,dj->blj", x, p["W_x"])
    dt_pre = np.einsum("blr,rd->bld", proj[..., :R], p["W_dt"]) + p["dt_bias"]
    delta = np.logaddexp(0.0, dt_pre)
    bc = np.sum(proj[..., R:R + N] * proj[..., R + N:], axis=-1, keepdims=True)
    y = (delta * bc + p["Dskip"]) * x
    gate = z / (1.0 + np.exp(-z))
    ref = np.einsum("bld,dm->blm", y * gate, p["W_out"])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_block_is_causal():
    p, R = _block_inputs(5, L=12)
    out = blk.mamba_block(**p, R=R, gemm_inputs_bf16=False)
    q = dict(p)
    q["u0"] = p["u0"].copy()
    q["u0"][:, 7:] += 1.0
    out2 = blk.mamba_block(**q, R=R, gemm_inputs_bf16=False)
    np.testing.assert_array_equal(out[:, :7], out2[:, :7])
    assert np.all(np.abs(out[:, 7] - out2[:, 7]) > 0)


def test_zero_gate_branch_silences_the_block():
    """z = 0 (gate columns of W_in zero) -> SiLU(0) = 0 -> out = 0, while the
    SSM branch is active (a bias on the conv keeps x away from zero)."""
    p, R = _block_inputs(7)
    Di = p["W_in"].shape[1] // 2
    p["W_in"] = p["W_in"].copy()
    p["W_in"][:, Di:] = 0.0
    out, parts = blk.mamba_block(**p, R=R, gemm_inputs_bf16=False, return_parts=True)
    assert np.all(out == 0.0)
    assert np.abs(parts["x"]).max() > 0.01


def test_feedthrough_only_closed_form_over_many_tokens():
    """B = 0 (its x_proj columns zero): the state stays 0, so the SSM output is
    D x and the block is out = (D x SiLU(z)) W_out for every token, with x the
    SiLU of the causal filter (computed here with numpy's convolution)."""
    p, R = _block_inputs(9, L=15)
    N = p["A"].shape[1]
    p["W_x"] = p["W_x"].copy()
    p["W_x"][:, R:R + N] = 0.0
    out = blk.mamba_block(**p, R=R, gemm_inputs_bf16=False)
    Di = p["W_in"].shape[1] // 2
    uz = np.einsum("blm,mj->blj", p["u0"], p["W_in"])
    u, z = uz[..., :Di], uz[..., Di:]
    conv = np.empty_like(u)
    for b in range(u.shape[0]):
        for d in range(Di):
            conv[b, :, d] = np.convolve(u[b, :, d], p["conv_w"][d, ::-1])[:u.shape[1]]
    pre = conv + p["conv_b"]
    x = pre / (1.0 + np.exp(-pre))
    ref = np.einsum("bld,dm->blm", p["Dskip"] * x * (z / (1.0 + np.exp(-z))), p["W_out"])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_rounding_points_only_touch_the_gemm_inputs():
    p, R = _block_inputs(11)
    exact, pe = blk.mamba_block(**p, R=R, gemm_inputs_bf16=False, return_parts=True)
    rounded, pr = blk.mamba_block(**p, R=R, gemm_inputs_bf16=True, return_parts=True)
    np.testing.assert_array_equal(pe["x"], pr["x"])        # the scan input is not rounded
    assert not np.array_equal(pe["B"], pr["B"])             # x_proj read the bf16 copy
    np.testing.assert_allclose(rounded, exact, rtol=0, atol=2e-2 * np.abs(exact).max())
