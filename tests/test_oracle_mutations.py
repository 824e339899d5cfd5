"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin suite against that
build in a subprocess; the suite must fail.  The unmodified source must pass.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mssm_oracle.c")

MUTATIONS = {
    "dropped_input_term": ("h[n] = Abar * h[n] + Bbar * x_t;", "h[n] = Abar * h[n];"),
    "wrong_exp_sign": ("exp(delta_t * a)", "exp(-delta_t * a)"),
    "readout_uses_B": ("y_t += j->C[s + n] * h[n];", "y_t += j->B[s + n] * h[n];"),
    "A_transposed": ("j->A[d * N + n]", "j->A[n * D + d]"),
    "readout_before_update": (
        "h[n] = Abar * h[n] + Bbar * x_t;\n            y_t += j->C[s + n] * h[n];",
        "y_t += j->C[s + n] * h[n];\n            h[n] = Abar * h[n] + Bbar * x_t;"),
    "zoh_missing_divide": ("(Abar - 1.0) / a * j->B[s + n]", "(Abar - 1.0) * j->B[s + n]"),
    "euler_missing_delta": ("            else\n                Bbar = delta_t * j->B[s + n];",
                            "            else\n                Bbar = j->B[s + n];"),
    "x_off_by_one_step": ("const double x_t = j->x[i];",
                          "const double x_t = j->x[i >= D ? i - D : i];"),
    "h0_ignored": ("h[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "BC_row_stride_D": ("const int64_t s = (b * L + t) * N;", "const int64_t s = (b * L + t) * D;"),
    "feedthrough_dropped": ("if (j->Dskip) y_t += j->Dskip[d] * x_t;", ""),
    "gate_sign": ("oracle_silu(j->z[i])", "oracle_silu(-j->z[i])"),
    "delta_uses_x": ("const double delta_t = j->delta[i];", "const double delta_t = j->x[i] * j->x[i];"),
}


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", "-pthread", str(c), "-o", str(so), "-lm"], check=True)
    return so


def _run_pins(so):
    env = dict(os.environ, MSSM_ORACLE_LIBRARY=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_unmodified_source_passes(tmp_path):
    so = _build(open(SRC).read(), tmp_path, "clean")
    assert _run_pins(so) == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation {name} no longer applies to the source"
    so = _build(src.replace(old, new, 1), tmp_path, name)
    assert _run_pins(so) != 0, f"the pins did not catch mutation {name}"


# ---- the block oracle (Python): the same idea, in-process ------------------------------

BLOCK_SRC = os.path.join(ROOT, "oracle", "block.py")

BLOCK_MUTATIONS = {
    "conv_taps_reversed": ("out += w[:, i] * padded[:, i:i + L, :]",
                           "out += w[:, k - 1 - i] * padded[:, i:i + L, :]"),
    "conv_pads_the_future": ("padded = np.concatenate([np.zeros((batch, k - 1, D)), u], axis=1)",
                             "padded = np.concatenate([u, np.zeros((batch, k - 1, D))], axis=1)"),
    "conv_bias_dropped": ("    if b is not None:\n", "    if False:\n"),
    "branches_swapped": ("u, z = proj[..., :Di], proj[..., Di:]",
                         "z, u = proj[..., :Di], proj[..., Di:]"),
    "no_silu_after_conv": ("x = silu(causal_conv1d(u, conv_w, conv_b))",
                           "x = causal_conv1d(u, conv_w, conv_b)"),
    "gate_dropped": ("Dskip=Dskip, z=z,", "Dskip=Dskip, z=None,"),
    "feedthrough_dropped": ("Dskip=Dskip, z=z,", "Dskip=None, z=z,"),
    "selection_from_u": ("fused_projections(xq,", "fused_projections(u,"),
    "scan_input_u": ("gated = selective_scan(x, delta", "gated = selective_scan(u, delta"),
}


def _load_block_variant(text):
    import importlib.util
    import types
    import oracle  # noqa: F401  (the package the relative imports resolve in)
    mod = types.ModuleType("oracle._block_variant")
    mod.__package__ = "oracle"
    mod.__file__ = BLOCK_SRC
    exec(compile(text, BLOCK_SRC, "exec"), mod.__dict__)
    return mod


def _block_pins_fail(monkeypatch, mod):
    import oracle
    import test_oracle_block_pins as pins
    monkeypatch.setattr(oracle.block, "causal_conv1d", mod.causal_conv1d)
    monkeypatch.setattr(oracle.block, "mamba_block", mod.mamba_block)
    cases = [lambda: pins.test_conv_equals_numpy_convolution(4),
             pins.test_conv_impulse_response_reads_the_taps_backwards,
             pins.test_single_token_closed_form, pins.test_block_is_causal,
             pins.test_zero_gate_branch_silences_the_block,
             pins.test_feedthrough_only_closed_form_over_many_tokens,
             pins.test_rounding_points_only_touch_the_gemm_inputs]
    failed = 0
    for case in cases:
        try:
            case()
        except Exception:   # an assertion, or a shape error from the planted mistake
            failed += 1
    return failed


def test_unmodified_block_source_passes(monkeypatch):
    mod = _load_block_variant(open(BLOCK_SRC).read())
    assert _block_pins_fail(monkeypatch, mod) == 0


@pytest.mark.parametrize("name", sorted(BLOCK_MUTATIONS))
def test_planted_block_mistake_is_caught(monkeypatch, name):
    old, new = BLOCK_MUTATIONS[name]
    text = open(BLOCK_SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    mod = _load_block_variant(text.replace(old, new))
    assert _block_pins_fail(monkeypatch, mod) > 0, f"no pin caught {name}"


# ---- the backward oracle (Python) ------------------------------------------------------

BWD_SRC = os.path.join(ROOT, "oracle", "backward.py")

BWD_MUTATIONS = {
    "adjoint_not_decayed": ("lam_next = a * lam", "lam_next = lam"),
    "dA_uses_h_t": ("out[\"dA\"] += lam * db[t][:, None] * a * hprev",
                    "out[\"dA\"] += lam * db[t][:, None] * a * hist[t + 1]"),
    "ddelta_drops_decay_term": ("+ A * a * hprev),", "),"),
    "dB_missing_delta": ("out[\"dB\"][b, t] = (db[t] * xb[t]) @ lam",
                         "out[\"dB\"][b, t] = xb[t] @ lam"),
    "gate_slope_wrong": ("s * (1.0 + v * (1.0 - s))", "s"),
    "dC_from_previous_state": ("out[\"dC\"][b, t] = g[t] @ hist[t + 1]",
                               "out[\"dC\"][b, t] = g[t] @ hist[t]"),
    "feedthrough_grad_dropped": ("out[\"dx\"][b] += g * Dk", "pass"),
}


def _bwd_pins_fail(monkeypatch, mod):
    import oracle
    import test_oracle_backward_pins as pins
    monkeypatch.setattr(oracle.backward, "selective_scan_backward", mod.selective_scan_backward)
    monkeypatch.setattr(pins, "selective_scan_backward", mod.selective_scan_backward)
    failed = 0
    cases = [lambda g=g, n=n, k=k: pins.test_gradients_match_finite_differences(g, n, k)
             for g, n, k in pins.NAMES]
    cases.append(pins.test_single_step_closed_forms)
    for case in cases:
        try:
            case()
        except Exception:
            failed += 1
    return failed


def _load_bwd_variant(text):
    import types
    mod = types.ModuleType("oracle._backward_variant")
    mod.__package__ = "oracle"
    mod.__file__ = BWD_SRC
    exec(compile(text, BWD_SRC, "exec"), mod.__dict__)
    return mod


def test_unmodified_backward_source_passes(monkeypatch):
    assert _bwd_pins_fail(monkeypatch, _load_bwd_variant(open(BWD_SRC).read())) == 0


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_planted_backward_mistake_is_caught(monkeypatch, name):
    old, new = BWD_MUTATIONS[name]
    text = open(BWD_SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    assert _bwd_pins_fail(monkeypatch, _load_bwd_variant(text.replace(old, new))) > 0, \
        f"no pin caught {name}"
