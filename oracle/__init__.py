"""Oracle for the Mamba selective scan -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation, in float64, of what the
GPU library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``selective_state_space_54_amd``) never imports it,
and this package never imports the product path: the two share no code.

Sources, cited by page title and section:

* "Understanding Mamba" (james-library-blog): the continuous model, section 2.1
  eq. (1); zero-order-hold discretisation, section 2.2 eq. (2); the discrete
  recurrence, section 2.3 eq. (3); the convolution view, section 3.1 eq. (5);
  selection, section 5.1 eq. (6); the combine operator, section 7.1 eq. (8);
  the Mamba block, section 8.1 eq. (9).
* "State Space Models and Mamba" (aicomputerinstitute, grade-12 chapter): the
  scalar selective recurrence with the first-order input term and its traced
  examples.
* "Selective State Space Models" (aiwiki): the batched tensor shapes and the
  statement that the first-order input term Delta*B is what Mamba uses.
* "Mathematical Prerequisites for Mamba" (prathamp.com): the leaky-bucket
  closed form, zero-order hold (section 5), the unrolled sum (section 6) and the
  1-semiseparable matrix (section 7).
* "Mamba and Selective State Spaces" (quantmemo): worked example 1.

Modules:
    scan       -- the sequential recurrence (C core, fp64) and its Python wrapper
    selection  -- softplus, SiLU, the fused x_proj/dt_proj projections
    forms      -- independent closed forms used as pins: combine operator and
                  tree scans, unrolled sum, semiseparable matrix, convolution
    block      -- the Mamba block around the scan: causal depthwise conv1d,
                  SiLU, projections, gate (eq. (9))
    backward   -- gradients of the scan (adjoint recurrence, float64)
Parity status of each function is stated in its docstring; every function is
pinned by a ``-m "not gpu"`` test unless it says "parity unpinned".
"""
from .scan import selective_scan, selective_scan_step, load_library, build_library  # noqa: F401
from .selection import softplus, silu, selective_ssm_fused, round_to_bf16  # noqa: F401
from . import forms  # noqa: F401
from . import block  # noqa: F401
from . import backward  # noqa: F401
