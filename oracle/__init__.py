"""CPU oracle of the Mamba-2 mixer-core prefill (fp64, plain and slow).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__
and the bench's CPU-baseline leg may import this package.  It shares no
code with the HIP library (mamba_ssd_selective_amd) and never imports it.

  recurrence  -- token-by-token definition: conv + SiLU, selective-state
                 recurrence, grouped gated RMSNorm, varlen batch driver.
  chunked     -- closed-form chunked evaluation (exponent checks, clamp) and
                 the materialised quadratic form, used to pin the recurrence.
  inproj      -- the packed in-projection row (z | xBC | dt), the step size
                 softplus(dt + bias), and mixed decode + prefill batches.
  precision   -- the definitions run with one narrower rounding inserted (the
                 conv output, the per-chunk entry state, a bf16 product), to
                 measure the error budget behind the library's fp32 choices.

Every function is pinned by a CPU test (tests/test_oracle_pins.py) against a
closed form, an invariant, a library routine or a hand-derived fixture.
"""
from . import recurrence, chunked, inproj, precision  # noqa: F401
