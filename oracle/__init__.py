"""CPU oracle for the MXFP4-weight / FP8-activation routed MoE FFN.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct CPU
statement of what the GPU path computes. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product package
(``mxfp4_weights_fp8_amd``) never imports, calls or links anything here, and this
package shares no code, tables or helpers with the HIP kernels.

What the path computes is fixed by the sources as follows (citations name the
page and its section):

* "Pushing the Limits of Serving DeepSeek-V4-Pro" (LMSYS blog; both the news
  summary and the numbered translation carry it): MXFP4 expert weights with FP8
  activations quantized online (§2.2 "Capacity"), W13 and W2 expert GEMMs tuned
  separately on routed shapes (§3.3), SwiGLU fused with the quantization that
  produces W2's FP8 data and scales (§4.3), a top-k reduction plus a shared-expert
  add (§3.2), MoE-TP slices of the intermediate dimension (§3.1).
* "Optimization progress report" (DeepSeek-V4-Flash on GB10): tokens packed by
  expert ahead of the MoE launch with the token-to-expert mapping unchanged
  (Optimization 14); the 4-bit weights are consumed as stored, no re-quantization
  (Optimization 05).

The element formats themselves (E2M1, E8M0, E4M3FN) are those of the OCP
Microscaling v1.0 and OCP 8-bit floating point specifications, which the pages
name only as "MXFP4" and "FP8"; ``formats.py`` writes their definitions out.

Modules:
  formats  -- exact decode tables, round-to-nearest-even E4M3 encoding, the
              power-of-two (E8M0) scale rule for activation blocks.
  moe      -- plan_ref, quant_act_ref, ffn_ref (fp64, exact dequantization).
  brute    -- an independent per-token, per-expert loop version with its own
              codecs (fractions / brute-force nearest search, math.fsum), used only
              to pin ``moe`` on tiny inputs.
  compare  -- the parity metrics and the SwiGLU-code comparison rule.

Parity status of each function is stated in its docstring; every function here
is pinned by a ``-m "not gpu"`` test (tests/test_oracle_*.py).
"""

from . import formats, moe, compare  # noqa: F401
from .moe import plan_ref, quant_act_ref, ffn_ref  # noqa: F401
