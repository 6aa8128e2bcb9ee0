"""CPU oracle for the NVFP4 W4A4 MoE expert GEMM with residual activation
compensation, the trainer-side weight QDQ and the rollout-guided rounding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``precision_gemm_nvfp4_amd``) and imports nothing from it.

Everything here is plain numpy, written to be checked by eye against the pages:

* "QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE via
  QUantization-error Alignment across Dual Sides" (gist.science technical
  summary, English and Chinese/Portuguese versions; yfxerp.com digest), and
* "TRACE: Rollout-Guided Quantization-Aware Training for FP4 Reinforcement
  Learning of MoE Language Models" (paper.rainbus.top summary).

Numerical rule of the oracle: every stored fp32/bf16/E4M3/E2M1 value is the
correctly rounded (round-to-nearest-even) result of an exact real expression of
stored inputs.  Every rounding decision is taken by an exact comparison in
float64, where each product involved has at most 31 significant bits and is
therefore exact.  Sums whose order matters (residual channel scores) run in one
fixed, documented order.  Reference GEMM results are accumulated in float64.

Modules:
  formats  -- E2M1 (FP4) and E4M3 codebooks and exact nearest rounding.
  nvfp4    -- global/block scales, quantize, dequantize, residual, channel
              scores, top-k selection, residual requantization (compact, and
              the dense binary-mask form), weight QDQ, rollout-guided
              rounding.
  gemm     -- compensated W4A4 GEMM (compact and dense-mask correction) and
              the MoE FFN layer stages.
  mxfp4    -- the MXFP4 variant (32-element blocks, E8M0 power-of-two
              scales): quantize, dequantize, residual selection and
              requantization, compensated GEMM, weight QDQ and guided
              rounding; MXFP8 activations and the W4A8 GEMM.

Every function states which passage of the pages it follows.  Functions with
no independent pin say "parity unpinned" (none at present).
"""

from . import formats, nvfp4, gemm, mxfp4  # noqa: F401
