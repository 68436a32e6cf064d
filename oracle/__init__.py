"""CPU oracle for the fused Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables or constants with the HIP library and never imports it.

It is a plain, slow definition of what the layer computes, written from the
pages on "Mixture-of-Experts kernel engineering on Amazon SageMaker AI":

* a token activates only a few experts chosen by a router, each expert is a
  feed-forward network, and the layer combines the chosen experts' outputs
  (toolboxkart.tech page, section "Why MoE inference needs specialized
  kernels"; kongchang.com page, section "Why MoE Inference Is So Sensitive to
  Kernel Engineering");
* the fused kernel does scaling, the matrix multiplications and the expert
  aggregation in one pass, which changes where data lives but not the result
  (aib.vote page, third paragraph);
* weights may be FP8 E4M3, four exponent and three mantissa bits, with a
  per-tensor scale (kongchang.com page, FP8 explainer under "Triton Backend
  Routing"; aib.vote page, third paragraph).

Arithmetic is float64 unless a step turns a float into an integer (an FP8
code); there both sides decide in float32, the precision of the device.

Modules:
    fp8    -- OCP E4M3 ("fn") and E5M2 decode tables and encoders, the
              per-tensor and per-row quantisers, bfloat16
              round-to-nearest-even.
    moe    -- router (top-k), align (stable counting sort padded to a block
              size), the sparse layer (bf16, or FP8 with per-tensor or
              per-row scales), and the dense masked formulation.
    rope   -- inverse rotary position embedding of attention heads followed
              by one FP8 scale per (token, head) (the pages' attention-side
              kernel with a variable token count).
"""

from . import fp8, moe, rope  # noqa: F401
