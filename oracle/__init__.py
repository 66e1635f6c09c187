"""Plain, slow CPU oracle for MXFP4 block quantization and the MXFP4-weight x BF16-activation MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (``mixed_precision_moe_amd``)
never imports it, and this package never imports the product path: the two share no code.

Floating point is evaluated in float64 unless a page fixes the precision.  Each function cites the
passage it follows.  Page tags used throughout:

* [P1] prhub summary of vLLM PR #46915 (weight/scale interleave fix in the SM90 MXFP4 fused-MoE test).
* [P2] prhub report of vLLM PR #51038, "[Bugfix][Quantization] Fix MXFP4 conversion for FlashInfer
  CUTLASS" (the checkpoint-to-kernel weight conversion, the [w1; w3] -> [w3; w1] swap, bias -> bf16).
* [P3] prhub summary of vLLM PR #43557 (the E8M0 scale fix in the MXFP4 MoE CUTLASS kernel: the 0.75
  round-up rule, the tiled scale layout and the Python reference helpers).
* [DEF] definitions this library adopts where the pages name a step without spelling it out: the
  OCP Microscaling MXFP4 format (32-element blocks, E2M1 elements rounded to nearest even and
  saturating at +-6, two nibbles per byte), top-k routing over softmax(router logits), SwiGLU as
  silu(w1 half) * (w3 half), grouped GEMMs and a routing-weighted combine; the comparison tolerance
  |y - y_ref| <= 2e-2 * rms(y_ref) + 1e-3 for floating-point outputs.

Readings of points the pages leave open are stated where they are used.

Quantized-activation variants (``moe.moe_ref(act="mxfp8" | "mxfp4")``): the layer input and the
SwiGLU output are quantized per 32-element block before the two products (MXFP8 with E4M3 elements,
or MXFP4 with the weights' rule).  The E8M0 rule for E4M3 elements is a reading: the pages' round-up of
the block maximum at a significand of 1.75, minus E4M3's largest exponent (8) instead of E2M1's (2).

NVFP4 (``quant.nvfp4_quantize_ref``): the converter's non-E8M0 branch -- 16-element blocks, an E4M3
scale of global_scale * max / 6 computed in binary32, elements scaled by the dequantized stored scale
(the fix the pages record).  The element step and the block size are readings (the pages show the scale
step only).

Dense linear (``linear.linear_ref``): y = x . dequant(W)^T + b, the MXFP4-weight linear layer of the
pages' W4A16 models (a MoE layer of one expert without routing or activation function).

Parity status:  every function here is pinned by a ``-m "not gpu"`` test against something other than
itself (hand values, closed forms, brute force, textbook cases or an independent library routine),
except the two layout conventions the pages never state -- the nibble order inside a byte and the
sign kept on codes that round to zero.  Those two are "parity unpinned" with respect to the pages:
they are fixed by this library's ABI and tested only for internal consistency.
"""

from . import quant, convert, route, moe, linear  # noqa: F401
