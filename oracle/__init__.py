"""CPU oracle for the quantized linear: BFL fp8r / nvfp4, the SVDQuant W4A4 layer
(NVFP4 and INT4 variants), the weight-only 4-bit layer and the model-specific
epilogues.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library under
``precision_quantized_linear_amd/`` and does not import it.

What it computes, and the page each part follows (all pages are the Diffusers
"BFL (fp8r / nvfp4)" quantization guide unless named otherwise):

* ``formats``   E4M3 and E2M1 encode/decode (the two element formats the guide's
                intro bullets name), bf16 round-to-nearest-even.
* ``quant``     fp8r row-wise quantization and nvfp4 block quantization with the
                nibble packing and the global-scale rule (intro bullets).
* ``reference`` dequantize-then-fp64 GEMM references for both schemes, the
                SVDQuant low-rank branch ("Bringing Nunchaku 4-bit Diffusion
                Inference to Diffusers", section "Background: SVDQuant and
                Nunchaku"), the dequantize-to-compute_dtype fallback (guide,
                "Kernels" section, last paragraph) and the GEMM acceptance test.
* ``awq``       the weight-only 4-bit (awq_w4a16) format and layer (Nunchaku post,
                "Introducing Nunchaku Lite", layer list).
* ``int4``      the INT4 variant of svdq_w4a4 (same post and section).
* ``epilogue``  GELU (tanh form), the GELU MLP and the fused QKV scatter (same post,
                "Introducing Nunchaku Lite", first paragraph), with the interval
                bounds that check outputs passing through GELU and requantization.

Plain numpy throughout: float32 array arithmetic for the quantizers (every
operation IEEE binary32 round-to-nearest-even, division correctly rounded, no
fused multiply-add, no denormal flush) and float64 for the references.
Every function is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``.
"""
from . import awq, epilogue, formats, int4, quant, reference  # noqa: F401
