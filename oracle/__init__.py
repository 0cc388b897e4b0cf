"""CPU oracle for the SVDQuant W4A4 + low-rank linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import anything from this package.
The product (the HIP library and its Python binding) never imports it and
never falls back to it.  It shares no code with the HIP path.

What it computes, step by step in the order and notation of the pages
(SVDQuant notes page, hoonably.github.io/blog/svdquant; "Nunchaku 4-bit
diffusion inference in Diffusers" page; SVDQuant abstract, arXiv 2411.05007):

* formats.py   -- rounding to bf16 / fp16 / fp32 and the E2M1, E8M0 and E4M3
                  number formats (format definitions; the FP4 maximum of 6 is
                  the q_max of the notes page, section 3).
* quant.py     -- the max-scaled symmetric quantizer of section 3 applied per
                  group along K (MXFP4: groups of 32 with a power-of-two scale;
                  INT4: groups of 64 with an fp16 scale; NVFP4-style: groups of
                  16 with an E4M3 scale and a float32 tensor scale, the
                  Blackwell format the Nunchaku in Diffusers page names),
                  dequantization and the canonical two-codes-per-byte packing.
* decompose.py -- offline calibration: per-input-channel smoothing factors,
                  the smoothed weight, its truncated SVD (section 4.2,
                  W_hat = L1 L2 + R with L1 = U Sigma_r, L2 = V_r^T), the 16-bit
                  factors and the residual R.
* qkv.py       -- the fused QKV step's Q/K RMS normalization and rotary
                  embedding on the layer output (the Nunchaku in Diffusers
                  page, section "Quantizing your own model").
* w4a16.py     -- the 4-bit weight x 16-bit activation linear of the second
                  kernel family (AWQ) on the Nunchaku in Diffusers page.
* layer.py     -- the layer output of section 4.2:
                  X W = X_hat W_hat ~ X_hat L1 L2 + Q(X_hat) Q(R), plus bias and
                  an optional GELU, in float64; the error measure and bound of
                  section 4.1; the parity comparison.

Floating point is float64 except where the layer fixes a narrower type (the
fp32 smoothing divide, the fp32 quantizer arithmetic, the bf16/fp16 stored
operands).  Precision-dependent decisions that pick an integer (a code, a
scale exponent) are taken in float32, the precision the quantizer is defined
in.  Every readings of a point the pages leave open is listed in the module
that takes it.

Parity status of each function is stated in its docstring ("pinned by ...");
the GPU accumulation order and the bf16 rounding inside the GPU's low-rank
branch are parity unpinned beyond the stated output tolerance.
"""
from . import formats, quant, decompose, layer  # noqa: F401
