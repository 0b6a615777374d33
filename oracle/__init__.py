"""CPU oracle for the SVDQuant W4A4 linear layer (test infrastructure only).

This package is the slow, plain, obviously-correct reference that the HIP
path is checked against.  It is NOT part of the product: only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may import it.  The
product library never calls it and shares no code with it.

Sources (the pages are news/tutorial prose about Nunchaku / SVDQuant in
Diffusers; they fix the method in words, not formulas):

* "Bringing Nunchaku 4-bit Diffusion Inference to Diffusers" (aiphreaks.com),
  section "Technical Breakdown and Performance Metrics": SVDQuant is W4A4,
  activation outliers move into a 16-bit low-rank branch, the remainder is
  quantized to 4 bits; NVFP4 and INT4 precisions.
* "Nunchaku Lite: 4-Bit Diffusion-Inferenz direkt in Diffusers"
  (chaosnode.de), section "Die Technik: SVDQuant": outliers are moved from the
  activations into the weights, the hard part becomes a 16-bit low-rank
  branch, the rest is quantized to 4 bits; section "Hardware-Support":
  schemes svdq_w4a4 (NVFP4 | INT4) and awq_w4a16 (INT4).
* "Nunchaku 4-Bit Diffusion Inference in Diffusers: A Practical Guide"
  (imaginepro.ai), section "Under the Hood": the low-rank term captures the
  outlier structure and runs in higher precision, the 4-bit term carries the
  bulk of the compute.
* Hugging Face / watch-ia.com announcement (French page): checkpoints are
  named "nvfp4_r32", i.e. rank 32.

Where the pages leave a step open (rounding, scale format, group size, the
smoothing exponent), the oracle takes the plainest reading; every such reading
is listed in the design notes.

Modules
-------
formats : fp32 / bf16 / E4M3 / E2M1 rounding, from the format definitions.
svdq    : smoothing, truncated SVD, residual, INT4 group quantizer, forward.
nvfp4   : FP4-E2M1 / E4M3 block-16 variant of the quantizer and forward.
awq     : asymmetric INT4 weight-only (W4A16) quantizer and forward.
"""

from . import formats, svdq, nvfp4, awq  # noqa: F401
