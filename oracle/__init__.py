"""CPU oracle for the 4-bit quantized linear layer of a diffusion transformer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute this package: only the test suite, the smoke check of ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or constant generators); the only thing
both sides consume is the seeded synthetic input produced by
``bit_quantized_gemm_quantize_amd.synth``, which holds none of the method's
arithmetic.

What it computes, in plain NumPy (fp64 unless the step is defined in fp32):

* ``formats`` -- element and scale encoders: bf16 decode/RNE, FP4 E2M1 round to
  nearest even with saturation, E8M0 power-of-two exponent, FP8 E4M3FN round to
  nearest even with saturation.
* ``quant``   -- the three block quantizers (MXFP4 block-32, NVFP4-style block-16
  with a per-tensor fp32 scale, asymmetric int4 group-64) and their dequantizers.
* ``layer``   -- the linear layer: dequantized fp64 GEMM, the low-rank branch
  evaluated right to left, bias, and the per-element error bound.
* ``attention`` -- FP8 attention (NVIDIA Technical Blog summary, second
  optimization layer): MXFP8 Q, K (along head_dim) and V (along the keys), the
  blocked online softmax with P quantized to MXFP8, and per element the most that
  codes decided differently in fp32 could move the result.

Sources.  The pages define the layer's structure: the SVDQuant Guide (aifetchly),
"The Three Pillars of SVDQuant", 1. Mathematical Outlier Factorization (forward
equation Y = QuantGEMM(W, X) + L1 (L2 X)) and "Step 2: The SVDQuant Dual-Branch
Linear Layer" (low-rank branch right to left, then bias, then cast back).  The pages
only *name* FP4 E2M1 ("Quantization for the impatient", bitsandbytes backend) and
NVFP4 (NVIDIA Technical Blog summary, first optimization layer); the E2M1 value grid
and the MX scale rule follow the public OCP Microscaling Formats (MX) v1.0
specification (section 5.3 element types, section 6.3 conversion), and the E4M3
range of +-448 is the one "Quantization for the impatient" states in its stability
section.  The division-then-round order of every quantizer follows the
per-channel quantizer of the SVDQuant Guide, "Step 1: Low-Rank Outlier
Decomposition in PyTorch".

Parity status: every function here is pinned by the CPU tests
(``tests/test_oracle_*.py``) against brute force, closed forms, library casts or
exact special cases.  None is "parity unpinned".
"""

from . import formats, quant, layer, attention  # noqa: F401
