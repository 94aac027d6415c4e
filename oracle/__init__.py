"""CPU oracle for the SVDQuant-style W4A4 linear and its AWQ W4A16 sibling.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

What it follows
---------------
The method is the one the "Nunchaku Lite" pages (Hugging Face Diffusers
quantization docs) describe:

* "Supported quantization types" table: ``svdq_w4a4`` with precision ``int4``
  and group size 64, or precision ``nvfp4`` and group size 16, each "with SVDQ
  low-rank correction"; ``awq_w4a16`` with ``int4`` weights, group size 64.
* "NunchakuLiteQuantizationConfig" section: ``rank`` 32 in the example,
  ``compute_dtype`` bfloat16 for every floating-point buffer.
* The news article "Memangkas VRAM Model Diffusi ... Lewat Nunchaku Lite",
  section on what happens when a diffusion model is quantized: outliers are
  moved into a 16-bit low-rank branch while the rest runs with 4-bit weights
  and activations.

The pages give names and group sizes only; every numeric step below is a
stated *reading* (scale = amax/7, E4M3 block scales with one fp32 weight
tensor scale, smoothing by sqrt(amax_x/amax_w), low-rank split by SVD of the
smoothed weight, fp64 accumulation).  Each function's docstring names the
reading it implements.

Modules
-------
formats   bit-level encoders/decoders: bf16, OCP E4M3, OCP E2M1, nibble packing
quant     group quantizers (int4 symmetric, nvfp4, AWQ uint4)
layers    weight preparation, reference quantized linears, int partial sums

Pins (tests/test_oracle_*.py) tie these functions to brute force, closed forms,
library casts (torch bfloat16 / float8_e4m3fn) and linear-algebra identities.
"""

from . import formats, quant, layers  # noqa: F401
