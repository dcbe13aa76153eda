"""CPU oracle for the block-diffusion denoising-step hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The HIP library never calls it and shares no code, header, table or
constant generator with it: the two are independent implementations of the same
definitions, and the tests compare them.

Everything here is plain numpy in float64 unless a definition fixes another
precision (the acceptance rule's float32 running sum, the 24-bit uniforms).  Each
function names the passage it follows.  The pages are:

* "srswti/axe-diffusion-ksl-xe" (model card of a 26B-A4B block-diffusion LM):
  sections "what the model is", "the kernels we built", "requirements".
* "Block-diffusion generation (DiffusionGemma)" (mlxcel documentation):
  sections "How it works", "Samplers", "CLI flags", "Reproducibility".

Modules
-------
philox   Philox4x32-10 counter-based generator (Salmon et al., SC'11).
moe      uint4 dequantisation, top-k routing, GeGLU expert FFN, fixed-order combine.
layer    the RMS norm before the FFN and the router projection that feeds the top-k.
loop     the denoising-loop driver: canvas length, random initial canvas, stability update.
sampler  per-position entropy and top-1 probability, temperature-0 argmax, two-level
         gumbel-max token, entropy-bound and confidence-threshold acceptance.

Pins: every function is checked in ``tests/test_oracle_*.py`` against closed forms,
brute force, library routines or published known-answer values.  None is
"parity unpinned".
"""

from . import philox, moe, layer, loop, sampler  # noqa: F401
