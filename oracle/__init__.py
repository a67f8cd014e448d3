"""CPU oracle for QJL KV-cache compression (test infrastructure only).

This package is the plain, slow reference that the HIP kernels are checked
against.  It is imported only by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; the product path never calls
it and shares no code with it.

Sources (cited by page title and section):

* "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero
  Overhead" (research summary page), Abstract -- the method: a JL transform
  followed by sign-bit quantization, an asymmetric inner-product estimator
  (quantize one side, plain JL on the other) that is unbiased, and no stored
  quantization constants.
* "The Geometry of Forgetting: How Three Papers Cracked KV Cache
  Quantization" (blog), sections "The overhead nobody tells you about",
  "Random rotation, and what high dimensions do to your intuitions" and
  "QJL: one bit, zero parameters, unbiased inner products" -- the formulas:
  Gaussian S with i.i.d. N(0,1) entries, Q(x) = sign(Sx), the dequantizer
  sqrt(pi/2)/d * S^T z, unbiasedness, the variance bound, S regenerated from
  a seed, the per-block overhead arithmetic, random rotations and the
  scaled-Beta coordinate density.

* The same page, section "TurboQuant: bridging MSE and inner product, in two
  stages" -- TurboQuant_prod on keys (``oracle.turboquant``): a Lloyd-Max
  codebook for the rotated-coordinate density after a random rotation, then
  QJL on the residual.

* The same page, section "PolarQuant: skipping Cartesian altogether" -- the
  PolarQuant key encode (``oracle.polarquant``): a recursive polar transform
  of the rotated key and per-level angle codebooks.

Parity status of each function is stated in its module header.
"""

from . import polarquant, turboquant  # noqa: F401

from .qjl import (  # noqa: F401
    splitmix64_mix,
    sketch,
    sketch_bf16_bits,
    bf16_bits_to_float64,
    float64_to_bf16_bits,
    encode,
    exact_sign_fraction,
    unpack_signs,
    query_sketch,
    estimate_scores,
    dequantize,
    decode,
    exact_attention,
    ESTIMATOR_CONST,
)
from .geometry import (  # noqa: F401
    haar_rotation,
    rotated_coordinate_density,
    rotated_coordinate_cdf,
)
from .overhead import (  # noqa: F401
    effective_bits_per_number,
    overhead_fraction,
    qjl_bits_per_coordinate,
    qjl_stored_bytes,
    qjl_per_block_constants,
)
