"""CPU oracle of the compressed-KV hot path.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the GPU path
computes: nearest-centre assignment, Lloyd fitting of the centres, the residual
codec (encode and dequantize), attention over the reconstructed history, the
low-dimensional variant and log-sum-exp merging.  The codec runs in fp32 with a
fixed operation order, because its codes are compared bit for bit; distances,
means and attention run in fp64.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP path and imports
nothing from it.

Sources (the text of five web pages on compressed KV caches for autoregressive
video generation):
* TempoKV (arxiv 2610.15324), section 3.1 Eq. 1 (affine min/max quantizer) and
  section 3.3 Eq. 2 (residual against a prediction, reconstruction = prediction
  + dequantized residual);
* QuantWM (2609.26425), section 4.1 (k-means assignment of each token to its
  nearest centre, then quantization of the residual; QSAC, the query-aware
  choice among the nearest centres, Eqs. 6-12, and its cold start in the
  appendix; section 4.2, PSAC, the compensation of the remaining key error
  along the principal query directions);
* TempoKV, section 3.3 Eqs. 2-4 and "Anchor frames" (keys predicted from their
  reconstructed history, values from the aligned reconstructed key and their
  own history, only the residual stored) and Eq. 5 (ridge calibration): tempo.py;
* NanoKV (2611.06377), Table 4 (256 centres each for K and V, two k-means
  iterations, one residual stage), Table 5 caption (centres fitted separately
  for K and V) and Figure 4 (mixed-dimensional attention: reduce the queries,
  attend in low dimension, restore the output dimension, merge by LSE).

Parity status: every function here is pinned by a test of ``tests/`` against
something other than itself (brute force, closed forms, exact rational
arithmetic, the pages' printed numbers).  Whether the method reproduces the
behaviour of the pages' own systems (QVG, NanoKV-Fast) is parity unpinned: no
page prints their formulas or their outputs for a given input.
"""
from .numerics import (  # noqa: F401
    f16_bits,
    f16_from_bits,
    fp16_round,
    round_to_bf16,
    round_to_f32,
    round_to_storage,
)
from .codec import (  # noqa: F401
    assign,
    dequant,
    encode,
    fit,
    objective,
    reconstruct,
    storage_bits_per_value,
    storage_bytes,
)
from .attention import attend, attend_lowdim, lse_merge, Segment  # noqa: F401
from .qsac import assign_qsac, query_stats  # noqa: F401
from .psac import attend_psac, psac_basis, psac_coeffs, query_moments  # noqa: F401
from . import tempo  # noqa: F401  (predictive residual coding over frames, TempoKV)
