"""Seeded synthetic inputs for the compressed-KV hot path.

This package is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It draws random numbers and lays them out; it performs none of the
codec or attention arithmetic (no assignment, quantization, packing or softmax).

Workload shapes follow the video backbones described on the source pages:
latent frames of 1560 spatial tokens in 3-frame chunks, keys that drift smoothly
from frame to frame (TempoKV, section 1 and section 3.2: a linear probe on the
key history reaches high cosine similarity), and a few channels carrying large
outliers (TempoKV, Figure 1).
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    AR1Stream,
    bf16_bits_to_f32,
    coupled_values,
    forgy_init,
    one_per_label_init,
    orthonormal_basis,
    queries,
    seed_for,
    tiny_kv,
)
