"""The five synthetic workloads, named by what they are.

Every workload is a set of attention heads, each with a compressed history of
K and V tokens and a block of current-chunk queries.  Sizes are the ones the
source pages' video backbones produce: 1560 spatial tokens per latent frame and
3-frame chunks of 4680 tokens (TempoKV, section 3.1 and section 4.1; NanoKV,
Table 9 for head and layer counts).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    index: int              # position in the workload table; feeds the seed
    heads: int              # attention heads per call (layers x heads for streaming)
    dim: int                # head dimension d
    hist: int               # history tokens attended per call (at the last step for streaming)
    n_q: int                # current-chunk queries per head
    n_centroids: int        # C, centres per head per tensor
    k_bits: int
    v_bits: int
    group: int              # channel-group size g of the residual quantizer
    dtype: str              # "f32" or "bf16" storage of K, V, Q and the centres
    n_segments: int = 1     # history segments, each with its own centre table
    far: int = 0            # tokens of the far history read in low dimension
    rank: int = 0           # low dimension r of the far history (0 = none)
    layers: int = 1
    steps: int = 1          # streaming steps (one new chunk each)
    chunk: int = 0          # tokens per streaming chunk
    frame_tokens: int = 1560
    rho: float = 0.95       # AR(1) frame-to-frame correlation of K and V
    n_outlier_ch: int = 4   # outlier channels per (head, tensor)
    outlier_gain: float = 8.0
    n_iter: int = 2         # Lloyd iterations of the centre fit
    notes: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 20261203 + self.index

    @property
    def recent(self) -> int:
        return self.hist - self.far


CONFIGS: dict[str, Config] = {
    "tiny": Config(
        name="tiny", index=0, heads=1, dim=64, hist=1024, n_q=64, n_centroids=16,
        k_bits=4, v_bits=4, group=32, dtype="f32",
        notes="fp32 K/V around 16 random cluster means with per-channel scale in [0.5, 4]"),
    "self_forcing_layer": Config(
        name="self_forcing_layer", index=1, heads=12, dim=128, hist=9360, n_q=4680,
        n_centroids=256, k_bits=2, v_bits=2, group=16, dtype="bf16",
        notes="6 latent frames x 1560 tokens of history, one chunk of queries"),
    "long_history": Config(
        name="long_history", index=2, heads=12, dim=128, hist=70200, n_q=4680,
        n_centroids=256, k_bits=4, v_bits=4, group=32, dtype="bf16", n_segments=8,
        notes="45 latent frames split into 8 equal history segments"),
    "larger_backbone": Config(
        name="larger_backbone", index=3, heads=40, dim=128, hist=32760, n_q=4680,
        n_centroids=256, k_bits=2, v_bits=4, group=16, dtype="bf16",
        far=28080, rank=32,
        notes="far history (all but the last 4680 tokens) in rank-32 coefficients"),
    "streaming": Config(
        name="streaming", index=4, heads=720, dim=128, hist=46800, n_q=4680,
        n_centroids=256, k_bits=2, v_bits=4, group=16, dtype="bf16",
        layers=30, steps=10, chunk=4680,
        notes="30 layers x 24 heads; 10 steps each adding one 4680-token chunk"),
}

ORDER = ["tiny", "self_forcing_layer", "long_history", "larger_backbone", "streaming"]


def get_config(name: str) -> Config:
    return CONFIGS[name]
