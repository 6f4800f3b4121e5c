"""Seeded generators of K, V, Q, initial centres and projection bases.

Recipes (all draws come from ``torch.Generator`` objects seeded by ``seed_for``):

* Tiny (fp32): per tensor, 16 cluster means mu_c ~ N(0, 2^2)^d, a per-channel
  scale sigma ~ U[0.5, 4], labels ~ U{0..15}; token = sigma * (mu_label + eps),
  eps ~ N(0, 1).  K and V use independent draws.  Q ~ N(0, 1).
* Video-like (bf16): per head and tensor an AR(1) chain over latent frames,
  x_0 ~ N(0, I), x_t = rho x_{t-1} + sqrt(1 - rho^2) eps_t, for each of the
  ``frame_tokens`` spatial positions (token index t * frame_tokens + s), with
  ``n_outlier_ch`` seeded channels per (head, tensor) multiplied by
  ``outlier_gain``; the emitted values are rounded to bf16 (round to nearest
  even).  K and V are independent chains; a streaming chain continues across
  chunks.  Q ~ N(0, I) in bf16, fresh per call.
* Initial centres: Forgy, i.e. C distinct tokens of the head drawn uniformly.
* Low-dimensional basis: G ~ N(0, 1)^{d x r} in fp64, thin QR, column signs
  flipped so that diag(R) > 0, stored as fp32.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .configs import Config

TENSOR_IDS = {"k": 0, "v": 1, "q": 2}
PURPOSE_IDS = {"data": 0, "init": 1, "basis": 2, "outlier": 3, "label": 4}


def seed_for(config_seed: int, *path: int) -> int:
    """A 63-bit seed derived from the workload seed and an integer path."""
    ss = np.random.SeedSequence([int(config_seed)] + [int(p) for p in path])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the float32 values they encode."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def tiny_kv(cfg: Config, tensor: str, device="cpu"):
    """Clustered fp32 tokens [heads, hist, dim] plus their generating labels."""
    t = TENSOR_IDS[tensor]
    g = _gen(seed_for(cfg.seed, 0, t, PURPOSE_IDS["data"]), device)
    H, N, d, C = cfg.heads, cfg.hist, cfg.dim, cfg.n_centroids
    mu = 2.0 * torch.randn(H, C, d, generator=g, device=device)
    sigma = 0.5 + 3.5 * torch.rand(H, 1, d, generator=g, device=device)
    labels = torch.randint(0, C, (H, N), generator=g, device=device)
    eps = torch.randn(H, N, d, generator=g, device=device)
    x = sigma * (torch.gather(mu, 1, labels[..., None].expand(H, N, d)) + eps)
    return x.float().contiguous(), labels


class AR1Stream:
    """AR(1) frame chain for one tensor of ``heads`` heads; emits bf16 tokens."""

    def __init__(self, cfg: Config, tensor: str, heads: int | None = None, device="cpu",
                 stream_id: int = 0):
        self.cfg = cfg
        self.heads = cfg.heads if heads is None else heads
        self.device = device
        t = TENSOR_IDS[tensor]
        self.g = _gen(seed_for(cfg.seed, stream_id, t, PURPOSE_IDS["data"]), device)
        go = _gen(seed_for(cfg.seed, stream_id, t, PURPOSE_IDS["outlier"]), "cpu")
        gain = torch.ones(self.heads, 1, cfg.dim)
        for h in range(self.heads):
            ch = torch.randperm(cfg.dim, generator=go)[: cfg.n_outlier_ch]
            gain[h, 0, ch] = cfg.outlier_gain
        self.gain = gain.to(device)
        self.state = None
        self.frames = 0

    def next_frames(self, n_frames: int) -> torch.Tensor:
        """Return the next ``n_frames`` latent frames as bf16 [heads, n_frames*S, d]."""
        cfg = self.cfg
        H, S, d = self.heads, cfg.frame_tokens, cfg.dim
        rho = cfg.rho
        innov = math.sqrt(1.0 - rho * rho)
        out = torch.empty(H, n_frames, S, d, dtype=torch.bfloat16, device=self.device)
        for f in range(n_frames):
            eps = torch.randn(H, S, d, generator=self.g, device=self.device)
            if self.state is None:
                self.state = eps
            else:
                self.state = rho * self.state + innov * eps
            out[:, f] = (self.state * self.gain).to(torch.bfloat16)
            self.frames += 1
        return out.reshape(H, n_frames * S, d)

    def tokens(self, n_tokens: int) -> torch.Tensor:
        S = self.cfg.frame_tokens
        assert n_tokens % S == 0, "history must be a whole number of latent frames"
        return self.next_frames(n_tokens // S)


def queries(cfg: Config, heads: int | None = None, n_q: int | None = None, device="cpu",
            stream_id: int = 0) -> torch.Tensor:
    """Current-chunk queries ~ N(0, I): fp32 for the fp32 workload, else bf16."""
    H = cfg.heads if heads is None else heads
    n = cfg.n_q if n_q is None else n_q
    g = _gen(seed_for(cfg.seed, stream_id, TENSOR_IDS["q"], PURPOSE_IDS["data"]), device)
    q = torch.randn(H, n, cfg.dim, generator=g, device=device)
    return q.float() if cfg.dtype == "f32" else q.to(torch.bfloat16)


def forgy_init(x: torch.Tensor, n_centroids: int, seed: int) -> torch.Tensor:
    """C distinct tokens per head, drawn uniformly without replacement."""
    H, N, d = x.shape
    if n_centroids > N:
        raise ValueError("more centres than tokens")
    g = _gen(seed, "cpu")
    idx = torch.rand(H, N, generator=g).argsort(dim=1)[:, :n_centroids].to(x.device)
    return torch.gather(x, 1, idx[..., None].expand(H, n_centroids, d)).contiguous()


def one_per_label_init(x: torch.Tensor, labels: torch.Tensor, n_centroids: int) -> torch.Tensor:
    """The first token of each generating label, as initial centres (test helper)."""
    H, N, d = x.shape
    out = torch.empty(H, n_centroids, d, dtype=x.dtype, device=x.device)
    for h in range(H):
        for c in range(n_centroids):
            j = int(torch.nonzero(labels[h] == c)[0, 0])
            out[h, c] = x[h, j]
    return out


def orthonormal_basis(heads: int, dim: int, rank: int, seed: int) -> torch.Tensor:
    """Seeded orthonormal U [heads, dim, rank] (fp32), sign-fixed thin QR of a Gaussian."""
    g = _gen(seed, "cpu")
    G = torch.randn(heads, dim, rank, generator=g, dtype=torch.float64)
    Q, R = torch.linalg.qr(G, mode="reduced")
    sign = torch.sign(torch.diagonal(R, dim1=-2, dim2=-1))
    sign[sign == 0] = 1.0
    return (Q * sign[:, None, :]).float().contiguous()


def coupled_values(k: torch.Tensor, v_chain: torch.Tensor, seed: int, mix: float = 0.6) -> torch.Tensor:
    """Values that depend on the aligned key: V = mix * K M^T + sqrt(1 - mix^2) * V_chain,
    rounded to bf16, with M a seeded orthogonal d x d matrix per head and V_chain an
    independent value chain (e.g. AR1Stream(cfg, "v")).  Stands in for the
    key-to-value dependence TempoKV measures (section 3.2: the aligned key is a
    strong predictor of the value)."""
    H, N, d = k.shape
    M = orthonormal_basis(H, d, d, seed).to(k.device)
    mixed = mix * torch.bmm(k.float(), M.transpose(1, 2).contiguous()) + math.sqrt(1.0 - mix * mix) * v_chain.float()
    return mixed.to(torch.bfloat16).contiguous()
