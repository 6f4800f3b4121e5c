"""Streaming composition of the hot path: a growing compressed history.

Autoregressive video generation produces the cache one chunk of latent frames
at a time.  Each chunk is compressed as a unit with its own centre tables
(Coral-KV, section 2: per-block codebooks fitted online), kept in packed form,
and read back by on-demand reconstruction inside attention (QuantWM, Figure 9:
cache compression, packed storage and on-demand reconstruction in streaming
inference).  ``StreamingCache`` holds that history as one ``Segment`` per chunk:

    cache = StreamingCache(k_bits=2, v_bits=4, group=16)
    for k, v, q, k_init, v_init in chunks:        # all [heads, tokens, dim] on the GPU
        seg = cache.append(k, v, k_init, v_init)  # fit K and V centres, encode, keep
        out, lse = cache.attend(q)                # q over every chunk so far

Every step is a call of the C ABI (kvc_fit_assign, kvc_encode, kvc_attend);
this module only sequences them and keeps the segment list.  The K and V fits
of a chunk are independent, so they run side by side on two streams (default
priority); the current stream waits for both before the encode.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import torch

from . import Segment, attend, encode, fit_assign


class StreamingCache:
    """History of compressed chunks, one centre table per (head, tensor, chunk)."""

    def __init__(self, k_bits: int, v_bits: int, group: int, n_iter: int = 2):
        self.k_bits, self.v_bits, self.group, self.n_iter = k_bits, v_bits, group, n_iter
        self.segments: List[Segment] = []
        self._side: Optional[torch.cuda.Stream] = None

    @property
    def n_tokens(self) -> int:
        return sum(s.n_tokens for s in self.segments)

    def fit(self, k: torch.Tensor, v: torch.Tensor, k_init: torch.Tensor,
            v_init: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
        """Fit the chunk's K and V centres from the given initial tables (Lloyd,
        ``n_iter`` iterations, then the final assignment).  Returns
        (k_ids, k_cent, v_ids, v_cent); the initial tables are not modified."""
        kc, vc = k_init.clone(), v_init.clone()
        cur = torch.cuda.current_stream(k.device)
        if self._side is None:
            self._side = torch.cuda.Stream(k.device)
        self._side.wait_stream(cur)
        kid = fit_assign(k, kc, n_iter=self.n_iter)
        with torch.cuda.stream(self._side):
            vid = fit_assign(v, vc, n_iter=self.n_iter)
        vid.record_stream(cur)
        cur.wait_stream(self._side)
        return kid, kc, vid, vc

    def encode(self, k: torch.Tensor, v: torch.Tensor, kid: torch.Tensor, kc: torch.Tensor,
               vid: torch.Tensor, vc: torch.Tensor) -> Segment:
        """Encode the chunk's residuals against its fitted centres."""
        kco, kme, _ = encode(k, kc, self.k_bits, self.group, ids=kid)
        vco, vme, _ = encode(v, vc, self.v_bits, self.group, ids=vid)
        return Segment(kco, kme, kid, kc, vco, vme, vid, vc, self.k_bits, self.v_bits, self.group)

    def push(self, seg: Segment) -> Segment:
        """Append an encoded chunk to the history."""
        if self.segments and seg.k_ids.shape[0] != self.segments[0].k_ids.shape[0]:
            raise ValueError("every chunk must cover the same heads")
        self.segments.append(seg)
        return seg

    def append(self, k: torch.Tensor, v: torch.Tensor, k_init: torch.Tensor, v_init: torch.Tensor) -> Segment:
        """fit + encode + push of one chunk."""
        kid, kc, vid, vc = self.fit(k, v, k_init, v_init)
        return self.push(self.encode(k, v, kid, kc, vid, vc))

    def attend(self, q: torch.Tensor):
        """Attention of q [heads, n_q, dim] over every chunk so far: (out, lse)."""
        return attend(q, self.segments)
