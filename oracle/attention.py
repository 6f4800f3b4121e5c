"""Attention of the current chunk's queries over a compressed history (one head).

* attend: softmax(Q K_hat^T / sqrt(d)) V_hat over the concatenation of the
  history segments, each segment reconstructed from its own centre table and
  codes (TempoKV, section 3.3, Eq. 2 for the reconstruction; QuantWM, section 3
  for attention of the current chunk over the cache).  Also returns the
  natural-log log-sum-exp of each row so that parts of the history can be
  merged (NanoKV, Figure 4d: LSE merging).  No mask; an empty history gives
  O = 0 and LSE = -inf.
* attend_lowdim: NanoKV-Fast's mixed-dimensional read (NanoKV, Figure 4a/4d)
  with a per-head orthonormal basis: queries reduced to q' = U_K^T q, keys read
  as coefficients k' = U_K^T c^K[id] + a_hat^K, logits q'.k' / sqrt(d) with d
  the full head dimension, O' = softmax . v' with v' = U_V^T c^V[id] + a_hat^V,
  and the output dimension restored as O = U_V O'.
* lse_merge: L = logsumexp_p L_p, O = sum_p exp(L_p - L) O_p.

All arithmetic is fp64; the softmax subtracts the row maximum first.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .codec import reconstruct


@dataclass
class Segment:
    """One head's share of a contiguous run of history with one centre table."""
    k_codes: np.ndarray
    k_meta: Optional[np.ndarray]
    k_ids: np.ndarray
    k_cent: np.ndarray
    v_codes: np.ndarray
    v_meta: Optional[np.ndarray]
    v_ids: np.ndarray
    v_cent: np.ndarray
    k_bits: int
    v_bits: int
    group: int

    @property
    def n_tokens(self) -> int:
        return int(np.asarray(self.k_ids).shape[0])


def _history(segments, basis_k=None, basis_v=None):
    ks, vs = [], []
    for s in segments:
        if s.n_tokens == 0:
            continue
        ks.append(reconstruct(s.k_codes, s.k_meta, s.k_ids, s.k_cent, s.k_bits, s.group, basis_k))
        vs.append(reconstruct(s.v_codes, s.v_meta, s.v_ids, s.v_cent, s.v_bits, s.group, basis_v))
    if not ks:
        return None, None
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def _softmax_attend(q64, K, V, scale, out_dim, rows: int = 256):
    n_q = q64.shape[0]
    O = np.zeros((n_q, out_dim), dtype=np.float64)
    lse = np.full(n_q, -np.inf, dtype=np.float64)
    if K is None:
        return O, lse
    for s in range(0, n_q, rows):
        S = (q64[s:s + rows] @ K.T) * scale
        m = S.max(axis=1, keepdims=True)
        e = np.exp(S - m)
        l = e.sum(axis=1)
        O[s:s + rows] = (e @ V) / l[:, None]
        lse[s:s + rows] = m[:, 0] + np.log(l)
    return O, lse


def attend(q, segments, dim: Optional[int] = None):
    """(O [n_q, d], LSE [n_q]) in fp64 for one head."""
    q64 = np.asarray(q, dtype=np.float64)
    d = q64.shape[1] if dim is None else dim
    K, V = _history(segments)
    return _softmax_attend(q64, K, V, 1.0 / math.sqrt(d), d)


def attend_lowdim(q, basis_k, basis_v, segments):
    """(O [n_q, d], LSE [n_q]) in fp64 for one head read in low dimension."""
    q64 = np.asarray(q, dtype=np.float64)
    Uk = np.asarray(basis_k, dtype=np.float64)
    Uv = np.asarray(basis_v, dtype=np.float64)
    d = q64.shape[1]
    qr = q64 @ Uk                                   # q' = U_K^T q, row-wise
    K, V = _history(segments, Uk, Uv)               # coefficient-space keys and values
    Or, lse = _softmax_attend(qr, K, V, 1.0 / math.sqrt(d), Uv.shape[1])
    return Or @ Uv.T, lse                           # O = U_V O'


def lse_merge(outs, lses):
    """Merge P attention parts of the same queries: (O [n_q, d], L [n_q])."""
    outs = [np.asarray(o, dtype=np.float64) for o in outs]
    lses = np.stack([np.asarray(l, dtype=np.float64) for l in lses])  # [P, n_q]
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    w = np.exp(lses - msafe[None, :])               # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    L = np.where(finite, msafe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    O = np.zeros_like(outs[0])
    for p in range(len(outs)):
        coef = np.where(finite, w[p] / np.where(finite, tot, 1.0), 0.0)
        O += coef[:, None] * outs[p]
    return O, L
