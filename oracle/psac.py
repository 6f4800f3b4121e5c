"""Principal-subspace logit compensation of the remaining key error (PSAC).
TEST INFRASTRUCTURE ONLY (part of the oracle package).

What is computed, in the pages' terms (QuantWM, 2609.26425, section 4.2; the
equations are stripped from the text, so the formulas are rebuilt from its
prose):

* query_moments -- the second-moment matrix of the queries seen so far, per
  head, M = E[q q^T] (section 4.1, Eq. 6; the full matrix, not only its
  diagonal); a running mean over chunks.
* psac_basis -- the eigen-decomposition M = U Lambda U^T (Eq. 15); the r
  eigenvectors of the largest eigenvalues span the principal query subspace
  U_r (r = 8 in the page's implementation).
* psac_coeffs -- the error left after quantization, E = K - K_hat_0 (Eq. 13),
  is kept along the principal directions as C = E U_r (Eq. 16; r numbers per
  token).
* attend_psac -- the logits are corrected by the kept components (Eq. 17):
  s_ij = (q_i . k_hat_j + (U_r^T q_i) . c_j) / sqrt(d), i.e. attention on
  k_hat_j + U_r U_r^T e_j; the values are unchanged.  r = d with an orthonormal
  U gives the logits of the unquantized keys exactly; r = 0 is plain attention.
* At the cold start (no earlier queries) PSAC is inactive (appendix).

All arithmetic is fp64.  Pinned by tests/test_oracle_psac.py.
"""
from __future__ import annotations

import numpy as np

from .attention import _history
from .codec import reconstruct


def query_moments(q, m_prev=None, n_prev: int = 0):
    """M = mean over all queries seen so far of q q^T (fp64, [d, d])."""
    q64 = np.asarray(q, dtype=np.float64)
    s = q64.T @ q64
    n = q64.shape[0]
    if n_prev > 0:
        s = s + np.asarray(m_prev, dtype=np.float64) * n_prev
    return s / (n + n_prev)


def psac_basis(m, r: int):
    """The r eigenvectors of the largest eigenvalues of the symmetric M, as the
    columns of U_r [d, r] (largest first), and all eigenvalues (descending)."""
    w, v = np.linalg.eigh(np.asarray(m, dtype=np.float64))
    order = np.argsort(w)[::-1]
    return v[:, order[:r]], w[order]


def psac_coeffs(x, codes, meta, ids, cent, bits: int, group: int, u_r):
    """C = (x - x_hat_0) U_r per token ([N, r]), x_hat_0 the dequantized tokens."""
    xh = reconstruct(codes, meta, ids, cent, bits, group)
    e = np.asarray(x, dtype=np.float64) - xh
    return e @ np.asarray(u_r, dtype=np.float64)


def attend_psac(q, segments, u_r, coeffs):
    """Attention with compensated logits.  coeffs: one [n_tokens, r] array per
    segment (the stored C).  Returns (out [n_q, d], lse [n_q]) in fp64."""
    q64 = np.asarray(q, dtype=np.float64)
    n_q, d = q64.shape
    K, V = _history(segments)
    if K is None:
        return np.zeros((n_q, d)), np.full(n_q, -np.inf)
    C = np.concatenate([np.asarray(cf, dtype=np.float64) for cf, s in zip(coeffs, segments) if s.n_tokens])
    qp = q64 @ np.asarray(u_r, dtype=np.float64)             # U_r^T q, row-wise
    S = (q64 @ K.T + qp @ C.T) / np.sqrt(d)                 # q . k_hat + (U_r^T q) . c
    m = S.max(axis=1, keepdims=True)
    p = np.exp(S - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ V) / l, (m + np.log(l))[:, 0]
