"""Query-aware centre assignment of key tokens (QSAC) and the query statistics
it uses.  TEST INFRASTRUCTURE ONLY (part of the oracle package).

What is computed, in the pages' terms (QuantWM, 2609.26425, section 4.1; the
page's equations are stripped from the text, so the formulas below are rebuilt
from its prose):

* query_stats -- the second-moment statistics of the queries seen so far, per
  head; QSAC keeps only the diagonal, w_c = E[q_c^2] (section 4.1, Eqs. 6-8:
  the expected squared logit error of a key error e is e^T M e, and the
  diagonal of M weighs channel c).  Cold start (appendix, causal
  initialization): no earlier queries means w_c = 1 for every channel.
* assign_qsac -- for each key token x:
    1. the query-aware distance d_w(x, mu_j) = sum_c w_c (x_c - mu_jc)^2
       (Eq. 9, the diagonal form) selects the M candidate centres with the
       smallest d_w (top-M; ties to the lower centre index);
    2. for each candidate, the residual r = x - mu_j and its range per group of
       g channels, R_g = max r - min r (Eq. 10);
    3. uniform b-bit quantization of a group with step R_g / (2^b - 1) has the
       error variance step^2 / 12 (the Widrow model, Eq. 11); weighted by w and
       summed, the expected squared logit error is
       sum_g (sum_{c in g} w_c) R_g^2 / (12 (2^b - 1)^2);
       the constant factor is common to all candidates and dropped, leaving the
       QSAC score  S_j = sum_g W_g R_g^2,  W_g = sum_{c in g} w_c  (Eq. 12);
    4. the token takes the candidate with the smallest score, ties to the lower
       centre index.
  M = 1 with w = 1 is the plain nearest-centre assignment.  Reading: the bit
  width drops out of the choice (it only scales every score alike).

All arithmetic is fp64 from the stored values (bf16 and fp32 widen exactly).
Pinned by tests/test_oracle_qsac.py (hand-derived examples, brute force over
Fractions, the M = 1 special case, invariances, the Widrow constant by Monte
Carlo, the closed form of the statistics).
"""
from __future__ import annotations

import numpy as np


def query_stats(q, w_prev=None, n_prev: int = 0):
    """w_c = mean over all queries seen so far of q_c^2 (fp64), per head.

    q: [n_q, d] queries of one head; w_prev: the statistics of the n_prev
    earlier queries (ignored when n_prev = 0).  Returns the updated w [d].
    """
    q64 = np.asarray(q, dtype=np.float64)
    s = (q64 * q64).sum(axis=0)
    n = q64.shape[0]
    if n_prev > 0:
        s = s + np.asarray(w_prev, dtype=np.float64) * n_prev
    return s / (n + n_prev)


def weighted_dist(x, cent, w):
    """d_w[j, k] = sum_c w_c (x[j, c] - cent[k, c])^2 in fp64 (the definition)."""
    x64 = np.asarray(x, dtype=np.float64)
    c64 = np.asarray(cent, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    diff = x64[:, None, :] - c64[None, :, :]
    return (diff * diff * w64[None, None, :]).sum(axis=-1)


def qsac_score(x_row, cent_row, w, group: int) -> float:
    """S = sum over groups of (sum of w in the group) * (range of x - mu)^2."""
    r = np.asarray(x_row, dtype=np.float64) - np.asarray(cent_row, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    d = r.shape[0]
    s = 0.0
    for g0 in range(0, d, group):
        rg = r[g0:g0 + group]
        R = rg.max() - rg.min()
        s += w64[g0:g0 + group].sum() * R * R
    return s


def assign_qsac(x, cent, w, n_cand: int, group: int, chunk: int = 64):
    """QSAC ids of one head's key tokens.

    x [N, d], cent [C, d] (stored values), w [d] channel weights (None: all 1),
    n_cand = M, group = g (divides d).  Returns (ids, cand_gap, score_gap):
    ids int64 [N]; cand_gap = relative gap (d_(M+1) - d_(M)) / d_(M+1) between
    the last candidate and the first excluded centre (inf when C <= M);
    score_gap = relative gap (S_2nd - S_best) / S_2nd between the two best
    candidate scores (inf with a single candidate).  The gaps let a comparison
    skip tokens whose answer turns on a near tie.
    """
    x64 = np.asarray(x, dtype=np.float64)
    c64 = np.asarray(cent, dtype=np.float64)
    N, d = x64.shape
    C = c64.shape[0]
    if d % group:
        raise ValueError("group must divide the dimension")
    w64 = np.ones(d) if w is None else np.asarray(w, dtype=np.float64)
    M = min(n_cand, C)
    ids = np.empty(N, np.int64)
    cand_gap = np.full(N, np.inf)
    score_gap = np.full(N, np.inf)
    for s in range(0, N, chunk):
        D = weighted_dist(x64[s:s + chunk], c64, w64)
        for jj in range(D.shape[0]):
            j = s + jj
            order = np.argsort(D[jj], kind="stable")        # ties keep the lower index first
            cands = order[:M]
            if C > M:
                a, b = D[jj, order[M - 1]], D[jj, order[M]]
                cand_gap[j] = (b - a) / b if b > 0 else 0.0
            scores = [(qsac_score(x64[j], c64[k], w64, group), int(k)) for k in cands]
            scores.sort()                                    # by score, then by index
            ids[j] = scores[0][1]
            if len(scores) > 1:
                s1, s2 = scores[0][0], scores[1][0]
                score_gap[j] = (s2 - s1) / s2 if s2 > 0 else 0.0
    return ids, cand_gap, score_gap
