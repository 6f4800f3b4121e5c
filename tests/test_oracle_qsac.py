"""Pins of the oracle's query-aware assignment (QSAC) and query statistics.

QuantWM (2609.26425), section 4.1.  Each test checks the oracle against
something other than itself: hand-derived cases, brute force over Fractions,
the plain nearest-centre assignment (M = 1, w = 1), invariances of the
definition, the Widrow error model by Monte Carlo, and the closed form of the
statistics.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import assign, assign_qsac, query_stats
from oracle.qsac import qsac_score, weighted_dist


def test_hand_derived_cases(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "qsac_examples.json")))["cases"]
    for case in cases:
        x = np.array(case["x"])
        cent = np.array(case["cent"])
        w = case["w"]
        for m, want in case["expect"].items():
            ids, _, _ = assign_qsac(x, cent, w, int(m), case["group"])
            assert list(ids) == want, (case["note"], m)
        for m, want in case.get("unweighted_expect", {}).items():
            ids, _, _ = assign_qsac(x, cent, None, int(m), case["group"])
            assert list(ids) == want, (case["note"], m)
        ww = np.ones(x.shape[1]) if w is None else np.array(w)
        assert list(weighted_dist(x, cent, ww)[0]) == case["dist"]
        if "scores" in case:
            got = [qsac_score(x[0], c, ww, case["group"]) for c in cent]
            assert got == case["scores"]


def _frac_rows(a):
    return [[Fraction(float(v)) for v in row] for row in a]


def _brute_qsac(x, cent, w, m, group):
    """The definition over Fractions: top-m by weighted distance (ties to the
    lower index), then the smallest sum_g W_g R_g^2 (ties to the lower index)."""
    xs, cs = _frac_rows(x), _frac_rows(cent)
    ws = [Fraction(float(v)) for v in w]
    d = len(ws)
    out = []
    for xr in xs:
        dist = []
        for k, cr in enumerate(cs):
            dist.append((sum(ws[i] * (xr[i] - cr[i]) ** 2 for i in range(d)), k))
        cands = [k for _, k in sorted(dist)[:m]]
        best = None
        for k in cands:
            r = [xr[i] - cs[k][i] for i in range(d)]
            s = Fraction(0)
            for g0 in range(0, d, group):
                grp = r[g0:g0 + group]
                s += sum(ws[g0:g0 + group]) * (max(grp) - min(grp)) ** 2
            if best is None or (s, k) < best:
                best = (s, k)
        out.append(best[1])
    return out


@pytest.mark.parametrize("m,C,d,group,seed", [(1, 7, 8, 4, 0), (2, 9, 8, 2, 1), (4, 12, 8, 4, 2),
                                              (12, 12, 6, 3, 3), (3, 5, 8, 8, 4)])
def test_matches_brute_force_over_fractions(m, C, d, group, seed):
    rng = np.random.default_rng(seed)
    # small dyadic values, so that exact ties occur and the tie rules are exercised
    x = rng.integers(-4, 5, size=(60, d)) / 4.0
    cent = rng.integers(-4, 5, size=(C, d)) / 4.0
    w = rng.integers(1, 5, size=d) / 2.0
    ids, _, _ = assign_qsac(x, cent, w, m, group)
    assert list(ids) == _brute_qsac(x, cent, w, m, group)


def test_one_candidate_unit_weights_is_plain_assignment():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((300, 16))
    cent = rng.standard_normal((20, 16))
    ids, _, _ = assign_qsac(x, cent, None, 1, 4)
    plain, _, _ = assign(x, cent)
    assert np.array_equal(ids, plain)


def test_invariances():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((200, 16))
    cent = rng.standard_normal((24, 16))
    w = rng.uniform(0.2, 3.0, 16)
    ids, cg, sg = assign_qsac(x, cent, w, 4, 4)
    # a common positive scale of the weights changes no choice
    ids2, _, _ = assign_qsac(x, cent, w * 7.5, 4, 4)
    assert np.array_equal(ids, ids2)
    # relabelling the centres relabels the ids (tokens clear of near ties)
    perm = rng.permutation(24)
    ids3, _, _ = assign_qsac(x, cent[perm], w, 4, 4)
    ok = (cg > 1e-9) & (sg > 1e-9)
    assert ok.sum() > 150
    assert np.array_equal(perm[ids3][ok], ids[ok])
    # more candidates never raise the chosen centre's score
    ids8, _, _ = assign_qsac(x, cent, w, 8, 4)
    s4 = np.array([qsac_score(x[j], cent[ids[j]], w, 4) for j in range(len(x))])
    s8 = np.array([qsac_score(x[j], cent[ids8[j]], w, 4) for j in range(len(x))])
    assert np.all(s8 <= s4)


def test_score_is_the_widrow_logit_error_up_to_its_constant():
    """E[(q . e)^2] for queries with E[q_c^2] = w_c and uniform rounding errors
    of step R_g / (2^b - 1) in each group equals score / (12 (2^b - 1)^2)."""
    rng = np.random.default_rng(9)
    d, g, b = 16, 4, 2
    w = rng.uniform(0.5, 2.0, d)
    x = rng.standard_normal(d)
    mu = rng.standard_normal(d)
    r = x - mu
    step = np.repeat([np.ptp(r[i:i + g]) / (2 ** b - 1) for i in range(0, d, g)], g)
    n = 400_000
    q = rng.standard_normal((n, d)) * np.sqrt(w)
    e = (rng.random((n, d)) - 0.5) * step
    mc = np.mean(np.einsum("nd,nd->n", q, e) ** 2)
    want = qsac_score(x, mu, w, g) / (12 * (2 ** b - 1) ** 2)
    assert mc == pytest.approx(want, rel=0.02)


def test_query_stats_closed_form_and_running_update():
    q = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert list(query_stats(q)) == [5.0, 10.0]
    rng = np.random.default_rng(10)
    a = rng.standard_normal((37, 8))
    b = rng.standard_normal((11, 8))
    both = query_stats(np.concatenate([a, b]))
    run = query_stats(b, query_stats(a), n_prev=37)
    assert np.allclose(run, both, rtol=1e-14, atol=0)
    # n_prev = 0 ignores whatever statistics are passed in (cold start)
    assert np.array_equal(query_stats(b, np.full(8, 123.0), n_prev=0), query_stats(b))
