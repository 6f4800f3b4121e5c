"""Pins of the oracle's principal-subspace logit compensation (PSAC, QuantWM
section 4.2): closed forms of the query statistics, the eigen-equation and a
planted spectrum for the basis, the reduction to exact-key attention at r = d
and to plain attention at r = 0, and the stated effect on the expected logit
error (only the energy outside the kept directions remains)."""
import math

import numpy as np

from oracle import attend, dequant, encode
from oracle.attention import Segment
from oracle.psac import attend_psac, psac_basis, psac_coeffs, query_moments


def test_query_moments_closed_form_and_running_mean():
    q = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert np.array_equal(query_moments(q), np.array([[5.0, 7.0], [7.0, 10.0]]))
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal((40, 6)), rng.standard_normal((13, 6))
    run = query_moments(b, query_moments(a), n_prev=40)
    assert np.allclose(run, query_moments(np.concatenate([a, b])), rtol=1e-13, atol=1e-15)


def _planted(d, r, gap, seed):
    rng = np.random.default_rng(seed)
    A, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.concatenate([np.linspace(10.0, 10.0 * gap * 1.5, r), np.linspace(1.0, 0.1, d - r)])
    return A, lam, (A * lam) @ A.T


def test_basis_recovers_a_planted_subspace_and_solves_the_eigen_equation():
    d, r = 32, 8
    A, lam, M = _planted(d, r, 0.5, 2)
    U, w = psac_basis(M, r)
    assert np.allclose(U @ U.T, A[:, :r] @ A[:, :r].T, atol=1e-10)       # same projector
    assert np.allclose(M @ U, U * w[:r], atol=1e-10)                     # M u = lambda u
    assert np.allclose(U.T @ U, np.eye(r), atol=1e-12)
    assert np.all(np.diff(w) <= 0) and np.allclose(np.sort(w)[::-1], np.sort(lam)[::-1])


def _cache(d, n, bits, group, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, d)).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    kc = k[:4].copy()
    vc = v[:4].copy()
    kid = np.argmin(((k[:, None] - kc[None]) ** 2).sum(-1), 1)
    vid = np.argmin(((v[:, None] - vc[None]) ** 2).sum(-1), 1)
    kco, kme = encode(k, kc, kid, bits, group)
    vco, vme = encode(v, vc, vid, bits, group)
    return k, Segment(kco, kme, kid, kc, vco, vme, vid, vc, bits, bits, group)


def test_full_rank_compensation_gives_the_exact_key_logits():
    d, n = 16, 50
    k, seg = _cache(d, n, 2, 8, 3)
    q = np.random.default_rng(4).standard_normal((7, d))
    U, _ = np.linalg.qr(np.random.default_rng(5).standard_normal((d, d)))   # any orthonormal basis
    C = psac_coeffs(k, seg.k_codes, seg.k_meta, seg.k_ids, seg.k_cent, 2, 8, U)
    o, l = attend_psac(q, [seg], U, [C])
    # reference: attention on the unquantized keys with the dequantized values
    vh = seg.v_cent[seg.v_ids].astype(np.float64) + dequant(seg.v_codes, seg.v_meta, 2, 8, d)
    s = q @ k.astype(np.float64).T / math.sqrt(d)
    m = s.max(1, keepdims=True)
    p = np.exp(s - m)
    assert np.allclose(o, (p @ vh) / p.sum(1, keepdims=True), rtol=1e-12, atol=1e-12)
    assert np.allclose(l, m[:, 0] + np.log(p.sum(1)), rtol=1e-12, atol=1e-12)


def test_zero_rank_is_plain_attention():
    d, n = 16, 40
    k, seg = _cache(d, n, 4, 16, 6)
    q = np.random.default_rng(7).standard_normal((5, d))
    U = np.zeros((d, 0))
    C = psac_coeffs(k, seg.k_codes, seg.k_meta, seg.k_ids, seg.k_cent, 4, 16, U)
    o, l = attend_psac(q, [seg], U, [C])
    o2, l2 = attend(q, [seg])
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-13) and np.allclose(l, l2, rtol=1e-13, atol=1e-13)


def test_remaining_logit_error_is_the_energy_outside_the_kept_directions():
    """E_q[(q . e')^2] = e'^T M e' for the error e' left after compensation; with
    U_r the top-r eigenvectors it equals sum_{i>r} lambda_i (u_i . e)^2."""
    d, r = 24, 8
    A, lam, M = _planted(d, r, 0.3, 8)
    U, w = psac_basis(M, r)
    e = np.random.default_rng(9).standard_normal(d)
    e_rest = e - U @ (U.T @ e)
    assert math.isclose(e_rest @ M @ e_rest, float(np.sum(lam[r:] * (A[:, r:].T @ e) ** 2)), rel_tol=1e-10)
    assert e_rest @ M @ e_rest <= e @ M @ e
