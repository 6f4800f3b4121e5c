"""GPU parity of the principal-subspace logit compensation (PSAC, QuantWM
section 4.2) against the oracle: query second-moment matrices (1e-5 relative),
the top-8 basis on a planted spectrum (projector within 1e-4), the kept error
coefficients (fp16 storage: 2e-3), and the compensated attention (rel-L2 1e-2,
max-abs 2e-2, |dLSE| 2e-2) given the same basis and coefficients."""
import numpy as np
import pytest
import torch

import oracle
from oracle.psac import attend_psac, psac_basis, psac_coeffs, query_moments
from tests.helpers import Cache, check_attention, np32

pytestmark = pytest.mark.gpu
DEV = "cuda"
R = 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X: torch.cuda.is_available() is False")
    import compressed_kv_cache_kvc_amd as kvc
    kvc.library()
    yield


def kvc():
    import compressed_kv_cache_kvc_amd as m
    return m


def _structured_queries(H, n, d, seed, dtype=torch.bfloat16):
    """Queries whose energy sits mostly in 8 directions per head (the pages'
    observation: the top 8 directions hold more than 60% of it)."""
    g = torch.Generator().manual_seed(seed)
    A = torch.linalg.qr(torch.randn(H, d, d, generator=g, dtype=torch.float64))[0]
    scale = torch.cat([torch.linspace(6.0, 3.0, R, dtype=torch.float64), torch.full((d - R,), 0.5, dtype=torch.float64)])
    z = torch.randn(H, n, d, generator=g, dtype=torch.float64) * scale
    return (z @ A.transpose(1, 2)).to(dtype)


def _cache(H, N, d, C, kb, vb, g, seed):
    gen = torch.Generator().manual_seed(seed)
    k = (torch.randn(H, N, d, generator=gen)).to(torch.bfloat16)
    v = (torch.randn(H, N, d, generator=gen)).to(torch.bfloat16)
    k[:, :, :4] *= 8
    kn, vn = np32(k), np32(v)
    rng = np.random.default_rng(seed)
    kc = np.stack([kn[h][rng.choice(N, C, replace=False)] for h in range(H)])
    vc = np.stack([vn[h][rng.choice(N, C, replace=False)] for h in range(H)])
    kid = np.stack([oracle.assign(kn[h], kc[h])[0] for h in range(H)])
    vid = np.stack([oracle.assign(vn[h], vc[h])[0] for h in range(H)])
    return k, Cache(kn, vn, kc, vc, kid, vid, kb, vb, g)


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float32)])
def test_query_moments(d, dtype):
    H = 3
    a = _structured_queries(H, 1001, d, 1, dtype)
    b = _structured_queries(H, 77, d, 2, dtype)
    m = kvc().query_moments(a.to(DEV))
    m = kvc().query_moments(b.to(DEV), m, n_prev=1001)
    torch.cuda.synchronize()
    for h in range(H):
        want = query_moments(np32(b[h]), query_moments(np32(a[h])), n_prev=1001)
        got = m[h].cpu().numpy()
        assert np.allclose(got, want, rtol=1e-5, atol=1e-5 * np.abs(want).max())


def test_basis_planted_spectrum():
    H, d = 4, 128
    q = _structured_queries(H, 4000, d, 3, torch.float32)
    Ms = np.stack([query_moments(np32(q[h])) for h in range(H)]).astype(np.float32)
    u, lam = kvc().psac_basis(torch.from_numpy(Ms).to(DEV), n_iter=32)
    torch.cuda.synchronize()
    u, lam = u.cpu().numpy().astype(np.float64), lam.cpu().numpy()
    for h in range(H):
        U, w = psac_basis(Ms[h].astype(np.float64), R)
        assert np.abs(u[h] @ u[h].T - U @ U.T).max() < 1e-4
        assert np.allclose(lam[h], w[:R], rtol=1e-4)
        assert np.allclose(u[h].T @ u[h], np.eye(R), atol=1e-5)
        # each column's largest component is positive
        for k in range(R):
            assert u[h][np.argmax(np.abs(u[h][:, k])), k] > 0
    # a warm start from the result converges as well
    u2, _ = kvc().psac_basis(torch.from_numpy(Ms).to(DEV), n_iter=2, u_prev=torch.from_numpy(u.astype(np.float32)).to(DEV))
    torch.cuda.synchronize()
    assert np.abs(u2.cpu().numpy() - u).max() < 1e-4


def _basis(H, d, seed):
    q = _structured_queries(H, 2000, d, seed, torch.float32)
    return np.ascontiguousarray(np.stack([psac_basis(query_moments(np32(q[h])), R)[0] for h in range(H)]), dtype=np.float32)


@pytest.mark.parametrize("kb,g", [(2, 16), (4, 32)])
def test_coefficients(kb, g):
    H, N, d = 2, 999, 128
    k, cache = _cache(H, N, d, 32, kb, 2, g, 4)
    U = _basis(H, d, 5)
    coef = kvc().psac_coeffs(k.to(DEV), torch.from_numpy(cache.kc).to(torch.bfloat16).to(DEV),
                             torch.from_numpy(cache.kid.astype(np.uint8)).to(DEV),
                             torch.from_numpy(cache.k_codes).to(DEV),
                             torch.from_numpy(cache.k_meta.view(np.int16)).to(DEV).view(torch.uint16),
                             kb, g, torch.from_numpy(U).to(DEV))
    torch.cuda.synchronize()
    got = coef.cpu().numpy().view(np.float16).astype(np.float64)
    for h in range(H):
        want = psac_coeffs(np32(k[h]), cache.k_codes[h], cache.k_meta[h], cache.kid[h], cache.kc[h], kb, g, U[h])
        assert np.allclose(got[h], want, rtol=2e-3, atol=2e-3)


def _attend_psac_check(q, caches, U, what):
    """Compensated attention with oracle-made coefficients (rounded to fp16, the
    stored precision) fed to both sides."""
    H = q.shape[0]
    coefs16 = []
    for c, kx in caches:
        cf = np.stack([psac_coeffs(kx[h], c.k_codes[h], c.k_meta[h], c.kid[h], c.kc[h], c.k_bits, c.group, U[h])
                       for h in range(H)]).astype(np.float16)
        coefs16.append(cf)
    segs = [c.gpu_segment() for c, _ in caches]
    out, lse = kvc().attend_psac(q.to(DEV), torch.from_numpy(U).to(DEV), segs,
                                 [torch.from_numpy(cf.view(np.int16)).to(DEV).view(torch.uint16) for cf in coefs16])
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qn = np32(q)
    for h in range(H):
        o_ref, l_ref = attend_psac(qn[h], [c.oracle_segment(h) for c, _ in caches], U[h].astype(np.float64),
                                   [cf[h].astype(np.float64) for cf in coefs16])
        check_attention(out[h], lse[h], o_ref, l_ref, f"{what} head {h}")
    # the compensation moves the result: plain attention differs
    o_plain, _ = oracle.attend(qn[0], [c.oracle_segment(0) for c, _ in caches])
    assert np.abs(o_plain - out[0]).max() > 1e-4


def test_attend_psac_single_segment():
    H, N, d, n_q = 2, 1300, 128, 300
    k, cache = _cache(H, N, d, 32, 2, 2, 16, 6)
    U = _basis(H, d, 7)
    q = _structured_queries(H, n_q, d, 8)
    _attend_psac_check(q, [(cache, np32(k))], U, "psac")


def test_attend_psac_mixed_codecs_and_split():
    # one query block: the history is split; two codecs: two launches, merged
    H, d, n_q = 1, 128, 200
    k1, c1 = _cache(H, 3000, d, 64, 2, 4, 16, 9)
    k2, c2 = _cache(H, 1560, d, 64, 4, 4, 32, 10)
    U = _basis(H, d, 11)
    q = _structured_queries(H, n_q, d, 12)
    _attend_psac_check(q, [(c1, np32(k1)), (c2, np32(k2))], U, "psac mixed split")
