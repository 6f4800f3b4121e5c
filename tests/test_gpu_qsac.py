"""GPU parity of the query-aware key assignment (QSAC, QuantWM section 4.1) and
the query statistics against the oracle.

ids must match the oracle except for tokens whose answer turns on a near tie:
a relative gap between the M-th and (M+1)-th query-weighted distance, or
between the two best candidate scores, above 0 and below 1e-5 (the GPU scores
the candidates in fp32); such tokens must stay under 1%.  Exact ties (a
duplicated centre) must resolve to the lower index on both sides.  The
statistics must match within 1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import np32

pytestmark = pytest.mark.gpu
DEV = "cuda"
GAP = 1e-5


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


def _weights(H, d, seed):
    """Channel weights from synthetic queries (the statistics a later chunk sees)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(H, 700, d, generator=g) * torch.linspace(0.3, 2.0, d)
    return torch.stack([torch.from_numpy(oracle.query_stats(np32(q[h]))).float() for h in range(H)])


def _valid_on_near_tie(gid, xr, cent, w, m, group):
    """Whether id gid is a valid QSAC answer for token xr when its answer turns
    on a near tie: some resolution of the near ties at the candidate boundary
    must put gid among the M candidates (its weighted distance within GAP of
    the M-th smallest), and its score must be within GAP of the smallest score
    of the candidates every resolution keeps (those clearly inside)."""
    from oracle.qsac import qsac_score, weighted_dist
    C = cent.shape[0]
    if not 0 <= gid < C:
        return False
    wv = np.ones(xr.shape[0]) if w is None else w
    D = weighted_dist(xr[None], cent, wv)[0]
    M = min(m, C)
    dm = np.sort(D)[M - 1]
    if D[gid] > dm * (1 + GAP):
        return False
    sure = np.nonzero(D < dm * (1 - GAP))[0]
    if len(sure) == 0:
        return True
    s_sure = min(qsac_score(xr, cent[k], wv, group) for k in sure)
    return qsac_score(xr, cent[gid], wv, group) <= s_sure * (1 + GAP)


def _check(ids_gpu, x, cent, w, m, group, tokens=None):
    """ids equal the oracle's except on near ties (a relative gap in (0, GAP) at
    the candidate boundary or between the two best scores), where the GPU's id
    must still be a valid answer (_valid_on_near_tie)."""
    H = x.shape[0]
    excluded = total = 0
    for h in range(H):
        sel = np.arange(x.shape[1]) if tokens is None else tokens
        wh = None if w is None else w[h]
        ids, cg, sg = oracle.assign_qsac(x[h][sel], cent[h], wh, m, group)
        # exact ties (a duplicated centre) have one answer, the lower index
        tie = ((cg > 0) & (cg < GAP)) | ((sg > 0) & (sg < GAP))
        got = ids_gpu[h][sel]
        bad = (got != ids) & ~tie
        assert not bad.any(), f"head {h}: {int(bad.sum())} ids differ outside near ties"
        for j in np.nonzero(tie & (got != ids))[0]:
            assert _valid_on_near_tie(int(got[j]), x[h][sel[j]], cent[h], wh, m, group), \
                f"head {h} token {sel[j]}: id {got[j]} is not a valid answer on its near tie"
        excluded += int(tie.sum())
        total += len(sel)
    assert excluded <= max(2, 0.01 * total), f"{excluded} of {total} tokens near a tie"
    return excluded


@pytest.mark.parametrize("d,C,N,m,group,weighted", [
    (128, 256, 1300, 4, 16, True), (128, 256, 1000, 4, 32, False), (128, 100, 777, 8, 16, True),
    (128, 256, 600, 1, 16, True), (128, 64, 513, 2, 32, True), (64, 16, 700, 4, 32, True),
    (64, 256, 300, 8, 16, False), (128, 3, 200, 4, 16, True)])
def test_qsac_bf16_matches_oracle(d, C, N, m, group, weighted):
    cfg = synth.get_config("self_forcing_layer")
    H = 2
    x = synth.AR1Stream(cfg, "k", heads=H).tokens(1560)[:, :N, :d].contiguous()
    cent = synth.forgy_init(x, C, 11)
    if C > 2:
        cent[:, C - 1] = cent[:, 1]                # an exact duplicate: ties go to the lower index
    w = _weights(H, d, 12) if weighted else None
    ids = kvc().assign_qsac(x.to(DEV), cent.to(DEV), None if w is None else w.to(DEV), m, group)
    torch.cuda.synchronize()
    _check(ids.cpu().numpy().astype(np.int64), np32(x), np32(cent), None if w is None else w.numpy(), m, group)


def test_qsac_one_candidate_unit_weights_is_the_plain_assignment():
    cfg = synth.get_config("self_forcing_layer")
    H, N, C = 2, 1500, 256
    x = synth.AR1Stream(cfg, "k", heads=H).tokens(1560)[:, :N].contiguous()
    cent = synth.forgy_init(x, C, 13)
    plain = kvc().fit_assign(x.to(DEV), cent.to(DEV).clone(), n_iter=0)
    q1 = kvc().assign_qsac(x.to(DEV), cent.to(DEV), None, 1, 16)
    torch.cuda.synchronize()
    assert torch.equal(plain.cpu(), q1.cpu())


def test_qsac_fp32_tiny():
    cfg = synth.get_config("tiny")
    x, _ = synth.tiny_kv(cfg, "k")
    cent = synth.forgy_init(x, cfg.n_centroids, 14)
    w = _weights(1, cfg.dim, 15)
    for m in (1, 4, 8):
        ids = kvc().assign_qsac(x.to(DEV), cent.to(DEV), w.to(DEV), m, cfg.group)
        torch.cuda.synchronize()
        _check(ids.cpu().numpy().astype(np.int64), np32(x), np32(cent), w.numpy(), m, cfg.group)


def test_qsac_full_size_sampled_tokens():
    """The self-forcing layer's keys at full size (12 heads x 9360 tokens, C = 256,
    M = 4, g = 16), checked on a sample of tokens of every head."""
    cfg = synth.get_config("self_forcing_layer")
    x = synth.AR1Stream(cfg, "k").tokens(cfg.hist)
    cent = synth.forgy_init(x, cfg.n_centroids, 16)
    w = _weights(cfg.heads, cfg.dim, 17)
    ids = kvc().assign_qsac(x.to(DEV), cent.to(DEV), w.to(DEV), 4, cfg.group)
    torch.cuda.synchronize()
    rng = np.random.default_rng(18)
    sample = np.sort(rng.choice(cfg.hist, 300, replace=False))
    _check(ids.cpu().numpy().astype(np.int64), np32(x), np32(cent), w.numpy(), 4, cfg.group, tokens=sample)


def test_qsac_empty_and_single_token():
    x = torch.randn(1, 1, 128).to(torch.bfloat16)
    cent = torch.randn(1, 5, 128).to(torch.bfloat16)
    ids = kvc().assign_qsac(x.to(DEV), cent.to(DEV), None, 4, 16)
    torch.cuda.synchronize()
    want, _, _ = oracle.assign_qsac(np32(x[0]), np32(cent[0]), None, 4, 16)
    assert int(ids[0, 0]) == int(want[0])
    empty = kvc().assign_qsac(x[:, :0].to(DEV), cent.to(DEV), None, 4, 16)
    assert empty.shape == (1, 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_query_stats_matches_oracle(dtype):
    g = torch.Generator().manual_seed(19)
    H, d = 3, 128
    a = (torch.randn(H, 1001, d, generator=g) * 2).to(dtype)
    b = (torch.randn(H, 37, d, generator=g)).to(dtype)
    w = kvc().query_stats(a.to(DEV))
    w = kvc().query_stats(b.to(DEV), w, n_prev=1001)
    torch.cuda.synchronize()
    for h in range(H):
        want = oracle.query_stats(np32(b[h]), oracle.query_stats(np32(a[h])), n_prev=1001)
        assert np.allclose(w[h].cpu().numpy(), want, rtol=1e-6, atol=0)
