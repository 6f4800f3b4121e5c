"""kvc_attend_noalloc (the attention call for callers that cannot allocate)
against kvc_attend with a caller workspace: the same kernels and split plan on
the same inputs, so the outputs must agree bit for bit; they are also checked
against the fp64 oracle at the attention tolerances.  Two calls in a row share
the library's static scratch array, the second on a smaller input (and with the
history split across workgroups, so the array also holds split partials); a
call whose workspace would exceed the array is refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import Cache, check_attention, np32

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X: torch.cuda.is_available() is False")
    import compressed_kv_cache_kvc_amd as kvc
    kvc.library()
    yield


def _tokens(H, N, d, seed, outliers=True):
    """Keys and values with four x8 outlier channels; queries ~ N(0, I)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(H, N, d, generator=g)
    if outliers:
        x[:, :, :4] *= 8.0
    return x.to(torch.bfloat16)


def _cache(H, N, d, C, kb, vb, g, seed):
    k, v = _tokens(H, N, d, seed), _tokens(H, N, d, seed + 1)
    kc, vc = synth.forgy_init(k, C, seed + 2), synth.forgy_init(v, C, seed + 3)
    kn, vn, kcn, vcn = np32(k), np32(v), np32(kc), np32(vc)
    kid = np.stack([oracle.assign(kn[h], kcn[h])[0] for h in range(H)])
    vid = np.stack([oracle.assign(vn[h], vcn[h])[0] for h in range(H)])
    return Cache(kn, vn, kcn, vcn, kid, vid, kb, vb, g)


def _both(q, caches, what):
    import compressed_kv_cache_kvc_amd as kvc
    segs = [c.gpu_segment() for c in caches]
    ref_out, ref_lse = kvc.attend(q, segs)
    H, n_q, d = q.shape
    out = torch.full((H, n_q, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((H, n_q), float("nan"), dtype=torch.float32, device=DEV)
    kvc.attend_noalloc(q, segs, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"{what}: differs from kvc_attend"
    qn = np32(q)
    for h in (0, H - 1):
        o_ref, l_ref = oracle.attend(qn[h], [c.oracle_segment(h) for c in caches])
        check_attention(out[h].cpu().numpy(), lse[h].cpu().numpy(), o_ref, l_ref, f"{what} head {h}")


def test_noalloc_matches_attend_two_calls():
    import compressed_kv_cache_kvc_amd as kvc
    from compressed_kv_cache_kvc_amd import _lib
    d = 128
    # first call: 12 heads x 1100 queries over three segments of two codecs
    # (one launch per codec, partials merged: the scratch holds tables and partials)
    caches = [_cache(12, 1560, d, 64, 2, 4, 16, 80), _cache(12, 700, d, 32, 4, 4, 16, 84),
              _cache(12, 333, d, 16, 2, 4, 16, 88)]
    arr = (_lib.KvcSegment * 3)(*[c.gpu_segment().to_c() for c in caches])
    assert kvc.library().kvc_attend_workspace_bytes(12, 1100, d, _lib.KVC_BF16, arr, 3) > 0
    _both(_tokens(12, 1100, d, 90, outliers=False).to(DEV), caches, "first call")
    # second call, smaller: 2 heads x 200 queries (one query block) over one
    # segment of 5000 tokens, so the history is split across workgroups
    small = [_cache(2, 5000, d, 64, 2, 4, 16, 91)]
    _both(_tokens(2, 200, d, 95, outliers=False).to(DEV), small, "second call")


def test_noalloc_refuses_a_workspace_above_the_scratch():
    import compressed_kv_cache_kvc_amd as kvc
    from compressed_kv_cache_kvc_amd import _lib
    # 720 heads over ten 256-centre segments need 943 MiB of fp16 centre tables
    s = _lib.KvcSegment()
    s.n_tokens, s.n_centroids, s.rank, s.k_bits, s.v_bits, s.group, s.cent_dtype = 4680, 256, 0, 2, 4, 16, 1
    P = 1 << 20
    for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_ids", "v_ids", "k_cent", "v_cent"):
        setattr(s, name, P)                       # never dereferenced: the call stops before any launch
    arr = (_lib.KvcSegment * 10)(*([s] * 10))
    lib = kvc.library()
    need = lib.kvc_attend_workspace_bytes(720, 4680, 128, _lib.KVC_BF16, arr, 10)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    st = lib.kvc_attend_noalloc(720, 4680, 128, _lib.KVC_BF16, P, arr, 10, P, P, None)
    assert st == _lib.KVC_ERR_WORKSPACE
    assert "static scratch" in lib.kvc_last_error().decode()
