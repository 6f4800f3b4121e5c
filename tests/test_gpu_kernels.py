"""GPU parity of each kernel against the oracle at sizes the oracle finishes in
seconds, spanning several tiles with ragged tails, plus the edge cases.

Codes and metadata must be bit-exact given the same ids and centres; ids must
match except where the oracle's top-2 distance gap is below 1e-5 relative;
attention must be within rel-L2 1e-2, max-abs 2e-2 and |dLSE| 2e-2 of the fp64
oracle on the same (oracle-made) cache; the LSE merge within 1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import Cache, check_attention, check_ids, encode_heads, near_tie, np32

pytestmark = pytest.mark.gpu
DEV = "cuda"


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


def _bf16_tokens(H, N, d, seed, scale=1.0, outliers=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(H, N, d, generator=g) * scale
    if outliers:
        x[:, :, :4] *= 8.0
    return x.to(torch.bfloat16)


# ------------------------------------------------------------------------------ encode
@pytest.mark.parametrize("d,bits,group,dtype", [
    (128, 2, 16, torch.bfloat16), (128, 4, 32, torch.bfloat16), (128, 2, 32, torch.bfloat16),
    (128, 4, 16, torch.bfloat16), (64, 2, 16, torch.bfloat16), (64, 4, 32, torch.bfloat16),
    (64, 4, 32, torch.float32), (128, 2, 16, torch.float32),
    (128, 16, 16, torch.bfloat16), (64, 16, 32, torch.float32), (128, 16, 16, torch.float32)])
def test_encode_bit_exact(d, bits, group, dtype):
    H, N, C = 3, 1037, 37
    x = _bf16_tokens(H, N, d, 1).to(dtype)
    if dtype == torch.float32:
        x = x + 1e-3 * torch.randn(H, N, d, generator=torch.Generator().manual_seed(2))
    cent = synth.forgy_init(x, C, 3)
    cent[:, 0] = 0                                  # an all-zero centre for the edge cases
    xn, cn = np32(x), np32(cent)
    ids = np.stack([oracle.assign(xn[h], cn[h])[0] for h in range(H)])
    # edge cases (ids are inputs of encode, so they may point anywhere): a token
    # equal to its centre, tiny residuals (subnormal fp16 scales), a constant
    # group, a large-magnitude token
    x2 = x.clone()
    g = torch.Generator().manual_seed(12)
    for h in range(H):
        x2[h, 5] = cent[h, ids[h, 5]]
        ids[h, 6:9] = 0
        x2[h, 6] = (1e-6 * torch.randn(d, generator=g)).to(dtype)
        x2[h, 7, :group] = 0.5
        x2[h, 8] = (torch.linspace(-300, 300, d)).to(dtype)
    xn = np32(x2)
    ref_codes, ref_meta = encode_heads(xn, cn, ids, bits, group)
    codes, meta, _ = kvc().encode(x2.to(DEV), cent.to(DEV), bits, group,
                                  ids=torch.from_numpy(ids.astype(np.uint8)).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), ref_codes)
    if bits == 16:                                  # fp16 residuals carry no metadata
        assert meta is None and ref_meta is None
    else:
        assert np.array_equal(meta.cpu().numpy(), ref_meta)


@pytest.mark.parametrize("bits,group", [(2, 16), (4, 32), (16, 16)])
def test_encode_more_heads_than_one_launch_covers(bits, group):
    """65537 heads of 3 tokens: the encoder's grid takes at most 65535 heads per
    launch, so this call needs two; codes and metadata are checked bit-exactly on
    heads at both ends of each launch and around the boundary."""
    H, N, d, C = 65537, 3, 64, 4
    g = torch.Generator().manual_seed(21)
    x = (torch.randn(H, N, d, generator=g) * 2.0).to(torch.bfloat16)
    cent = (torch.randn(H, C, d, generator=g) * 2.0).to(torch.bfloat16)
    ids = torch.randint(0, C, (H, N), generator=g, dtype=torch.uint8)
    codes, meta, _ = kvc().encode(x.to(DEV), cent.to(DEV), bits, group, ids=ids.to(DEV))
    torch.cuda.synchronize()
    sel = np.array([0, 1, 65533, 65534, 65535, 65536])
    xs, cs, ids_s = np32(x[sel]), np32(cent[sel]), ids[sel].numpy().astype(np.int64)
    ref_codes, ref_meta = encode_heads(xs, cs, ids_s, bits, group)
    assert np.array_equal(codes.cpu().numpy()[sel], ref_codes)
    if bits == 16:
        assert meta is None
    else:
        assert np.array_equal(meta.cpu().numpy()[sel], ref_meta)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_encode_with_assignment_more_heads_than_one_launch_covers(dtype):
    """65537 heads of 5 tokens, ids left to the call: the assignment inside it
    also takes at most 65535 heads per launch (the matrix-core kernel for bf16,
    the exact kernel for fp32).  Ids are checked against the oracle and codes
    bit-exactly (given those ids) on heads at both ends of each launch."""
    H, N, d, C, bits, group = 65537, 5, 64, 4, 4, 32
    g = torch.Generator().manual_seed(23)
    x = (torch.randn(H, N, d, generator=g) * 2.0).to(dtype)
    cent = (torch.randn(H, C, d, generator=g) * 2.0).to(dtype)
    codes, meta, ids = kvc().encode(x.to(DEV), cent.to(DEV), bits, group)
    torch.cuda.synchronize()
    sel = np.array([0, 1, 65533, 65534, 65535, 65536])
    xs, cs = np32(x[sel]), np32(cent[sel])
    ids_s = ids.cpu().numpy()[sel]
    for i, h in enumerate(sel):
        check_ids(ids_s[i], xs[i], cs[i], what=f"head {h}")
    ref_codes, ref_meta = encode_heads(xs, cs, ids_s.astype(np.int64), bits, group)
    assert np.array_equal(codes.cpu().numpy()[sel], ref_codes)
    assert np.array_equal(meta.cpu().numpy()[sel], ref_meta)


def test_encode_lowdim_more_heads_than_one_launch_covers():
    """Coefficient codes over 65537 heads (two launches); seven distinct bases
    repeat over the heads, so a basis read from the wrong head of the second
    launch (65535 is not a multiple of 7) changes the codes."""
    H, N, d, C, rank, bits, group = 65537, 3, 128, 4, 32, 2, 16
    g = torch.Generator().manual_seed(24)
    x = (torch.randn(H, N, d, generator=g) * 2.0).to(torch.bfloat16)
    cent = (torch.randn(H, C, d, generator=g) * 2.0).to(torch.bfloat16)
    ids = torch.randint(0, C, (H, N), generator=g, dtype=torch.uint8)
    B = synth.orthonormal_basis(7, d, rank, 25)
    U = B[torch.arange(H) % 7].contiguous()
    codes, meta, _ = kvc().encode(x.to(DEV), cent.to(DEV), bits, group, ids=ids.to(DEV), basis=U.to(DEV))
    torch.cuda.synchronize()
    sel = np.array([0, 1, 65533, 65534, 65535, 65536])
    ref_codes, ref_meta = encode_heads(np32(x[sel]), np32(cent[sel]), ids[sel].numpy().astype(np.int64), bits,
                                       group, U[sel].numpy())
    assert np.array_equal(codes.cpu().numpy()[sel], ref_codes)
    assert np.array_equal(meta.cpu().numpy()[sel], ref_meta)


@pytest.mark.parametrize("rank,bits,group", [(32, 2, 16), (32, 4, 16), (64, 4, 32), (64, 2, 32)])
def test_encode_lowdim_bit_exact(rank, bits, group):
    H, N, C, d = 2, 777, 20, 128
    x = _bf16_tokens(H, N, d, 4)
    cent = synth.forgy_init(x, C, 5)
    U = synth.orthonormal_basis(H, d, rank, 6)
    xn, cn = np32(x), np32(cent)
    ids = np.stack([oracle.assign(xn[h], cn[h])[0] for h in range(H)])
    ref_codes, ref_meta = encode_heads(xn, cn, ids, bits, group, U.numpy())
    codes, meta, _ = kvc().encode(x.to(DEV), cent.to(DEV), bits, group,
                                  ids=torch.from_numpy(ids.astype(np.uint8)).to(DEV), basis=U.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), ref_codes)
    assert np.array_equal(meta.cpu().numpy(), ref_meta)


# ------------------------------------------------------------------------------ assign / fit
def _check_ids(ids_gpu, x, cent):
    """ids equal except near-ties, where the GPU's id must still be among the
    nearest centres; exact ties (D1 == D2) must go to the lowest index like the
    oracle's.  Returns the number of excluded near-ties."""
    return sum(check_ids(ids_gpu[h], x[h], cent[h], what=f"head {h}")[0] for h in range(x.shape[0]))


@pytest.mark.parametrize("d,C,N", [(128, 256, 1300), (128, 100, 999), (128, 80, 777), (64, 16, 700), (64, 256, 513)])
def test_assign_bf16(d, C, N):
    cfg = synth.get_config("self_forcing_layer")
    H = 2
    x = synth.AR1Stream(cfg, "k", heads=H).tokens(1560)[:, :N, :d].contiguous() if d == 128 else \
        _bf16_tokens(H, N, d, 7)
    cent = synth.forgy_init(x, C, 8)
    cent[:, C - 1] = cent[:, 0]                    # exact duplicate: ties go to the lower index
    ids = kvc().fit_assign(x.to(DEV), cent.to(DEV).clone(), n_iter=0)
    torch.cuda.synchronize()
    excl = _check_ids(ids.cpu().numpy().astype(np.int64), np32(x), np32(cent))
    assert excl <= max(2, 0.001 * H * N)


@pytest.mark.parametrize("d,N", [(128, 1000), (64, 600)])
def test_assign_every_token_flagged_many_rounds(d, N):
    """Centres 32..63 duplicate centres 0..31, so every token is an exact tie
    between its nearest centre and that centre's copy and takes the exact pass.
    1024 heads give each workgroup several consecutive rounds of 256 tokens (a
    ragged last one), so the per-wavefront list of such tokens fills and is
    resolved more than once.  Ties go to the lowest index, like the oracle's."""
    H, C0 = 1024, 32
    x = _bf16_tokens(H, N, d, 91)
    base = synth.forgy_init(x, C0, 92)
    cent = torch.cat([base, base], dim=1).contiguous()
    ids = kvc().fit_assign(x.to(DEV), cent.to(DEV).clone(), n_iter=0).cpu().numpy().astype(np.int64)
    assert ids.max() < C0, "a token took the copy of its centre (ties go to the lower index)"
    xn, cn = np32(x), np32(cent)
    for h in (0, 1, 2, 511, 512, 1022, 1023):
        check_ids(ids[h], xn[h], cn[h], what=f"head {h}")
    # identical centres: every token ties with all of them and takes id 0
    same = cent[:, :1].expand(H, 8, d).contiguous()
    ids0 = kvc().fit_assign(x.to(DEV), same.to(DEV).clone(), n_iter=0)
    assert int(ids0.max().item()) == 0


def test_assign_fp32_tiny():
    cfg = synth.get_config("tiny")
    x, _ = synth.tiny_kv(cfg, "k")
    cent = synth.forgy_init(x, cfg.n_centroids, 9)
    ids = kvc().fit_assign(x.to(DEV), cent.to(DEV).clone(), n_iter=0)
    torch.cuda.synchronize()
    _check_ids(ids.cpu().numpy().astype(np.int64), np32(x), np32(cent))


@pytest.mark.parametrize("dtype,storage", [(torch.bfloat16, "bf16"), (torch.float32, "f32")])
def test_fit_matches_oracle_per_iteration(dtype, storage):
    cfg = synth.get_config("self_forcing_layer")
    H, N, C = 2, 1560, 64
    x = synth.AR1Stream(cfg, "v", heads=H).tokens(1560).to(dtype)
    init = synth.forgy_init(x, C, 10)
    xn = np32(x)
    cent_o = np32(init).copy()
    for it in range(2):
        # one GPU iteration from the oracle's current centres
        cg = torch.from_numpy(cent_o).to(dtype).to(DEV)
        ids_g = kvc().fit_assign(x.to(DEV), cg, n_iter=1)
        torch.cuda.synchronize()
        for h in range(H):
            ids0, d1, d2 = oracle.assign(xn[h], cent_o[h])
            assert not near_tie(d1, d2).any(), "near-tie in the update test input"
            c1, ids1 = oracle.fit(xn[h], cent_o[h], n_iter=1, storage=storage)
            assert np.array_equal(np32(cg)[h].view(np.uint32), c1.view(np.uint32)), f"iteration {it} head {h}"
            assert np.array_equal(ids_g.cpu().numpy()[h].astype(np.int64), ids1)
            cent_o[h] = c1


def test_fit_many_heads():
    # 200 heads x 100 centres: C = 100 leaves a partial last workgroup of centres
    H, N, C, d = 200, 300, 100, 64
    x = _bf16_tokens(H, N, d, 13)
    init = synth.forgy_init(x, C, 14)
    cg = init.to(DEV).clone()
    ids_g = kvc().fit_assign(x.to(DEV), cg, n_iter=1)
    torch.cuda.synchronize()
    xn, cn = np32(x), np32(init)
    checked = 0
    for h in (0, 1, 99, 199):
        _, d1, d2 = oracle.assign(xn[h], cn[h])
        if near_tie(d1, d2).any():
            continue
        c1, ids1 = oracle.fit(xn[h], cn[h], n_iter=1, storage="bf16")
        assert np.array_equal(np32(cg)[h].view(np.uint32), c1.view(np.uint32)), f"head {h}"
        check_ids(ids_g.cpu().numpy()[h].astype(np.int64), xn[h], c1, what=f"head {h} after the update")
        checked += 1
    assert checked >= 3


def test_fit_long_history_member_list_chunks():
    # 40000 tokens in one head, more than the update's LDS takes: the member
    # lists are sorted in the workspace in 10 chunks (16 centres), and a centre's
    # list runs across chunk boundaries
    # (seed 16 with these centres has no near-tie token, before or after the update)
    H, N, C, d = 1, 40000, 16, 64
    x = _bf16_tokens(H, N, d, 16)
    init = synth.forgy_init(x, C, 116)
    cg = init.to(DEV).clone()
    ids_g = kvc().fit_assign(x.to(DEV), cg, n_iter=1)
    torch.cuda.synchronize()
    xn, cn = np32(x), np32(init)
    for h in range(H):
        _, d1, d2 = oracle.assign(xn[h], cn[h])
        assert not near_tie(d1, d2).any(), "near-tie in the update test input"
        c1, ids1 = oracle.fit(xn[h], cn[h], n_iter=1, storage="bf16")
        assert np.array_equal(np32(cg)[h].view(np.uint32), c1.view(np.uint32)), f"head {h}"
        check_ids(ids_g.cpu().numpy()[h].astype(np.int64), xn[h], c1, what=f"head {h} after the update")


def test_single_centre_fit_encode_attend():
    # C = 1: every id is 0, the fitted centre is the mean of all tokens, and the
    # codes and the attention follow from that one centre
    H, N, d, n_q = 2, 777, 64, 130
    x_k, x_v = _bf16_tokens(H, N, d, 60), _bf16_tokens(H, N, d, 61)
    xk, xv = np32(x_k), np32(x_v)
    cent = {}
    for name, x, seed in (("k", x_k, 62), ("v", x_v, 63)):
        init = synth.forgy_init(x, 1, seed)
        cg = init.to(DEV).clone()
        ids = kvc().fit_assign(x.to(DEV), cg, n_iter=2)
        torch.cuda.synchronize()
        assert not ids.cpu().numpy().any()
        for h in range(H):
            c2, ids2 = oracle.fit(np32(x)[h], np32(init)[h], n_iter=2, storage="bf16")
            assert not ids2.any()
            assert np.array_equal(np32(cg)[h].view(np.uint32), c2.view(np.uint32)), f"{name} head {h}"
        cent[name] = np32(cg)
    zeros = np.zeros((H, N), dtype=np.int64)
    codes, meta, _ = kvc().encode(x_k.to(DEV), torch.from_numpy(cent["k"]).to(torch.bfloat16).to(DEV), 2, 16,
                                  ids=torch.zeros(H, N, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    ref_codes, ref_meta = encode_heads(xk, cent["k"], zeros, 2, 16)
    assert np.array_equal(codes.cpu().numpy(), ref_codes)
    assert np.array_equal(meta.cpu().numpy(), ref_meta)
    cache = Cache(xk, xv, cent["k"], cent["v"], zeros, zeros, 2, 4, 16)
    _attend_check(_bf16_tokens(H, n_q, d, 64, outliers=False), [cache], what="one centre")


def test_fit_duplicate_centre_stays_empty():
    # an exact duplicate of centre 2 at index 5 draws no member in the first
    # assignment (ties go to the lower index), so the update keeps it unchanged
    H, N, C, d = 2, 900, 8, 128
    x = _bf16_tokens(H, N, d, 65)
    init = synth.forgy_init(x, C, 66)
    init[:, 5] = init[:, 2]
    cg = init.to(DEV).clone()
    ids_g = kvc().fit_assign(x.to(DEV), cg, n_iter=1)
    torch.cuda.synchronize()
    xn, cn = np32(x), np32(init)
    for h in range(H):
        ids0, d1, d2 = oracle.assign(xn[h], cn[h])
        assert not (ids0 == 5).any()
        assert not (near_tie(d1, d2) & (d1 != d2)).any(), "near-tie in the update test input"
        c1, ids1 = oracle.fit(xn[h], cn[h], n_iter=1, storage="bf16")
        assert np.array_equal(c1[5].view(np.uint32), cn[h, 5].view(np.uint32))
        assert np.array_equal(np32(cg)[h].view(np.uint32), c1.view(np.uint32)), f"head {h}"
        check_ids(ids_g.cpu().numpy()[h].astype(np.int64), xn[h], c1, what=f"head {h} after the update")


def test_zero_sizes():
    # no tokens, no queries, no heads: every call returns without a launch
    d = 128
    x = torch.empty(2, 0, d, dtype=torch.bfloat16, device=DEV)
    cent = torch.zeros(2, 4, d, dtype=torch.bfloat16, device=DEV)
    ids = kvc().fit_assign(x, cent, n_iter=2)
    codes, meta, ids2 = kvc().encode(x, cent, 2, 16)
    assert tuple(ids.shape) == (2, 0) and tuple(ids2.shape) == (2, 0)
    assert tuple(codes.shape) == (2, 0, 32) and tuple(meta.shape) == (2, 0, 8, 2)
    assert not cent.float().cpu().numpy().any()
    H, N = 2, 300
    x_k = _bf16_tokens(H, N, d, 67)
    kc = synth.forgy_init(x_k, 8, 68)
    kn, kcn = np32(x_k), np32(kc)
    kid = np.stack([oracle.assign(kn[h], kcn[h])[0] for h in range(H)])
    seg = Cache(kn, kn, kcn, kcn, kid, kid, 2, 2, 16).gpu_segment()
    out, lse = kvc().attend(torch.empty(H, 0, d, dtype=torch.bfloat16, device=DEV), [seg])
    torch.cuda.synchronize()
    assert tuple(out.shape) == (H, 0, d) and tuple(lse.shape) == (H, 0)
    out, lse = kvc().attend(torch.empty(0, 5, d, dtype=torch.bfloat16, device=DEV), [])
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 5, d)


# ------------------------------------------------------------------------------ attention
def _cache(H, N, d, C, kb, vb, g, seed, dtype=torch.bfloat16):
    x_k = _bf16_tokens(H, N, d, seed).to(dtype)
    x_v = _bf16_tokens(H, N, d, seed + 1).to(dtype)
    kc = synth.forgy_init(x_k, C, seed + 2)
    vc = synth.forgy_init(x_v, C, seed + 3)
    kn, vn, kcn, vcn = np32(x_k), np32(x_v), np32(kc), np32(vc)
    kid = np.stack([oracle.assign(kn[h], kcn[h])[0] for h in range(H)])
    vid = np.stack([oracle.assign(vn[h], vcn[h])[0] for h in range(H)])
    return Cache(kn, vn, kcn, vcn, kid, vid, kb, vb, g)


def _attend_check(q, caches, cent_dtype=torch.bfloat16, what=""):
    segs = [c.gpu_segment(cent_dtype) for c in caches]
    out, lse = kvc().attend(q.to(DEV), segs)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qn = np32(q)
    res = []
    for h in range(q.shape[0]):
        o_ref, l_ref = oracle.attend(qn[h], [c.oracle_segment(h) for c in caches])
        res.append(check_attention(out[h], lse[h], o_ref, l_ref, f"{what} head {h}"))
    return res


@pytest.mark.parametrize("d,kb,vb,g", [(128, 2, 2, 16), (128, 4, 4, 32), (128, 2, 4, 16), (128, 4, 2, 32),
                                       (64, 4, 4, 32), (64, 2, 2, 16)])
def test_attend_single_segment(d, kb, vb, g):
    H, N, n_q = 2, 1000, 300
    cache = _cache(H, N, d, 32, kb, vb, g, 20)
    q = _bf16_tokens(H, n_q, d, 21, outliers=False)
    _attend_check(q, [cache], what=f"d{d} k{kb}v{vb}g{g}")


def test_attend_many_ragged_segments():
    H, d, n_q = 3, 128, 517
    caches = [_cache(H, n, d, min(16, n), 2, 4, 16, 30 + i) for i, n in enumerate([130, 64, 1, 333, 700])]
    q = _bf16_tokens(H, n_q, d, 39, outliers=False)
    _attend_check(q, caches, what="5 segments")


def test_attend_split_history():
    # one query block and 80 tiles: the history is split across workgroups and merged
    H, d, n_q, N = 1, 128, 200, 5100
    cache = _cache(H, N, d, 64, 4, 4, 32, 40)
    q = _bf16_tokens(H, n_q, d, 41, outliers=False)
    _attend_check(q, [cache], what="split")


def test_attend_16bit_residual_segment():
    # fp16 residuals (no quantizer): k_hat = fp16(r + c) with one rounding
    H, d, n_q = 2, 128, 300
    cache = _cache(H, 777, d, 32, 16, 16, 16, 45)
    q = _bf16_tokens(H, n_q, d, 46, outliers=False)
    _attend_check(q, [cache], what="16-bit")


def test_attend_mixed_codecs_one_call():
    # an anchor frame at 4 bits, the history at 2 bits, a raw 16-bit segment, a
    # second 2-bit run: one launch per codec, merged by LSE
    H, d, n_q = 2, 128, 333
    caches = [_cache(H, 1560, d, 64, 4, 4, 16, 47), _cache(H, 3000, d, 64, 2, 2, 16, 48),
              _cache(H, 200, d, 16, 16, 16, 16, 49), _cache(H, 450, d, 32, 2, 2, 16, 50)]
    q = _bf16_tokens(H, n_q, d, 51, outliers=False)
    _attend_check(q, caches, what="mixed codecs")


def test_attend_mixed_codecs_split():
    # one query block: each codec's history is also split across workgroups
    H, d, n_q = 1, 128, 200
    caches = [_cache(H, 4100, d, 64, 2, 4, 16, 52), _cache(H, 1560, d, 64, 4, 4, 32, 53)]
    q = _bf16_tokens(H, n_q, d, 54, outliers=False)
    _attend_check(q, caches, what="mixed codecs split")


def test_attend_empty_history():
    q = _bf16_tokens(2, 70, 128, 42, outliers=False).to(DEV)
    out, lse = kvc().attend(q, [])
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any() and np.all(np.isneginf(lse.cpu().numpy()))


def test_attend_fp32_tiny():
    cfg = synth.get_config("tiny")
    k, _ = synth.tiny_kv(cfg, "k")
    v, _ = synth.tiny_kv(cfg, "v")
    q = synth.queries(cfg)
    kc = synth.forgy_init(k, 16, 43)
    vc = synth.forgy_init(v, 16, 44)
    kn, vn, kcn, vcn = np32(k), np32(v), np32(kc), np32(vc)
    kid = np.stack([oracle.assign(kn[0], kcn[0])[0]])
    vid = np.stack([oracle.assign(vn[0], vcn[0])[0]])
    cache = Cache(kn, vn, kcn, vcn, kid, vid, 4, 4, 32)
    _attend_check(q, [cache], cent_dtype=torch.float32, what="tiny fp32")


@pytest.mark.parametrize("d", [128, 64])
def test_attend_fp32_many_ragged_segments(d):
    # fp32 queries and centres over several segments of one codec (ragged sizes,
    # a one-token segment), several heads, a query count that is not a multiple
    # of the four wavefronts of a workgroup; then an empty history
    H, n_q = 3, 203
    caches = [_cache(H, n, d, min(16, n), 4, 2, 16, 70 + i, dtype=torch.float32)
              for i, n in enumerate([130, 1, 517])]
    q = torch.randn(H, n_q, d, generator=torch.Generator().manual_seed(79))
    _attend_check(q, caches, cent_dtype=torch.float32, what=f"fp32 d{d}")
    out, lse = kvc().attend(q.to(DEV), [])
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


# ------------------------------------------------------------------------------ low-dim attention
@pytest.mark.parametrize("rank,kb,vb,g", [(32, 2, 4, 16), (64, 4, 4, 32), (32, 4, 2, 32)])
def test_attend_lowdim(rank, kb, vb, g):
    H, N, d, n_q, C = 2, 900, 128, 270, 24
    x_k = _bf16_tokens(H, N, d, 50)
    x_v = _bf16_tokens(H, N, d, 51)
    kc, vc = synth.forgy_init(x_k, C, 52), synth.forgy_init(x_v, C, 53)
    Uk, Uv = synth.orthonormal_basis(H, d, rank, 54), synth.orthonormal_basis(H, d, rank, 55)
    kn, vn, kcn, vcn = np32(x_k), np32(x_v), np32(kc), np32(vc)
    kid = np.stack([oracle.assign(kn[h], kcn[h])[0] for h in range(H)])
    vid = np.stack([oracle.assign(vn[h], vcn[h])[0] for h in range(H)])
    caches = []
    for part in (slice(0, 500), slice(500, N)):
        caches.append(Cache(kn[:, part], vn[:, part], kcn, vcn, kid[:, part], vid[:, part], kb, vb, g,
                            Uk.numpy(), Uv.numpy()))
    q = _bf16_tokens(H, n_q, d, 56, outliers=False)
    out, lse = kvc().attend_lowdim(q.to(DEV), Uk.to(DEV), Uv.to(DEV), [c.gpu_segment() for c in caches])
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qn = np32(q)
    for h in range(H):
        o_ref, l_ref = oracle.attend_lowdim(qn[h], Uk.numpy()[h], Uv.numpy()[h], [c.oracle_segment(h) for c in caches])
        check_attention(out[h], lse[h], o_ref, l_ref, f"lowdim r{rank} head {h}")


# ------------------------------------------------------------------------------ merge
@pytest.mark.parametrize("P", [1, 2, 5, 40])
def test_lse_merge(P):
    H, n_q, d = 3, 129, 128
    g = torch.Generator().manual_seed(60 + P)
    outs = [torch.randn(H, n_q, d, generator=g) for _ in range(P)]
    lses = [torch.randn(H, n_q, generator=g) * 5 for _ in range(P)]
    if P > 1:
        lses[1][:, :10] = -float("inf")          # empty parts
        for p in range(P):
            lses[p][0, 20] = -float("inf")       # a row with no history at all
    out, lse = kvc().lse_merge([o.to(DEV) for o in outs], [l.to(DEV) for l in lses])
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for h in range(H):
        o_ref, l_ref = oracle.lse_merge([o[h].numpy() for o in outs], [l[h].numpy() for l in lses])
        fin = np.isfinite(l_ref)
        assert np.array_equal(fin, np.isfinite(lse[h]))
        assert np.allclose(lse[h][fin], l_ref[fin], rtol=1e-6, atol=1e-6)
        assert np.allclose(out[h], o_ref, rtol=1e-5, atol=1e-6)
        assert not out[h][~fin].any()


def test_lse_merge_in_place():
    H, n_q, d = 2, 64, 64
    g = torch.Generator().manual_seed(70)
    o0, o1 = torch.randn(H, n_q, d, generator=g), torch.randn(H, n_q, d, generator=g)
    l0, l1 = torch.randn(H, n_q, generator=g), torch.randn(H, n_q, generator=g)
    ref = [oracle.lse_merge([o0[h].numpy(), o1[h].numpy()], [l0[h].numpy(), l1[h].numpy()]) for h in range(H)]
    a, b = o0.to(DEV), l0.to(DEV)
    kvc().lse_merge([a, o1.to(DEV)], [b, l1.to(DEV)], out=a, lse=b)
    torch.cuda.synchronize()
    for h in range(H):
        assert np.allclose(a.cpu().numpy()[h], ref[h][0], rtol=1e-5, atol=1e-6)
        assert np.allclose(b.cpu().numpy()[h], ref[h][1], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("d", [128, 64])
def test_attend_logit_jumps(d):
    """Logits far below the later maximum in the first tiles (the first tile sets
    the reference), then two jumps far above the running maximum mid-history
    (probabilities past the fp16 range before the rescale), then ordinary keys:
    the lazily raised reference must still give the oracle's output and LSE."""
    H, N, n_q, C = 2, 900, 200, 32
    g = torch.Generator().manual_seed(61)
    u = torch.randn(H, 1, d, generator=g)
    u = u / u.norm(dim=-1, keepdim=True)            # one shared direction per head
    q = torch.randn(H, n_q, d, generator=g) + 10.0 * u
    k = torch.randn(H, N, d, generator=g)
    beta = torch.zeros(N)
    beta[:200] = -20.0                               # first tiles: logits ~ -18 below the rest
    beta[300:311] = 40.0                             # jump: ~ +35
    beta[700:706] = 90.0                             # second jump: ~ +80
    k = k + beta[None, :, None] * u
    v = torch.randn(H, N, d, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    kn, vn = np32(k), np32(v)
    kc = synth.forgy_init(k, C, 62)
    vc = synth.forgy_init(v, C, 63)
    kcn, vcn = np32(kc), np32(vc)
    kid = np.stack([oracle.assign(kn[h], kcn[h])[0] for h in range(H)])
    vid = np.stack([oracle.assign(vn[h], vcn[h])[0] for h in range(H)])
    cache = Cache(kn, vn, kcn, vcn, kid, vid, 4, 4, 32)
    # the logits of the dequantized keys do jump as intended
    seg = cache.oracle_segment(0)
    khat = oracle.reconstruct(seg.k_codes, seg.k_meta, seg.k_ids, seg.k_cent, 4, 32)
    s = np32(q)[0] @ khat.T / np.sqrt(d)
    assert s[:, 700:706].max() - s[:, :64].max() > 60 and s[:, 300:311].max() - s[:, :300].max() > 20
    _attend_check(q, [cache], what=f"logit jumps d{d}")


@pytest.mark.parametrize("direction", ["basis_vector", "in_span"])
def test_attend_lowdim_logit_jumps(direction):
    """The rank-32 path (one tile per step) with the full-dimensional test's logit
    jumps, along a direction the reduced key basis keeps: the first tiles far
    below, then jumps of about +35 and +80 (probabilities past the fp16 range
    before the rescale).  Along a basis vector the logit sits on one reduced
    coefficient, so its error is that coefficient's rounding alone (no averaging
    over channels): the reduced queries are carried as fp16 hi + lo for this."""
    H, N, d, n_q, C, rank = 2, 900, 128, 200, 24, 32
    g = torch.Generator().manual_seed(64)
    Uk, Uv = synth.orthonormal_basis(H, d, rank, 65), synth.orthonormal_basis(H, d, rank, 66)
    if direction == "basis_vector":
        u = Uk[:, :, 0].unsqueeze(1)                 # [H, 1, d], unit length, kept by the projection
    else:
        a = torch.randn(H, rank, 1, generator=torch.Generator().manual_seed(69))
        u = (Uk @ (a / a.norm(dim=1, keepdim=True))).transpose(1, 2)
    q = torch.randn(H, n_q, d, generator=g) + 10.0 * u
    k = torch.randn(H, N, d, generator=g)
    beta = torch.zeros(N)
    beta[:200] = -20.0
    beta[300:311] = 40.0
    beta[700:706] = 90.0
    k = k + beta[None, :, None] * u
    v = torch.randn(H, N, d, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    kn, vn = np32(k), np32(v)
    kcn, vcn = np32(synth.forgy_init(k, C, 67)), np32(synth.forgy_init(v, C, 68))
    kid = np.stack([oracle.assign(kn[h], kcn[h])[0] for h in range(H)])
    vid = np.stack([oracle.assign(vn[h], vcn[h])[0] for h in range(H)])
    cache = Cache(kn, vn, kcn, vcn, kid, vid, 2, 4, 16, Uk.numpy(), Uv.numpy())
    out, lse = kvc().attend_lowdim(q.to(DEV), Uk.to(DEV), Uv.to(DEV), [cache.gpu_segment()])
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qn = np32(q)
    for h in range(H):
        o_ref, l_ref = oracle.attend_lowdim(qn[h], Uk.numpy()[h], Uv.numpy()[h], [cache.oracle_segment(h)])
        assert l_ref.max() > 80                         # the jumps reach the reduced logits
        check_attention(out[h], lse[h], o_ref, l_ref, f"lowdim jumps ({direction}) head {h}")
