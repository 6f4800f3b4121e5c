"""GPU parity at the five workloads' full sizes, in the launch configurations
the benchmark times, on outputs the oracle can compute one by one: sampled
heads for the assignment, the centre update and the codes; sampled query rows
(including the ragged last query block) for attention.

Every input of a GPU call compared here comes from the generators or from the
oracle: attention reads caches the oracle encoded for a few source heads, tiled
over the workload's head count on the device, so each GPU head is checked
against the oracle attention of its source head."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import Cache, check_attention, check_ids, encode_heads, nearest_ids, np32

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


def _rows(n_q, seed, n=192):
    rng = np.random.default_rng(seed)
    last = np.arange(max(0, n_q - 40), n_q)                 # ragged last query block
    return np.unique(np.concatenate([rng.choice(n_q, n, replace=False), last, [0]]))


def _check_rows(out, lse, q, head_map, segs_of_source, rows, what, lowdim=None):
    """Compare GPU rows of every head with the oracle of its source head."""
    out = out.cpu().numpy()
    lse = lse.cpu().numpy()
    refs = {}
    worst = (0.0, 0.0, 0.0)
    for h, src in enumerate(head_map):
        if src not in refs:
            qs = np32(q[h])[rows]
            if lowdim is None:
                refs[src] = oracle.attend(qs, segs_of_source(src))
            else:
                Uk, Uv = lowdim
                refs[src] = oracle.attend_lowdim(qs, Uk[src], Uv[src], segs_of_source(src))
        o_ref, l_ref = refs[src]
        r = check_attention(out[h][rows], lse[h][rows], o_ref, l_ref, f"{what} head {h}")
        worst = tuple(max(a, b) for a, b in zip(worst, r))
    print(f"{what}: worst rel-L2 {worst[0]:.2e} max-abs {worst[1]:.2e} |dLSE| {worst[2]:.2e}")
    return worst


def _queries_tiled(cfg, head_map, n_q=None, stream_id=0):
    """Queries drawn per source head and tiled like the cache (same rows per source)."""
    src = sorted(set(head_map))
    qs = synth.queries(cfg, heads=max(src) + 1, n_q=n_q, stream_id=stream_id)
    return qs[torch.as_tensor(head_map)].contiguous()


# ------------------------------------------------------------------------------ tiny (everything, all elements)
def test_tiny_whole_path():
    cfg = synth.get_config("tiny")
    k, _ = synth.tiny_kv(cfg, "k")
    v, _ = synth.tiny_kv(cfg, "v")
    q = synth.queries(cfg)
    kc0 = synth.forgy_init(k, 16, synth.seed_for(cfg.seed, 0, 0, 1))
    vc0 = synth.forgy_init(v, 16, synth.seed_for(cfg.seed, 0, 1, 1))
    kc_g, vc_g = kc0.to(DEV).clone(), vc0.to(DEV).clone()
    kid_g = kvc().fit_assign(k.to(DEV), kc_g, n_iter=2)
    vid_g = kvc().fit_assign(v.to(DEV), vc_g, n_iter=2)
    torch.cuda.synchronize()
    kc_o, kid_o, hist = oracle.fit(np32(k)[0], np32(kc0)[0], 2, "f32", history=True)
    vc_o, vid_o = oracle.fit(np32(v)[0], np32(vc0)[0], 2, "f32")
    assert np.array_equal(np32(kc_g)[0], kc_o) and np.array_equal(kid_g.cpu().numpy()[0], kid_o)
    assert np.array_equal(np32(vc_g)[0], vc_o) and np.array_equal(vid_g.cpu().numpy()[0], vid_o)
    cache = Cache(np32(k), np32(v), kc_o[None], vc_o[None], kid_o[None], vid_o[None], cfg.k_bits, cfg.v_bits,
                  cfg.group)
    codes, meta, _ = kvc().encode(k.to(DEV), torch.from_numpy(kc_o[None]).to(DEV), cfg.k_bits, cfg.group,
                                  ids=torch.from_numpy(kid_o[None].astype(np.uint8)).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), cache.k_codes) and np.array_equal(meta.cpu().numpy(), cache.k_meta)
    out, lse = kvc().attend(q.to(DEV), [cache.gpu_segment(torch.float32)])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend(np32(q)[0], [cache.oracle_segment(0)])
    check_attention(out.cpu().numpy()[0], lse.cpu().numpy()[0], o_ref, l_ref, "tiny")


# ------------------------------------------------------------------------------ assignment + update, full size
@pytest.mark.parametrize("name", ["self_forcing_layer", "long_history", "larger_backbone", "streaming"])
def test_assign_and_update_full_size(name):
    """One assignment and one Lloyd iteration over every head at the workload's
    full size (long_history: 12 heads x 70200 tokens and larger_backbone: 40
    heads x 32760, whose updates sort member lists in the workspace, 18 and 8
    chunks a head), checked on sampled heads:
    ids against the oracle's assignment, and, wherever the GPU's ids equal the
    oracle's (a near-tie resolved the other way changes the update's input),
    the updated centres bit for bit and the ids after the update."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = synth.get_config(name)
    N = cfg.chunk if name == "streaming" else cfg.hist
    x = synth.AR1Stream(cfg, "k", device=DEV).tokens(N)
    cent0 = synth.forgy_init(x, cfg.n_centroids, synth.seed_for(cfg.seed, 0, 0, 1))
    sample = [0, cfg.heads - 1] if N > 20000 else [0, cfg.heads // 2, cfg.heads - 1]
    c_g = cent0.clone()
    ids_g = kvc().fit_assign(x, c_g, n_iter=0).cpu().numpy()
    c1_g = cent0.clone()
    ids1_g = kvc().fit_assign(x, c1_g, n_iter=1).cpu().numpy()
    torch.cuda.synchronize()
    xs, cs = np32(x[sample]), np32(cent0[sample])
    c1s = np32(c1_g[sample])

    def one(i):
        h = sample[i]
        ref0 = oracle.assign(xs[i], cs[i])
        tie, differ = check_ids(ids_g[h].astype(np.int64), xs[i], cs[i], what=f"{name} head {h}", ref=ref0)
        if differ:
            return tie, False
        c1, ids1, hist = oracle.fit(xs[i], cs[i], n_iter=1, storage="bf16", history=True)
        assert np.array_equal(hist[0][1], ref0[0])
        assert np.array_equal(c1s[i].view(np.uint32), c1.view(np.uint32)), f"{name} head {h}: centres"
        check_ids(ids1_g[h].astype(np.int64), xs[i], c1, what=f"{name} head {h} after the update")
        return tie, True

    # numpy releases the GIL inside the oracle's array operations: heads in parallel
    with ThreadPoolExecutor(max_workers=len(sample)) as ex:
        res = list(ex.map(one, range(len(sample))))
    excl = sum(t for t, _ in res)
    updated = sum(u for _, u in res)
    print(f"{name}: near-ties excluded {excl} of {len(sample) * N}; centre updates checked on {updated} heads")
    assert excl <= 0.001 * len(sample) * N
    assert updated >= 1


@pytest.mark.parametrize("H,N,stream", [(34, 17160, True), (32, 16390, False), (12, 9362, False),
                                        (512, 32772, False)])
def test_update_with_per_head_member_lists(H, N, stream):
    """Heads long enough for the update to sort each head's member lists once in
    the workspace: 34 heads x 17160 tokens of the synthetic stream (11 latent
    frames; the sort in 5 chunks a head), 32 heads x 16390 and 12 heads x 9362
    random tokens (lengths that are not a multiple of 4: the sort reads the ids
    byte by byte), and 512 heads x 32772 random tokens (longer than the LDS
    path takes, and heads enough for one sorting workgroup a head); 100 centres
    with one duplicated centre (no members: it keeps its value).  Centres after
    one Lloyd iteration bit for bit against the oracle on sampled heads whose
    ids equal the oracle's."""
    from concurrent.futures import ThreadPoolExecutor
    C = 100
    if stream:
        x = synth.AR1Stream(synth.get_config("larger_backbone"), "v", heads=H, device=DEV).tokens(N)
    else:
        g = torch.Generator(device=DEV).manual_seed(31)
        x = torch.randn(H, N, 128, generator=g, device=DEV).to(torch.bfloat16)
    cent0 = synth.forgy_init(x, C, 29)
    cent0[:, C - 1] = cent0[:, 5]
    assert kvc().library().kvc_fit_assign_workspace_bytes(H, N, 128, C) > 4 * H * N
    c1_g = cent0.clone()
    ids_g = kvc().fit_assign(x, cent0.clone(), n_iter=0).cpu().numpy()
    kvc().fit_assign(x, c1_g, n_iter=1)
    torch.cuda.synchronize()
    sample = [0, H // 2, H - 1]
    xs, cs, c1s = np32(x[sample]), np32(cent0[sample]), np32(c1_g[sample])
    assert np.array_equal(c1s[:, C - 1].view(np.uint32), cs[:, C - 1].view(np.uint32))

    def one(i):
        h = sample[i]
        ref0 = oracle.assign(xs[i], cs[i])
        _, differ = check_ids(ids_g[h].astype(np.int64), xs[i], cs[i], what=f"head {h}", ref=ref0)
        if differ:
            return False
        c1, _ = oracle.fit(xs[i], cs[i], n_iter=1, storage="bf16")
        assert np.array_equal(c1s[i].view(np.uint32), c1.view(np.uint32)), f"head {h}: centres"
        return True

    with ThreadPoolExecutor(max_workers=len(sample)) as ex:
        assert sum(ex.map(one, range(len(sample)))) >= 1


# ------------------------------------------------------------------------------ encode, full size
@pytest.mark.parametrize("name", ["self_forcing_layer", "long_history", "larger_backbone", "streaming"])
def test_encode_full_size(name):
    cfg = synth.get_config(name)
    N = cfg.chunk if name == "streaming" else cfg.hist
    x = synth.AR1Stream(cfg, "v", device=DEV).tokens(N)
    cent = synth.forgy_init(x, cfg.n_centroids, synth.seed_for(cfg.seed, 0, 1, 1))
    sample = [0, cfg.heads - 1]
    xs, cs = np32(x[sample]), np32(cent[sample])
    ids = torch.randint(0, cfg.n_centroids, (cfg.heads, N), generator=torch.Generator().manual_seed(5),
                        dtype=torch.int64)
    ids_s = nearest_ids(xs, cs)
    for i, h in enumerate(sample):
        ids[h] = torch.from_numpy(ids_s[i])
    ids_dev = ids.to(torch.uint8).to(DEV)
    for bits in sorted({cfg.k_bits, cfg.v_bits}):
        codes, meta, _ = kvc().encode(x, cent, bits, cfg.group, ids=ids_dev)
        torch.cuda.synchronize()
        ref_c, ref_m = encode_heads(xs, cs, ids_s, bits, cfg.group)
        assert np.array_equal(codes[sample].cpu().numpy(), ref_c), f"{name} codes b{bits}"
        assert np.array_equal(_u16(meta, sample), ref_m), f"{name} meta b{bits}"
    if cfg.rank:
        U = synth.orthonormal_basis(cfg.heads, cfg.dim, cfg.rank, synth.seed_for(cfg.seed, 0, 1, 2))
        xf = x[:, :cfg.far].contiguous()
        codes, meta, _ = kvc().encode(xf, cent, cfg.v_bits, cfg.group, ids=ids_dev[:, :cfg.far].contiguous(),
                                      basis=U.to(DEV))
        torch.cuda.synchronize()
        ref_c, ref_m = encode_heads(xs[:, :cfg.far], cs, ids_s[:, :cfg.far], cfg.v_bits, cfg.group,
                                    U.numpy()[sample])
        assert np.array_equal(codes[sample].cpu().numpy(), ref_c), f"{name} low-dim codes"
        assert np.array_equal(_u16(meta, sample), ref_m), f"{name} low-dim meta"


# ------------------------------------------------------------------------------ attention, full size
def _source_caches(cfg, n_src, bounds, basis=None, stream_tables=False):
    """Oracle-encoded caches for n_src source heads, one Cache per history segment."""
    N = bounds[-1]
    k = synth.AR1Stream(cfg, "k", heads=n_src).tokens(N)
    v = synth.AR1Stream(cfg, "v", heads=n_src).tokens(N)
    kn, vn = np32(k), np32(v)
    caches = []
    for si, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        if stream_tables or si == 0:
            base = (a, b) if stream_tables else (0, N)
            kc = np32(synth.forgy_init(k[:, base[0]:base[1]], cfg.n_centroids, synth.seed_for(cfg.seed, si, 0, 1)))
            vc = np32(synth.forgy_init(v[:, base[0]:base[1]], cfg.n_centroids, synth.seed_for(cfg.seed, si, 1, 1)))
        kid = nearest_ids(kn[:, a:b], kc)
        vid = nearest_ids(vn[:, a:b], vc)
        bk = None if basis is None else basis[0]
        bv = None if basis is None else basis[1]
        caches.append(Cache(kn[:, a:b], vn[:, a:b], kc, vc, kid, vid, cfg.k_bits, cfg.v_bits, cfg.group, bk, bv))
    return caches


@pytest.mark.parametrize("name", ["self_forcing_layer", "long_history", "streaming"])
def test_attend_full_size(name):
    cfg = synth.get_config(name)
    n_src = 2
    if name == "streaming":
        bounds = [cfg.chunk * i for i in range(cfg.steps + 1)]       # step 10: ten chunks of history
    else:
        bounds = [cfg.hist * i // cfg.n_segments for i in range(cfg.n_segments + 1)]
    caches = _source_caches(cfg, n_src, bounds, stream_tables=(name == "streaming"))
    head_map = [h % n_src for h in range(cfg.heads)]
    q = _queries_tiled(cfg, head_map)
    segs = [c.gpu_segment(head_map=head_map) for c in caches]
    out, lse = kvc().attend(q.to(DEV), segs)
    torch.cuda.synchronize()
    rows = _rows(cfg.n_q, cfg.seed, n=128 if name == "streaming" else 192)
    check_heads = list(range(cfg.heads)) if cfg.heads <= 40 else [0, 1, 2, 3, 357, 358, 718, 719]
    sub_map = [head_map[h] for h in check_heads]
    _check_rows(out[check_heads], lse[check_heads], q[check_heads], sub_map,
                lambda s: [c.oracle_segment(s) for c in caches], rows, name)


def test_larger_backbone_recent_far_merge():
    cfg = synth.get_config("larger_backbone")
    n_src = 2
    Uk = synth.orthonormal_basis(n_src, cfg.dim, cfg.rank, synth.seed_for(cfg.seed, 0, 0, 2)).numpy()
    Uv = synth.orthonormal_basis(n_src, cfg.dim, cfg.rank, synth.seed_for(cfg.seed, 0, 1, 2)).numpy()
    N, F = cfg.hist, cfg.far
    k = synth.AR1Stream(cfg, "k", heads=n_src).tokens(N)
    v = synth.AR1Stream(cfg, "v", heads=n_src).tokens(N)
    kn, vn = np32(k), np32(v)
    kc = np32(synth.forgy_init(k, cfg.n_centroids, 1))
    vc = np32(synth.forgy_init(v, cfg.n_centroids, 2))
    kid, vid = nearest_ids(kn, kc), nearest_ids(vn, vc)
    far = Cache(kn[:, :F], vn[:, :F], kc, vc, kid[:, :F], vid[:, :F], cfg.k_bits, cfg.v_bits, cfg.group, Uk, Uv)
    recent = Cache(kn[:, F:], vn[:, F:], kc, vc, kid[:, F:], vid[:, F:], cfg.k_bits, cfg.v_bits, cfg.group)
    head_map = [h % n_src for h in range(cfg.heads)]
    q = _queries_tiled(cfg, head_map).to(DEV)
    idx = torch.as_tensor(head_map, device=DEV)
    Ukd = torch.from_numpy(Uk).to(DEV).index_select(0, idx).contiguous()
    Uvd = torch.from_numpy(Uv).to(DEV).index_select(0, idx).contiguous()
    o1, l1 = kvc().attend(q, [recent.gpu_segment(head_map=head_map)])
    o2, l2 = kvc().attend_lowdim(q, Ukd, Uvd, [far.gpu_segment(head_map=head_map)])
    om, lm = kvc().lse_merge([o1, o2], [l1, l2])
    torch.cuda.synchronize()
    rows = _rows(cfg.n_q, cfg.seed)
    hs = [0, 1, 20, 39]
    sub = [head_map[h] for h in hs]
    qc = q[hs].cpu()
    _check_rows(o1[hs], l1[hs], qc, sub, lambda s: [recent.oracle_segment(s)], rows, "larger_backbone recent")
    _check_rows(o2[hs], l2[hs], qc, sub, lambda s: [far.oracle_segment(s)], rows, "larger_backbone far",
                lowdim=(Uk, Uv))
    # merged result against the oracle's merge of its own two parts
    om, lm = om.cpu().numpy(), lm.cpu().numpy()
    for h, s in zip(hs, sub):
        qs = np32(qc[hs.index(h)])[rows]
        a = oracle.attend(qs, [recent.oracle_segment(s)])
        b = oracle.attend_lowdim(qs, Uk[s], Uv[s], [far.oracle_segment(s)])
        o_ref, l_ref = oracle.lse_merge([a[0], b[0]], [a[1], b[1]])
        check_attention(om[h][rows], lm[h][rows], o_ref, l_ref, f"larger_backbone merged head {h}")


def test_larger_backbone_routed_frames_with_anchor():
    """Routing of NanoKV appendix Table 7 (4 recent frames, one anchor per 16 older
    frames) on the larger backbone's 21 frames, the oldest frame coded at
    b_a = max(4, b_K, b_V) bits: the full-dimensional frames (two codecs) go to one
    attention call, the other 15 to the low-dim call, then the LSE merge."""
    from oracle.routing import anchor_bits, route_frames
    cfg = synth.get_config("larger_backbone")
    n_src, S = 2, cfg.frame_tokens
    n_frames = cfg.hist // S
    mask = kvc().route_frames(n_frames, 4, 16)
    assert mask == route_frames(n_frames, 4, 16)
    ba = kvc().anchor_bits(cfg.k_bits, cfg.v_bits)
    assert ba == anchor_bits(cfg.k_bits, cfg.v_bits) == 4
    Uk = synth.orthonormal_basis(n_src, cfg.dim, cfg.rank, synth.seed_for(cfg.seed, 0, 0, 2)).numpy()
    Uv = synth.orthonormal_basis(n_src, cfg.dim, cfg.rank, synth.seed_for(cfg.seed, 0, 1, 2)).numpy()
    k = synth.AR1Stream(cfg, "k", heads=n_src).tokens(cfg.hist)
    v = synth.AR1Stream(cfg, "v", heads=n_src).tokens(cfg.hist)
    kn, vn = np32(k), np32(v)
    kc = np32(synth.forgy_init(k, cfg.n_centroids, 3))
    vc = np32(synth.forgy_init(v, cfg.n_centroids, 4))
    kid, vid = nearest_ids(kn, kc), nearest_ids(vn, vc)
    full, low = [], []
    f = 0
    while f < n_frames:
        e = f
        while e < n_frames and mask[e] == mask[f]:
            e += 1
        a, b = f * S, e * S
        if mask[f]:
            if f == 0:                               # the anchor frame, then the rest of the run
                full.append(Cache(kn[:, :S], vn[:, :S], kc, vc, kid[:, :S], vid[:, :S], ba, ba, cfg.group))
                a = S
            if b > a:
                full.append(Cache(kn[:, a:b], vn[:, a:b], kc, vc, kid[:, a:b], vid[:, a:b], cfg.k_bits, cfg.v_bits,
                                  cfg.group))
        else:
            low.append(Cache(kn[:, a:b], vn[:, a:b], kc, vc, kid[:, a:b], vid[:, a:b], cfg.k_bits, cfg.v_bits,
                             cfg.group, Uk, Uv))
        f = e
    assert len(full) == 2 and len(low) == 1          # anchor frame 0; frames 16-20; frames 1-15
    head_map = [h % n_src for h in range(cfg.heads)]
    q = _queries_tiled(cfg, head_map).to(DEV)
    idx = torch.as_tensor(head_map, device=DEV)
    Ukd = torch.from_numpy(Uk).to(DEV).index_select(0, idx).contiguous()
    Uvd = torch.from_numpy(Uv).to(DEV).index_select(0, idx).contiguous()
    o1, l1 = kvc().attend(q, [c.gpu_segment(head_map=head_map) for c in full])
    o2, l2 = kvc().attend_lowdim(q, Ukd, Uvd, [c.gpu_segment(head_map=head_map) for c in low])
    om, lm = kvc().lse_merge([o1, o2], [l1, l2])
    torch.cuda.synchronize()
    rows = _rows(cfg.n_q, cfg.seed)
    hs = [0, 1, 39]
    sub = [head_map[h] for h in hs]
    qc = q[hs].cpu()
    om, lm = om.cpu().numpy(), lm.cpu().numpy()
    for h, s in zip(hs, sub):
        qs = np32(qc[hs.index(h)])[rows]
        a = oracle.attend(qs, [c.oracle_segment(s) for c in full])
        b = oracle.attend_lowdim(qs, Uk[s], Uv[s], [c.oracle_segment(s) for c in low])
        o_ref, l_ref = oracle.lse_merge([a[0], b[0]], [a[1], b[1]])
        check_attention(om[h][rows], lm[h][rows], o_ref, l_ref, f"routed larger_backbone head {h}")


def _u16(t, idx):
    """Rows of a uint16 GPU tensor as numpy (torch has no uint16 indexing on the GPU)."""
    return t.view(torch.int16)[idx].cpu().numpy().view(np.uint16)
