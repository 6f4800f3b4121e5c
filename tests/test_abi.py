"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and rejects malformed arguments before any GPU work.  No call
here launches a kernel (all inputs fail validation or describe empty work)."""
import ctypes
import os
import re

import pytest

from compressed_kv_cache_kvc_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "kvc.h")

INV, UNS, WS, OK = _lib.KVC_ERR_INVALID_ARG, _lib.KVC_ERR_UNSUPPORTED, _lib.KVC_ERR_WORKSPACE, _lib.KVC_OK
P = ctypes.c_void_p(1 << 20)       # aligned fake device pointer: never dereferenced here
MIS = ctypes.c_void_p((1 << 20) + 8)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_symbols_exported(lib):
    text = open(HDR).read()
    declared = set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text))
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    for name in declared:
        assert getattr(lib, name) is not None


def test_version_and_status_strings(lib):
    assert lib.kvc_version().decode().startswith("kvc")
    for s, name in [(0, "KVC_OK"), (1, "KVC_ERR_INVALID_ARG"), (2, "KVC_ERR_UNSUPPORTED"),
                    (3, "KVC_ERR_WORKSPACE"), (4, "KVC_ERR_HIP")]:
        assert lib.kvc_status_string(s).decode() == name


def _encode(lib, **kw):
    a = dict(heads=2, n=100, dim=128, dt=1, x=P, C=16, cent=P, ids_in=P, ids_out=None, basis=None, rank=0,
             bits=2, group=16, codes=P, meta=P, ws=None, wsb=0)
    a.update(kw)
    return lib.kvc_encode(a["heads"], a["n"], a["dim"], a["dt"], a["x"], a["C"], a["cent"], a["ids_in"],
                          a["ids_out"], a["basis"], a["rank"], a["bits"], a["group"], a["codes"], a["meta"],
                          a["ws"], a["wsb"], None)


def test_encode_validation(lib):
    assert _encode(lib, dim=96) == INV
    assert _encode(lib, bits=3) == INV
    assert _encode(lib, group=12) == INV
    assert _encode(lib, group=8) == UNS
    assert _encode(lib, C=0) == INV and _encode(lib, C=257) == INV
    assert _encode(lib, rank=32) == INV                       # rank without a basis
    assert _encode(lib, basis=P, rank=48) == UNS              # valid, but no kernel for rank 48
    assert _encode(lib, basis=P, rank=8) == INV               # rank below the group
    assert _encode(lib, basis=P, rank=32, dim=64) == UNS
    assert _encode(lib, x=None) == INV
    assert _encode(lib, codes=MIS) == INV
    assert "aligned" in lib.kvc_last_error().decode()
    assert lib.kvc_encode_workspace_bytes(2, 100, 128, 16, 0) == 0   # the assignment needs no workspace
    assert _encode(lib, ids_in=None, ids_out=None) == INV
    assert _encode(lib, n=-1) == INV
    assert _encode(lib, n=0, x=None, codes=None, meta=None) == OK   # empty work: no launch
    assert lib.kvc_last_error().decode() == ""


def test_fit_assign_validation(lib):
    f = lib.kvc_fit_assign
    assert f(1, 10, 128, 1, P, 4, P, 2, P, None, 0, None) == WS
    need = lib.kvc_fit_assign_workspace_bytes(1, 10, 128, 4)
    assert need >= 16
    assert f(1, 10, 100, 1, P, 4, P, 2, P, P, need, None) == INV
    assert f(1, 10, 128, 7, P, 4, P, 2, P, P, need, None) == INV
    assert f(1, 10, 128, 1, P, 300, P, 2, P, P, need, None) == INV
    assert f(1, 10, 128, 1, P, 4, P, -1, P, P, need, None) == INV
    assert f(1, 1 << 31, 128, 1, P, 4, P, 0, P, P, 1 << 40, None) == INV   # 32-bit token indices
    assert f(65536, 10, 128, 1, P, 4, P, 2, P, P, 1 << 40, None) == UNS      # grid: at most 65535 heads
    assert f(0, 10, 128, 1, None, 4, None, 2, None, None, 0, None) == OK


def _seg(**kw):
    s = _lib.KvcSegment()
    s.n_tokens, s.n_centroids, s.rank, s.k_bits, s.v_bits, s.group, s.cent_dtype = 100, 16, 0, 2, 2, 16, 1
    for n in ("k_codes", "v_codes", "k_meta", "v_meta", "k_ids", "v_ids", "k_cent", "v_cent"):
        setattr(s, n, P.value)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _attend(lib, segs, **kw):
    a = dict(heads=2, n_q=10, dim=128, qdt=1, q=P, out=P, lse=P, ws=P, wsb=1 << 30)
    a.update(kw)
    arr = (_lib.KvcSegment * max(1, len(segs)))(*segs)
    return lib.kvc_attend(a["heads"], a["n_q"], a["dim"], a["qdt"], a["q"], arr, len(segs), a["out"], a["lse"],
                          a["ws"], a["wsb"], None)


def test_attend_validation(lib):
    assert _attend(lib, [_seg(k_bits=3)]) == INV
    assert _attend(lib, [_seg(group=24)]) == INV
    assert _attend(lib, [_seg(rank=32)]) == INV
    # segments of different codecs are attended in one launch per codec and merged;
    # a workspace of 0 bytes stops the call before any launch
    assert _attend(lib, [_seg(), _seg(v_bits=4)], wsb=0) == WS
    arr = (_lib.KvcSegment * 2)(_seg(n_tokens=9360), _seg(n_tokens=1560, k_bits=4, v_bits=4))
    rows = 12 * 4680                                          # two partial results, then the merge
    assert lib.kvc_attend_workspace_bytes(12, 4680, 128, 1, arr, 2) == \
        2 * rows * 128 * 4 + 2 * rows * 4 + 2 * _tables(12, 16, 128)
    raw = _seg(k_bits=16, v_bits=16, k_meta=None, v_meta=None)
    assert _attend(lib, [raw], wsb=0) == WS                   # 16-bit residual segments need no metadata
    assert _attend(lib, [_seg(k_bits=16, v_bits=2)]) == UNS   # 16-bit K needs 16-bit V
    assert _attend(lib, [raw], qdt=0) == UNS                  # fp32 queries read 2/4-bit codes only
    # 16-bit residual rows are 256 bytes at d = 128: at most 2^24 rows per head
    # keep the kernel's 32-bit row offsets in range; 2/4-bit segments allow 2^25
    big16 = _seg(k_bits=16, v_bits=16, k_meta=None, v_meta=None, n_tokens=(1 << 24) + 1)
    assert _attend(lib, [big16], wsb=0) == UNS
    assert "2^24" in lib.kvc_last_error().decode()
    ok16 = _seg(k_bits=16, v_bits=16, k_meta=None, v_meta=None, n_tokens=1 << 24)
    assert _attend(lib, [ok16], wsb=0) == WS                  # passes the limit, stops at the workspace
    assert _attend(lib, [_seg(n_tokens=(1 << 25) + 1)], wsb=0) == UNS
    assert _attend(lib, [_seg(n_tokens=1 << 25)], wsb=0) == WS
    assert _attend(lib, [_seg(k_codes=None)]) == INV
    assert _attend(lib, [_seg()] * 25) == UNS                 # more segments than one launch walks
    assert _attend(lib, [_seg(cent_dtype=0)]) == UNS          # bf16 queries with fp32 centres
    assert _attend(lib, [_seg()], heads=0) == OK
    arr = (_lib.KvcSegment * 1)(_seg(n_tokens=9360))
    need = lib.kvc_attend_workspace_bytes(1, 256, 128, 1, arr, 1)
    assert need > 0                                           # one query block: the history is split
    assert _attend(lib, [_seg(n_tokens=9360)], heads=1, n_q=256, ws=P, wsb=need - 1) == WS


def _tables(heads, C, dim):
    """fp16 copies of the K and V centre tables that full-dim attention stages in its workspace."""
    return 2 * heads * C * dim * 2


def test_split_plan_sizes(lib):
    # self-forcing-like layer: 12 heads x 19 query blocks = 228 workgroups: no split
    arr = (_lib.KvcSegment * 1)(_seg(n_tokens=9360))
    assert lib.kvc_attend_workspace_bytes(12, 4680, 128, 1, arr, 1) == _tables(12, 16, 128)
    # 2 heads x 4 query blocks over 146 tiles: split 8 ways (64 workgroups)
    rows = 2 * 1000
    need = lib.kvc_attend_workspace_bytes(2, 1000, 128, 1, arr, 1)
    assert need == pytest.approx(8 * rows * 128 * 4 + 8 * rows * 4 + _tables(2, 16, 128), rel=1e-3)
    # streaming: 720 heads fill the chip without a split
    arr = (_lib.KvcSegment * 1)(_seg(n_tokens=46800))
    assert lib.kvc_attend_workspace_bytes(720, 4680, 128, 1, arr, 1) == _tables(720, 16, 128)
    # fp32 queries read the fp32 centres directly and never split
    assert lib.kvc_attend_workspace_bytes(720, 4680, 128, 0, arr, 1) == 0


def test_lowdim_validation(lib):
    arr = (_lib.KvcSegment * 1)(_seg(rank=32))
    f = lib.kvc_attend_lowdim
    assert f(2, 10, 128, 1, P, P, P, 48, arr, 1, P, P, P, 1 << 30, None) == UNS
    assert f(2, 10, 128, 0, P, P, P, 32, arr, 1, P, P, P, 1 << 30, None) == UNS
    assert f(2, 10, 128, 1, P, None, P, 32, arr, 1, P, P, P, 1 << 30, None) == INV
    arr0 = (_lib.KvcSegment * 1)(_seg(rank=0))
    assert f(2, 10, 128, 1, P, P, P, 32, arr0, 1, P, P, P, 1 << 30, None) == INV


def test_merge_validation(lib):
    po = (ctypes.c_void_p * 2)(P.value, P.value)
    f = lib.kvc_lse_merge
    assert f(1, 10, 128, 0, po, po, P, P, None) == INV
    assert f(1, 10, 127, 2, po, po, P, P, None) == INV
    assert f(1, 10, 128, 2, po, po, P, P, None) == INV        # part 1 aliases the output
    assert f(0, 10, 128, 2, po, po, P, P, None) == OK


def test_qsac_validation(lib):
    f = lib.kvc_assign_qsac
    # (heads, n, dim, dt, x, C, cent, w, n_cand, group, ids, stream)
    assert f(1, 10, 100, 1, P, 16, P, None, 4, 16, P, None) == INV        # dim
    assert f(1, 10, 128, 7, P, 16, P, None, 4, 16, P, None) == INV        # dtype
    assert f(1, 10, 128, 1, P, 0, P, None, 4, 16, P, None) == INV         # C
    assert f(1, 10, 128, 1, P, 16, P, None, 0, 16, P, None) == INV        # n_cand
    assert f(1, 10, 128, 1, P, 16, P, None, 3, 16, P, None) == UNS        # n_cand not built
    assert f(1, 10, 128, 1, P, 16, P, None, 4, 24, P, None) == INV        # group does not divide dim
    assert f(1, 10, 128, 1, P, 16, P, None, 4, 64, P, None) == UNS        # group not built
    assert f(1, 10, 128, 1, None, 16, P, None, 4, 16, P, None) == INV     # x NULL
    assert f(1, 10, 128, 1, MIS, 16, P, None, 4, 16, P, None) == INV      # misaligned
    assert f(1, 10, 128, 1, P, 16, P, MIS, 4, 16, P, None) == INV         # misaligned weights
    assert f(70000, 10, 128, 1, P, 16, P, None, 4, 16, P, None) == UNS    # heads
    assert f(1, 0, 128, 1, None, 16, None, None, 4, 16, None, None) == OK  # empty


def test_query_stats_validation(lib):
    f = lib.kvc_query_stats
    # (heads, n_q, dim, dt, q, n_prev, w, ws, ws_bytes, stream)
    big = 1 << 30
    assert f(1, 10, 100, 1, P, 0, P, P, big, None) == INV
    assert f(1, 10, 128, 9, P, 0, P, P, big, None) == INV
    assert f(1, 10, 128, 1, P, -1, P, P, big, None) == INV
    assert f(1, 10, 128, 1, P, 0, None, P, big, None) == INV
    assert f(1, 0, 128, 1, None, 0, None, None, 0, None) == OK
    # fp64 partial sums per block of queries: 720 heads x 2 blocks, 12 heads x 19 blocks
    assert lib.kvc_query_stats_workspace_bytes(720, 4680, 128) == 720 * 2 * 128 * 8
    assert lib.kvc_query_stats_workspace_bytes(12, 4680, 128) == 12 * 19 * 128 * 8
    need = lib.kvc_query_stats_workspace_bytes(12, 4680, 128)
    assert f(12, 4680, 128, 1, P, 0, P, P, need - 1, None) == WS


def test_route_frames_matches_oracle(lib, golden_dir):
    import json
    from oracle.routing import anchor_bits, route_frames
    import compressed_kv_cache_kvc_amd as kvc
    g = json.load(open(os.path.join(golden_dir, "routing_table7.json")))
    for c in g["cases"]:
        args = (c["n_frames"], c["n_recent"], c["period"], c["n_sink"], c["all_full_until"])
        assert kvc.route_frames(*args) == route_frames(*args), c["rule"]
    for F in range(0, 40):
        for args in ((F, 4, 16, 0, 0), (F, 2, 0, 1, 9), (F, 5, 0, 0, 0), (F, 0, 3, 2, 0)):
            assert kvc.route_frames(*args) == route_frames(*args)
    for kb, vb, want in g["anchor_bits"]:
        assert kvc.anchor_bits(kb, vb) == anchor_bits(kb, vb) == want
    assert lib.kvc_route_frames(-1, 0, 0, 0, 0, None) == INV
