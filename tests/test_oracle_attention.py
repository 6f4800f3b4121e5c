"""Pins of the oracle's attention, low-dimensional attention and LSE merge.

Checks against closed forms (a single history token, identical keys), a
textbook softmax attention written independently with explicit loops and a
two-pass log-domain normalisation, the split/merge identity of the
log-sum-exp, exact special cases of the low-dimensional read, and the MAC
accounting identity the NanoKV page prints in Table 11.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import Segment, attend, attend_lowdim, encode, lse_merge, reconstruct


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _segment(k, v, kc, vc, k_bits, v_bits, group, basis_k=None, basis_v=None, rng=None):
    from oracle import assign
    kid, _, _ = assign(k, kc)
    vid, _, _ = assign(v, vc)
    kcodes, kmeta = encode(k, kc, kid, k_bits, group, basis_k)
    vcodes, vmeta = encode(v, vc, vid, v_bits, group, basis_v)
    return Segment(kcodes, kmeta, kid, kc, vcodes, vmeta, vid, vc, k_bits, v_bits, group)


def _textbook(q, K, V):
    """Softmax attention with explicit loops: max pass, then exp-sum pass."""
    n_q, d = q.shape
    O = np.zeros((n_q, V.shape[1]))
    L = np.zeros(n_q)
    for i in range(n_q):
        logits = [float(np.dot(q[i], K[j])) / math.sqrt(d) for j in range(K.shape[0])]
        m = max(logits)
        w = [math.exp(t - m) for t in logits]
        tot = math.fsum(w)
        for j in range(K.shape[0]):
            O[i] += (w[j] / tot) * V[j]
        L[i] = m + math.log(tot)
    return O, L


def test_single_token_history():
    rng = np.random.default_rng(1)
    k = _bf16(rng.standard_normal((1, 64)))
    v = _bf16(rng.standard_normal((1, 64)))
    q = _bf16(rng.standard_normal((5, 64)))
    seg = _segment(k, v, k * 0.5, v * 0.25, 4, 2, 16)
    O, L = attend(q, [seg])
    kh = reconstruct(seg.k_codes, seg.k_meta, seg.k_ids, seg.k_cent, 4, 16)
    vh = reconstruct(seg.v_codes, seg.v_meta, seg.v_ids, seg.v_cent, 2, 16)
    assert np.allclose(O, np.repeat(vh, 5, 0), rtol=0, atol=1e-14)
    assert np.allclose(L, (q.astype(np.float64) @ kh[0]) / 8.0, rtol=0, atol=1e-12)


def test_identical_keys_average_values():
    rng = np.random.default_rng(2)
    N = 37
    k = np.repeat(_bf16(rng.standard_normal((1, 128))), N, 0)
    v = _bf16(rng.standard_normal((N, 128)) * 3)
    q = _bf16(rng.standard_normal((4, 128)))
    seg = _segment(k, v, k[:1], v[:8], 2, 4, 32)
    O, L = attend(q, [seg])
    kh = reconstruct(seg.k_codes, seg.k_meta, seg.k_ids, seg.k_cent, 2, 32)
    vh = reconstruct(seg.v_codes, seg.v_meta, seg.v_ids, seg.v_cent, 4, 32)
    assert np.allclose(O, vh.mean(0)[None, :], rtol=0, atol=1e-12)
    s = (q.astype(np.float64) @ kh[0]) / math.sqrt(128)
    assert np.allclose(L, s + math.log(N), rtol=0, atol=1e-12)


def test_sixteen_bit_zero_centre_is_textbook_attention():
    # bits = 16 with an all-zero centre stores the fp16 tokens themselves; for
    # fp16-representable K and V the reconstruction is exact.
    rng = np.random.default_rng(3)
    N, d = 90, 32
    k = rng.standard_normal((N, d)).astype(np.float16).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float16).astype(np.float32)
    q = rng.standard_normal((6, d)).astype(np.float32)
    z = np.zeros((1, d), np.float32)
    seg = _segment(k, v, z, z, 16, 16, d)
    O, L = attend(q, [seg])
    Ot, Lt = _textbook(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    assert np.max(np.abs(O - Ot)) < 1e-12 and np.max(np.abs(L - Lt)) < 1e-12


def test_merge_of_split_history_equals_unsplit():
    rng = np.random.default_rng(4)
    d = 64
    toks = [int(t) for t in (150, 1, 0, 77, 40)]
    segs = []
    for n in toks:
        k = _bf16(rng.standard_normal((n, d)))
        v = _bf16(rng.standard_normal((n, d)))
        kc = _bf16(rng.standard_normal((4, d)))
        vc = _bf16(rng.standard_normal((4, d)))
        segs.append(_segment(k, v, kc, vc, 2, 4, 16) if n else
                    Segment(np.zeros((0, 16), np.uint8), np.zeros((0, 4, 2), np.uint16),
                            np.zeros(0, np.int64), kc, np.zeros((0, 32), np.uint8),
                            np.zeros((0, 4, 2), np.uint16), np.zeros(0, np.int64), vc, 2, 4, 16))
    q = _bf16(rng.standard_normal((9, d)))
    O_all, L_all = attend(q, segs)
    parts = [attend(q, [s]) for s in segs]
    O_m, L_m = lse_merge([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(O_m - O_all)) < 1e-12 and np.max(np.abs(L_m - L_all)) < 1e-12
    # associativity: merge of merges
    a = lse_merge([parts[0][0], parts[1][0]], [parts[0][1], parts[1][1]])
    b = lse_merge([parts[2][0], parts[3][0], parts[4][0]], [parts[2][1], parts[3][1], parts[4][1]])
    O_ab, L_ab = lse_merge([a[0], b[0]], [a[1], b[1]])
    assert np.max(np.abs(O_ab - O_all)) < 1e-12 and np.max(np.abs(L_ab - L_all)) < 1e-12


def test_empty_history_and_empty_merge():
    q = np.ones((3, 64), np.float32)
    O, L = attend(q, [])
    assert not O.any() and np.all(np.isneginf(L))
    O2, L2 = lse_merge([O, O], [L, L])
    assert not O2.any() and np.all(np.isneginf(L2))


def test_lowdim_identity_basis_equals_full_dim():
    rng = np.random.default_rng(5)
    d, N = 64, 120
    k = _bf16(rng.standard_normal((N, d)))
    v = _bf16(rng.standard_normal((N, d)))
    kc, vc = k[:8].copy(), v[:8].copy()
    q = _bf16(rng.standard_normal((7, d)))
    I = np.eye(d, dtype=np.float32)
    full = _segment(k, v, kc, vc, 4, 4, 16)
    low = _segment(k, v, kc, vc, 4, 4, 16, I, I)
    assert np.array_equal(full.k_codes, low.k_codes) and np.array_equal(full.v_meta, low.v_meta)
    O1, L1 = attend(q, [full])
    O2, L2 = attend_lowdim(q, I, I, [low])
    assert np.max(np.abs(O1 - O2)) < 1e-12 and np.max(np.abs(L1 - L2)) < 1e-12


def test_lowdim_equals_full_attention_on_projected_reconstruction():
    rng = np.random.default_rng(6)
    d, r, N = 128, 32, 200
    k = _bf16(rng.standard_normal((N, d)))
    v = _bf16(rng.standard_normal((N, d)))
    kc, vc = k[:16].copy(), v[:16].copy()
    Uk = synth.orthonormal_basis(1, d, r, 1)[0].numpy()
    Uv = synth.orthonormal_basis(1, d, r, 2)[0].numpy()
    q = _bf16(rng.standard_normal((5, d)))
    seg = _segment(k, v, kc, vc, 2, 4, 16, Uk, Uv)
    O, L = attend_lowdim(q, Uk, Uv, [seg])
    kc_coef = reconstruct(seg.k_codes, seg.k_meta, seg.k_ids, kc, 2, 16, Uk)
    vc_coef = reconstruct(seg.v_codes, seg.v_meta, seg.v_ids, vc, 4, 16, Uv)
    Kf = kc_coef @ Uk.T.astype(np.float64)          # full-dim keys U (c' + a_hat)
    Vf = vc_coef @ Uv.T.astype(np.float64)
    Ot, Lt = _textbook(q.astype(np.float64), Kf, Vf)
    assert np.max(np.abs(O - Ot)) < 1e-11 and np.max(np.abs(L - Lt)) < 1e-11


def test_lowdim_exact_for_tokens_in_a_coordinate_subspace():
    # U = r distinct unit vectors: coefficients are exact copies of the chosen
    # channels; tokens living in those channels are read exactly (bits = 16).
    rng = np.random.default_rng(7)
    d, r, N = 64, 16, 60
    ch = rng.permutation(d)[:r]
    U = np.zeros((d, r), np.float32)
    U[ch, np.arange(r)] = 1.0
    k = np.zeros((N, d), np.float32)
    v = np.zeros((N, d), np.float32)
    k[:, ch] = rng.standard_normal((N, r)).astype(np.float16)
    v[:, ch] = rng.standard_normal((N, r)).astype(np.float16)
    z = np.zeros((1, d), np.float32)
    q = rng.standard_normal((4, d)).astype(np.float32)
    seg = _segment(k, v, z, z, 16, 16, r, U, U)
    O, L = attend_lowdim(q, U, U, [seg])
    Ot, Lt = _textbook(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    assert np.max(np.abs(O - Ot)) < 1e-12 and np.max(np.abs(L - Lt)) < 1e-12


def test_mac_saving_identity(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "nanokv_table11.json")))
    for row in g["rows"]:
        prod = row["historical_share"] * row["history_saved"]
        assert abs(prod - row["all_saved"]) <= 1.5 * 10 ** -g["printed_decimals"]
    # the same accounting for the larger-backbone workload: 28080 of 32760
    # history tokens read at rank 32 of 128 save (1 - 32/128) of their MACs
    cfg = synth.get_config("larger_backbone")
    share = cfg.far / cfg.hist
    saved_within = 1 - cfg.rank / cfg.dim
    assert share * saved_within == pytest.approx(0.6429, abs=1e-4)
