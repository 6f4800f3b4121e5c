"""Pins of the oracle's assignment, fitting and residual codec.

Each test checks the oracle against something other than itself: hand-derived
groups of the TempoKV quantizer (section 3.1, Eq. 1), the quantizer formula
evaluated in exact rational arithmetic, brute-force assignment over Fractions,
the RTN compression ratios the TempoKV tables print, the BF16 cache size
formula of the Coral-KV summary, and invariants of Lloyd's algorithm.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (assign, dequant, encode, fit, objective, reconstruct,
                    storage_bits_per_value, storage_bytes)
from oracle.codec import residual, unpack
from oracle.numerics import f16_from_bits


def _meta_vals(meta):
    return (f16_from_bits(meta[..., 0]).astype(np.float64),
            f16_from_bits(meta[..., 1]).astype(np.float64))


# ----------------------------------------------------------------------------- quantizer
def test_quantizer_hand_derived_groups(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "quantizer_eq1.json")))["cases"]
    for case in cases:
        r = np.array([case["r"]], np.float32)
        zero_c = np.zeros((1, r.shape[1]), np.float32)
        codes, meta = encode(r, zero_c, np.array([0]), case["bits"], r.shape[1])
        q = unpack(codes, case["bits"], r.shape[1])[0]
        s, z = _meta_vals(meta)
        assert list(q) == case["q"], case
        assert s[0, 0] == case["scale"] and z[0, 0] == case["zero"], case
        assert np.signbit(s[0, 0]) == 0 and (z[0, 0] != 0 or np.signbit(z[0, 0]) == 0)


def _eq1_codes(group_vals, bits):
    """Eq. 1 evaluated exactly: Q = round(X/s) + z with s = (max-min)/(2^b-1) and
    z = round(-min/s), round = nearest with ties to even (Fractions)."""
    X = [Fraction(float(v)) for v in group_vals]
    mn, mx = min(X), max(X)
    s = (mx - mn) / (2 ** bits - 1)
    def rne(f):
        fl = f.numerator // f.denominator
        rem = f - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
            return fl + 1
        return fl
    z = rne(-mn / s)
    return [rne(x / s) + z for x in X]


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_equal_eq1_on_grid_aligned_groups(bits):
    # Groups whose minimum is a multiple of the scale and whose values are
    # exact in fp16: there Eq. 1's integer zero-point is exact, and the stored
    # codes must equal Eq. 1's codes.  Exact half-way values are left out: Eq. 1
    # breaks such a tie by the parity of X/s, this codec by the parity of the
    # code (X - z)/s; the two differ when the zero-point is odd.  The codec's
    # own tie rule is pinned by the hand-derived groups above.
    rng = np.random.default_rng(11)
    g, n = 16, 400
    L = 2 ** bits - 1
    s = (2.0 ** rng.integers(-6, 3, n)).astype(np.float32)          # power-of-two scales
    k0 = rng.integers(-40, 40, n)                                    # min = k0 * s
    frac = rng.integers(0, 4 * L + 1, (n, g))
    frac = np.where(frac % 4 == 2, frac + 1, frac) / 4.0             # quarter steps, no ties
    frac[:, 0] = 0.0
    frac[:, 1] = L
    r = ((k0[:, None] + frac) * s[:, None]).astype(np.float32)
    codes, meta = encode(r.reshape(n, g), np.zeros((1, g), np.float32), np.zeros(n, np.int64), bits, g)
    q = unpack(codes, bits, g)
    for j in range(n):
        eq1 = _eq1_codes(r[j], bits)
        # Eq. 1's code of the minimum is 0; both grids start at the minimum
        assert eq1[0] == 0 and list(q[j]) == eq1


def _random_tokens(n, d, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, d)) * scale).astype(np.float32)
    x[:, :4] *= 8.0
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("bits,group", [(2, 16), (4, 32), (2, 32), (4, 16)])
def test_dequant_error_within_half_scale(bits, group):
    x = _random_tokens(3000, 128, bits * 100 + group)
    cent = x[:16] * 0.5
    ids = np.arange(3000) % 16
    codes, meta = encode(x, cent, ids, bits, group)
    r = residual(x, cent, ids).astype(np.float64)
    rh = dequant(codes, meta, bits, group, 128)
    s, z = _meta_vals(meta)
    bound = np.repeat(s, group, axis=1) / 2 * (1 + 2.0 ** -16)
    assert np.all(np.abs(r - rh) <= bound)
    # the group minimum always takes code 0
    q = unpack(codes, bits, 128).reshape(3000, 128 // group, group)
    rg = r.reshape(3000, 128 // group, group)
    amin = rg.argmin(axis=-1)
    assert np.all(np.take_along_axis(q, amin[..., None], -1) == 0)
    # zero-point is the group minimum rounded down to fp16; scale covers the range
    assert np.all(z <= rg.min(-1))
    span = rg.max(-1) - z
    assert np.all(z + (2 ** bits - 1) * s >= rg.max(-1) - 2.0 ** -22 * span)


def test_token_equal_to_centre_encodes_to_zero():
    x = _random_tokens(64, 128, 5)
    codes, meta = encode(x, x, np.arange(64), 2, 16)
    assert not codes.any()
    assert not meta.any()                       # scale = zero = +0 (all bits zero)
    assert np.array_equal(reconstruct(codes, meta, np.arange(64), x, 2, 16), x.astype(np.float64))


def test_packing_bit_positions():
    # a single nonzero channel c lands at bit b*(c mod 8/b) of byte c // (8/b)
    for bits in (2, 4):
        per = 8 // bits
        for c in range(0, 32, 3):
            r = np.zeros((1, 32), np.float32)
            r[0, c] = 1.0
            codes, meta = encode(r, np.zeros((1, 32), np.float32), np.array([0]), bits, 32)
            expect = np.zeros(32 * bits // 8, np.uint8)
            expect[c // per] = (2 ** bits - 1) << (bits * (c % per))
            assert np.array_equal(codes[0], expect), (bits, c)


def test_sixteen_bit_mode_stores_fp16_residual():
    x = _random_tokens(50, 64, 9)
    cent = x[:4]
    ids = np.arange(50) % 4
    codes, meta = encode(x, cent, ids, 16, 64)
    assert meta is None
    rh = dequant(codes, None, 16, 64, 64)
    r = residual(x, cent, ids)
    assert np.array_equal(rh, r.astype(np.float16).astype(np.float64))


def test_rtn_compression_ratios(golden_dir):
    # RTN is the codec with one all-zero centre and no ids; its storage per
    # value is the code plus the group's 32 metadata bits (TempoKV Tables 1-2).
    g = json.load(open(os.path.join(golden_dir, "rtn_compression.json")))
    for b, ratio in g["ratios"].items():
        got = 16.0 / storage_bits_per_value(int(b), g["group"])
        assert round(got, g["printed_decimals"]) == pytest.approx(ratio, abs=1e-9)


def test_bf16_cache_bytes_formula(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "coral_bf16_cache.json")))
    for c in g["cases"]:
        heads = c["width"] // 128
        per_head = 2 * c["tokens"] * 128 * 2
        assert c["layers"] * heads * per_head == c["bytes"]


def test_storage_bytes_accounting():
    sb = storage_bytes(9360, 128, 2, 2, 16, n_centroids=256)
    assert sb["codes"] == 9360 * 64
    assert sb["meta"] == 9360 * 2 * 8 * 4
    assert sb["ids"] == 9360 * 2
    assert sb["centres"] == 2 * 256 * 128 * 2
    bf16 = 2 * 9360 * 128 * 2
    assert bf16 / (sb["codes"] + sb["meta"] + sb["ids"]) == pytest.approx(3.9, abs=0.05)


# ----------------------------------------------------------------------------- low-dim codes
def test_identity_basis_gives_full_dim_codes():
    x = _random_tokens(300, 128, 21)
    cent = x[:8] * 0.25
    ids = np.arange(300) % 8
    I = np.eye(128, dtype=np.float32)
    c_full = encode(x, cent, ids, 4, 16)
    c_low = encode(x, cent, ids, 4, 16, basis=I)
    assert np.array_equal(c_full[0], c_low[0]) and np.array_equal(c_full[1], c_low[1])


def test_coefficients_close_to_exact_projection():
    x = _random_tokens(200, 128, 22)
    cent = x[:4] * 0.5
    ids = np.arange(200) % 4
    U = synth.orthonormal_basis(1, 128, 32, 7)[0].numpy()
    a = residual(x, cent, ids, U).astype(np.float64)
    r = residual(x, cent, ids).astype(np.float64)
    exact = r @ U.astype(np.float64)
    # sequential fp32 accumulation of 128 products: |error| <= 2*128*u*sum|U r|
    bound = 2 * 128 * 2.0 ** -24 * (np.abs(r) @ np.abs(U.astype(np.float64)))
    assert np.all(np.abs(a - exact) <= bound)


# ----------------------------------------------------------------------------- assignment
def _brute_assign(x, c):
    xs = [[Fraction(float(v)) for v in row] for row in x]
    cs = [[Fraction(float(v)) for v in row] for row in c]
    ids = []
    for row in xs:
        best, bi = None, -1
        for k, cr in enumerate(cs):
            D = sum((a - b) ** 2 for a, b in zip(row, cr))
            if best is None or D < best:
                best, bi = D, k
        ids.append(bi)
    return np.array(ids)


def test_assign_matches_exact_brute_force_with_planted_ties():
    rng = np.random.default_rng(31)
    for trial in range(4):
        d = int(rng.integers(2, 9))
        C = int(rng.integers(4, 17))
        N = 150
        c = (rng.integers(-8, 9, (C, d)) / 4.0).astype(np.float32)
        c[C - 1] = c[0]                          # duplicate centre: exact tie, lowest index wins
        x = (rng.integers(-8, 9, (N, d)) / 4.0).astype(np.float32)
        x[:20] = ((c[1] + c[2]) / 2)             # equidistant from centres 1 and 2
        x[20:40] = rng.standard_normal((20, d)).astype(np.float32)
        ids, d1, d2 = assign(x, c)
        assert np.array_equal(ids, _brute_assign(x, c))
        assert np.all(d1 <= d2)


def test_assign_distances_match_definition():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((50, 16)).astype(np.float32)
    c = rng.standard_normal((7, 16)).astype(np.float32)
    ids, d1, d2 = assign(x, c)
    for j in range(50):
        D = sorted(sum((float(a) - float(b)) ** 2 for a, b in zip(x[j], c[k])) for k in range(7))
        assert d1[j] == pytest.approx(D[0], rel=1e-12) and d2[j] == pytest.approx(D[1], rel=1e-12)


def test_assign_non_finite_token_takes_the_lowest_index():
    # a token with a NaN or an infinite channel has no finite distance to any
    # centre: the first minimum of such a row is index 0, so the id stays a valid
    # index into the centre table (the kernels map this case to 0 as well)
    rng = np.random.default_rng(33)
    c = rng.standard_normal((9, 8)).astype(np.float32)
    x = rng.standard_normal((5, 8)).astype(np.float32)
    x[1, 3] = np.nan
    x[2, 0] = np.inf
    x[3, :] = -np.inf
    with np.errstate(invalid="ignore"):
        ids, d1, d2 = assign(x, c)
    assert list(ids[1:4]) == [0, 0, 0]
    assert ids[0] == _brute_assign(x[:1], c)[0] and ids[4] == _brute_assign(x[4:], c)[0]
    assert all(0 <= i < len(c) for i in ids)


# ----------------------------------------------------------------------------- fitting
def test_fit_objective_never_increases():
    cfg = synth.get_config("self_forcing_layer")
    st = synth.AR1Stream(cfg, "k", heads=1)
    x = st.next_frames(1)[0, :1200].float().numpy()
    init = synth.forgy_init(torch.from_numpy(x)[None].to(torch.bfloat16), 32, 5)[0].float().numpy()
    cent, ids, hist = fit(x, init, n_iter=4, storage="bf16", history=True)
    objs = [objective(x, c, i) for c, i in hist]
    # after the mean update the objective with the old ids can only drop; a
    # bf16 rounding of the mean can raise it by at most a rounding amount
    for a, b in zip(objs, objs[1:]):
        assert b <= a * (1 + 1e-4)


def test_fit_recovers_generating_clusters_from_one_point_each():
    cfg = synth.get_config("tiny")
    x, labels = synth.tiny_kv(cfg, "k")
    init = synth.one_per_label_init(x, labels, cfg.n_centroids)[0].numpy()
    cent, ids = fit(x[0].numpy(), init, n_iter=2, storage="f32")
    assert np.array_equal(ids, labels[0].numpy())


def test_fit_update_rules():
    x = np.array([[1.0, 0.0], [1.0078125, 2.0], [10.0, 10.0], [-5.0, 3.0]], np.float32)
    init = np.array([[1.0, 1.0], [10.0, 10.0], [100.0, 100.0], [-5.0, 3.0]], np.float32)
    cent, ids = fit(x, init, n_iter=1, storage="bf16")
    # members {x0, x1}: mean (1 + 2^-8, 1.0): the tie rounds to the even bf16 1.0
    assert np.array_equal(cent[0], np.array([1.0, 1.0], np.float32))
    assert np.array_equal(cent[1], x[2])          # singleton keeps the point
    assert np.array_equal(cent[2], init[2])       # empty cluster keeps its centre
    assert np.array_equal(cent[3], x[3])
    assert list(ids) == [0, 0, 1, 3]
