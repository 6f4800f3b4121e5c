"""Pins of the predictive residual codec (oracle/tempo.py, TempoKV section 3.3,
Eqs. 2-4, anchor frames; Eq. 5 calibration) against what the pages and the
mathematics fix, independent of the oracle's own formulas:

* with every predictor coefficient zero, each frame is coded as plain group
  quantization of the frame itself (the codec of codec.encode with a zero
  centre) -- this is also exactly the anchor frame's coding;
* on a static scene with identity predictors, the reconstruction error shrinks
  by at least the quantizer's factor 1/(2^b - 1) every frame (the prediction
  must use the reconstructed history, not the true one);
* the first frame after the anchor uses its own coefficient set (o = 1 < h_K);
* the value prediction maps K_hat through W, not W^T;
* decoding from the codes alone reproduces the encoder's reconstruction bit for
  bit, however the frames are split over calls (the carried state);
* the ridge solution of Eq. 5 on a hand-worked 3 x 2 system, and recovery of
  planted temporal and cross predictors by the calibration."""
import numpy as np
import pytest

import oracle
from oracle import tempo

D, S, G = 32, 40, 16


def _zero_params(d=D):
    return np.zeros(tempo.n_params(d), np.float32)


def _params(d=D, **kw):
    base = dict(beta_k1=np.zeros(d), a_k1=np.zeros(d), beta_k2=np.zeros(d), a_k21=np.zeros(d), a_k22=np.zeros(d),
                beta_v=np.zeros(d), a_v=np.zeros(d), w=np.zeros((d, d)))
    base.update(kw)
    return tempo.join_params(**base)


def _frames(T, seed, scale=1.0, d=D):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((T * S, d))).astype(np.float32)


def _encode_all(k, v, p, kb, vb, splits=None, d=D):
    """Anchor, then the remaining frames in the given call sizes."""
    T = k.shape[0] // S
    ba = tempo.anchor_bits(kb, vb)
    res = [tempo.encode_frames(k[:S], v[:S], p, 0, S, ba, ba, G)]
    state = res[0][6]
    f = 1
    for n in (splits or [T - 1]):
        r = tempo.encode_frames(k[f * S:(f + n) * S], v[f * S:(f + n) * S], p, f, S, kb, vb, G, state)
        res.append(r)
        state = r[6]
        f += n
    return res


def test_zero_predictor_is_plain_group_quantization():
    T, kb, vb = 4, 2, 4
    k, v = _frames(T, 1), _frames(T, 2)
    res = _encode_all(k, v, _zero_params(), kb, vb)
    zc = np.zeros((1, D), np.float32)
    ids = np.zeros(S, np.int64)
    ba = tempo.anchor_bits(kb, vb)
    assert ba == 4
    # anchor: frame 0 at b_a, no prediction
    ck, mk = oracle.encode(k[:S], zc, ids, ba, G)
    cv, mv = oracle.encode(v[:S], zc, ids, ba, G)
    assert np.array_equal(res[0][0], ck) and np.array_equal(res[0][1], mk)
    assert np.array_equal(res[0][2], cv) and np.array_equal(res[0][3], mv)
    # frames 1..T-1 with zero predictions: plain quantization of each frame
    ck, mk = oracle.encode(k[S:], np.zeros((1, D), np.float32), np.zeros((T - 1) * S, np.int64), kb, G)
    cv, mv = oracle.encode(v[S:], np.zeros((1, D), np.float32), np.zeros((T - 1) * S, np.int64), vb, G)
    assert np.array_equal(res[1][0], ck) and np.array_equal(res[1][1], mk)
    assert np.array_equal(res[1][2], cv) and np.array_equal(res[1][3], mv)
    # and the reconstruction is the plain dequantization (rounded once to fp32)
    want = oracle.dequant(ck, mk, kb, G, D).astype(np.float32)
    assert np.array_equal(res[1][4], want)


@pytest.mark.parametrize("bits", [2, 4])
def test_static_scene_error_contracts_every_frame(bits):
    # K_t = K_0 and V_t = V_0; identity predictors in time (W = 0).  The residual
    # of frame t is the previous frame's reconstruction error e_{t-1}, so
    # |e_t| <= s_t / 2 with s_t ~ range(e_{t-1}) / (2^b - 1): a contraction.
    T = 7
    k0, v0 = _frames(1, 3, scale=3.0), _frames(1, 4, scale=3.0)
    k, v = np.tile(k0, (T, 1)), np.tile(v0, (T, 1))
    one = np.ones(D)
    p = _params(a_k1=one, a_k21=one, a_v=one)
    res = _encode_all(k, v, p, bits, bits, splits=[2, 4])
    kh = np.concatenate([r[4] for r in res]).reshape(T, S, D)
    vh = np.concatenate([r[5] for r in res]).reshape(T, S, D)
    shrink = 1.0 / (2 ** bits - 1) * 1.01
    for xh, x0 in ((kh, k0), (vh, v0)):
        err = np.abs(xh - x0[None]).max(axis=(1, 2))
        assert err[0] > 1e-3
        for t in range(1, T):
            assert err[t] <= err[t - 1] * shrink + 1e-6, (t, err)


def test_first_frame_after_anchor_has_its_own_coefficients():
    T = 3
    k0 = _frames(1, 5, scale=4.0)
    k = np.tile(k0, (T, 1))
    v = np.zeros_like(k)
    one, zero = np.ones(D), np.zeros(D)
    scale = lambda res: [oracle.f16_from_bits(r[1][..., 0]).max() for r in res]   # noqa: E731
    # set 1 = identity, set 2 = zero: frame 1 codes only the anchor's error,
    # frame 2 the whole key
    r1 = _encode_all(k, v, _params(a_k1=one), 4, 4, splits=[1, 1])
    s1 = scale(r1)
    assert s1[1] < 0.1 * s1[2]
    # set 1 = zero, set 2 = identity on K_hat[t-1]: the reverse
    r2 = _encode_all(k, v, _params(a_k21=one), 4, 4, splits=[1, 1])
    s2 = scale(r2)
    assert s2[2] < 0.1 * s2[1]
    # set 2's second lag reads K_hat[t-2]: a_k22 = 1 predicts frame 2 from frame 0
    r3 = _encode_all(k, v, _params(a_k22=one), 4, 4, splits=[1, 1])
    s3 = scale(r3)
    assert s3[2] < 0.1 * s3[1]
    # and the biases enter: beta_k1 = k0's mean per channel moves frame 1's residual
    r4 = _encode_all(k, v, _params(beta_k1=k0.mean(axis=0)), 4, 4, splits=[1, 1])
    assert scale(r4)[1] < scale(r1)[2]


def test_value_prediction_maps_keys_through_w_not_its_transpose():
    T = 3
    rng = np.random.default_rng(6)
    W0 = np.triu(rng.standard_normal((D, D))).astype(np.float32)   # far from symmetric
    k = _frames(T, 7)
    v = (k.astype(np.float64) @ W0.T.astype(np.float64)).astype(np.float32)   # V = W0 K
    vs = lambda p: max(oracle.f16_from_bits(r[3][..., 0]).max() for r in _encode_all(k, v, p, 4, 4)[1:])  # noqa: E731
    good = vs(_params(w=W0))
    bad = vs(_params(w=W0.T))
    none = vs(_params())
    assert good < 0.25 * none and bad > 0.5 * none


def test_decode_reproduces_the_encoder_across_call_splits():
    T, kb, vb = 6, 2, 4
    rng = np.random.default_rng(8)
    k, v = _frames(T, 9), _frames(T, 10)
    p = _params(beta_k1=0.1 * rng.standard_normal(D), a_k1=0.9 + 0.05 * rng.standard_normal(D),
                beta_k2=0.1 * rng.standard_normal(D), a_k21=0.6 * np.ones(D), a_k22=0.3 * np.ones(D),
                beta_v=0.1 * rng.standard_normal(D), a_v=0.5 * np.ones(D), w=0.1 * rng.standard_normal((D, D)))
    enc = _encode_all(k, v, p, kb, vb, splits=[2, 3])
    one = _encode_all(k, v, p, kb, vb, splits=[5])
    kh_split = np.concatenate([r[4] for r in enc])
    kh_one = np.concatenate([r[4] for r in one])
    assert np.array_equal(kh_split, kh_one)
    # codes of the split encode equal the single call's
    assert np.array_equal(np.concatenate([r[0] for r in enc[1:]]), one[1][0])
    assert np.array_equal(np.concatenate([r[3] for r in enc[1:]]), one[1][3])
    # decode from codes only, in yet another split
    ba = tempo.anchor_bits(kb, vb)
    d0 = tempo.decode_frames(enc[0][0], enc[0][1], enc[0][2], enc[0][3], p, 0, S, ba, ba, G, D)
    codes = [np.concatenate([r[i] for r in enc[1:]]) for i in range(4)]
    d1 = tempo.decode_frames(*[c[:S] for c in codes], p, 1, S, kb, vb, G, D, d0[2])
    d2 = tempo.decode_frames(*[c[S:] for c in codes], p, 2, S, kb, vb, G, D, d1[2])
    assert np.array_equal(np.concatenate([d0[0], d1[0], d2[0]]), kh_one)
    assert np.array_equal(np.concatenate([d0[1], d1[1], d2[1]]), np.concatenate([r[5] for r in one]))


def test_ridge_hand_worked():
    # y = [2, 3, 5] on x = [1, 2, 3] with an intercept.  lambda = 0: slope 3/2,
    # intercept 1/3.  lambda = 1: (Z^T Z + I) = [[15, 6], [6, 4]], Z^T y = [23, 10],
    # det 24: slope (4*23 - 6*10)/24 = 4/3, intercept (15*10 - 6*23)/24 = 1/2.
    Z = np.array([[1.0, 1.0], [2.0, 1.0], [3.0, 1.0]])
    y = np.array([2.0, 3.0, 5.0])
    assert np.allclose(tempo._ridge(Z, y, 0.0), [1.5, 1.0 / 3.0], rtol=0, atol=1e-12)
    assert np.allclose(tempo._ridge(Z, y, 1.0), [4.0 / 3.0, 0.5], rtol=0, atol=1e-12)


def test_calibration_recovers_planted_predictors():
    rng = np.random.default_rng(11)
    T, Sx = 8, 400
    a1 = rng.uniform(0.5, 0.8, D)
    a2 = rng.uniform(0.0, 0.3, D)
    b = rng.uniform(-0.2, 0.2, D)
    W0 = (rng.standard_normal((D, D)) / np.sqrt(D)).astype(np.float64)
    av = rng.uniform(0.2, 0.5, D)
    bv = rng.uniform(-0.2, 0.2, D)
    sig = 0.05
    k = np.zeros((T, Sx, D))
    v = np.zeros((T, Sx, D))
    k[0] = rng.standard_normal((Sx, D))
    k[1] = rng.standard_normal((Sx, D))
    v[0] = rng.standard_normal((Sx, D))
    for t in range(1, T):
        if t >= 2:
            k[t] = b + a1 * k[t - 1] + a2 * k[t - 2] + sig * rng.standard_normal((Sx, D))
        v[t] = bv + k[t] @ W0.T + av * v[t - 1] + sig * rng.standard_normal((Sx, D))
    p = tempo.calibrate(k.reshape(-1, D).astype(np.float32), v.reshape(-1, D).astype(np.float32), Sx, 4, 4, G,
                        lam=1.0)
    prm = tempo.split_params(p, D)
    # 4-bit inputs add ~2% noise to the regressors (a small attenuation)
    assert np.abs(prm["a_k21"] - a1).max() < 0.06 and np.abs(prm["a_k22"] - a2).max() < 0.06
    assert np.abs(prm["beta_k2"] - b).max() < 0.06
    assert np.abs(prm["w"] - W0).max() < 0.06
    assert np.abs(prm["a_v"] - av).max() < 0.06
