"""Predictive residual coding of the KV cache over latent frames (TempoKV) and
the offline fit of its predictors.  TEST INFRASTRUCTURE ONLY (part of the
oracle package).

What is computed, in the pages' terms (TempoKV, arxiv 2610.15324):

* Frames t = 0, 1, ... of S spatial tokens each; a token keeps its spatial
  index s across frames (section 3.1).  Token index t*S + s.
* Eq. 2: each frame stores only the quantized residual against a prediction,
  R = X - X_tilde, and is reconstructed as X_hat = X_tilde + D(Q(R)).
* Eq. 3, keys: K_tilde[t,s] = beta_K + sum_{i=1..o} A_K[i] (.) K_hat[t-i,s], with
  o = min(t, h_K), h_K = 2, elementwise products; the first frame after the
  anchor (o = 1 < h_K) uses its own set of coefficients.
* Eq. 4, values: V_tilde[t,s] = beta_V + W K_hat[t,s] + A_V (.) V_hat[t-1,s]
  (h_V = 1, the key of the same frame and token through a dense D x D map).
* "Anchor frames": frame 0 is quantized without prediction (X_tilde = 0) at
  b_a = max(4, b_K, b_V) bits.
* Eq. 5, offline calibration: per head, ridge regression of the full-precision
  target on the reconstructed inputs, the key predictor first, then the value
  predictor on the keys the fitted key predictor reconstructs.

Readings of what the page leaves open (each also listed in the design notes):
  - the quantizer Q/D is this package's group quantizer (codec.encode with a
    zero centre: per group of g channels a real fp16 zero-point rounded down and
    an fp16 scale rounded up, round-half-even codes);
  - the arithmetic is fp32 with one fixed order, so that the codes are unique:
      k_tilde = ((beta + fl(A1*k1)) + fl(A2*k2))         (o = 2; o = 1 drops A2)
      v_tilde = acc + fl(A_V*v1), acc = beta_V, then acc += fl(W[c][j]*k_hat[j])
                for j = 0..D-1 ascending                   (multiply and add rounded
                                                            separately, no FMA)
      r = fl(x - x_tilde);  x_hat = fl(x_tilde + fl(q*s + z));
  - the calibration inputs: the key predictor's inputs are the keys of the
    earlier frames after plain quantization and reconstruction at b_K bits
    (the key history the codec reconstructs depends on the predictor being
    fitted); the value predictor's inputs are the keys the fitted key codec
    reconstructs and the previous frame's values after plain quantization at
    b_V bits; the ridge penalty covers every coefficient, the biases included;
    fp64 normal equations.

Parameter layout of one head (fp32, P = 7*D + D*D values), shared with the GPU
path as an interface: beta_K1, A_K1 (o = 1); beta_K2, A_K21, A_K22 (o = 2);
beta_V, A_V; W row-major (W[c][j] multiplies k_hat[j] for output channel c).
"""
from __future__ import annotations

import numpy as np

from .codec import dequant, encode as codec_encode

H_K, H_V = 2, 1


def n_params(dim: int) -> int:
    return 7 * dim + dim * dim


def split_params(p, dim: int) -> dict:
    """Named views of one head's flat parameter vector."""
    p = np.asarray(p, dtype=np.float32)
    if p.shape != (n_params(dim),):
        raise ValueError("parameter vector of the wrong length")
    D = dim
    names = ["beta_k1", "a_k1", "beta_k2", "a_k21", "a_k22", "beta_v", "a_v"]
    out = {n: p[i * D:(i + 1) * D] for i, n in enumerate(names)}
    out["w"] = p[7 * D:].reshape(D, D)
    return out


def join_params(beta_k1, a_k1, beta_k2, a_k21, a_k22, beta_v, a_v, w) -> np.ndarray:
    parts = [beta_k1, a_k1, beta_k2, a_k21, a_k22, beta_v, a_v, np.asarray(w).reshape(-1)]
    return np.concatenate([np.asarray(x, dtype=np.float32).reshape(-1) for x in parts])


def anchor_bits(k_bits: int, v_bits: int) -> int:
    """b_a = max(4, b_K, b_V) ("Anchor frames")."""
    return max(4, k_bits, v_bits)


# ----------------------------------------------------------------------------- predictions (fp32, fixed order)
def predict_key(k1, k2, prm: dict, o: int) -> np.ndarray:
    """Eq. 3 for the tokens of one frame: k1 = K_hat[t-1], k2 = K_hat[t-2] ([S, D]
    fp32), o = available history (1 or 2)."""
    f32 = np.float32
    k1 = np.asarray(k1, f32)
    if o == 1:
        return prm["beta_k1"][None, :] + prm["a_k1"][None, :] * k1
    k2 = np.asarray(k2, f32)
    return (prm["beta_k2"][None, :] + prm["a_k21"][None, :] * k1) + prm["a_k22"][None, :] * k2


def predict_value(khat, v1, prm: dict) -> np.ndarray:
    """Eq. 4 for the tokens of one frame: khat = K_hat[t], v1 = V_hat[t-1]."""
    f32 = np.float32
    khat = np.asarray(khat, f32)
    W = prm["w"]
    acc = np.broadcast_to(prm["beta_v"][None, :], khat.shape).astype(f32)
    for j in range(khat.shape[1]):                    # ascending input channel
        acc = acc + W[:, j][None, :] * khat[:, j:j + 1]
    return acc + prm["a_v"][None, :] * np.asarray(v1, f32)


# ----------------------------------------------------------------------------- quantize one frame
def _code_residual(r, bits: int, group: int):
    """Group quantization of fp32 residuals [S, D]: (codes, meta, r_hat fp32)."""
    r = np.asarray(r, np.float32)
    S, D = r.shape
    zero = np.zeros((1, D), np.float32)
    codes, meta = codec_encode(r, zero, np.zeros(S, np.int64), bits, group)
    rhat = dequant(codes, meta, bits, group, D).astype(np.float32)   # q*s is exact; one rounding of + z
    return codes, meta, rhat


# ----------------------------------------------------------------------------- encode / decode a run of frames
def encode_frames(k, v, params, first_frame: int, S: int, k_bits: int, v_bits: int, group: int, state=None):
    """Encode the frames first_frame, first_frame+1, ... of one head.

    k, v: [n_frames*S, D] (stored values); params: the head's flat vector;
    state: None for first_frame = 0, else (K_hat[f-1], K_hat[f-2], V_hat[f-1])
    as [S, D] fp32 (K_hat[f-2] unused when f = 1).  Frame 0 is the anchor: no
    prediction; the caller codes it alone, at anchor_bits(b_K, b_V).
    Returns (k_codes, k_meta, v_codes, v_meta, k_hat, v_hat, state_out)."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    D = k.shape[1]
    n_frames = k.shape[0] // S
    if n_frames * S != k.shape[0] or v.shape != k.shape:
        raise ValueError("tokens must be whole frames of S tokens, K and V alike")
    if first_frame == 0 and n_frames != 1:
        raise ValueError("the anchor frame is coded alone")
    prm = split_params(params, D)
    if first_frame > 0:
        k1, k2, v1 = (np.asarray(a, np.float32) for a in state)
    out = {n: [] for n in ("kc", "km", "vc", "vm", "kh", "vh")}
    for f in range(n_frames):
        t = first_frame + f
        xs = slice(f * S, (f + 1) * S)
        if t == 0:
            k_til = np.zeros((S, D), np.float32)
        else:
            k_til = predict_key(k1, k2, prm, min(t, H_K))
        kc, km, krh = _code_residual(k[xs] - k_til, k_bits, group)
        k_hat = k_til + krh
        if t == 0:
            v_til = np.zeros((S, D), np.float32)
        else:
            v_til = predict_value(k_hat, v1, prm)
        vc, vm, vrh = _code_residual(v[xs] - v_til, v_bits, group)
        v_hat = v_til + vrh
        for n, a in zip(("kc", "km", "vc", "vm", "kh", "vh"), (kc, km, vc, vm, k_hat, v_hat)):
            out[n].append(a)
        k2 = k1 if t > 0 else np.zeros((S, D), np.float32)
        k1, v1 = k_hat, v_hat
    cat = {n: np.concatenate(a, axis=0) for n, a in out.items()}
    return cat["kc"], cat["km"], cat["vc"], cat["vm"], cat["kh"], cat["vh"], (k1, k2, v1)


def decode_frames(k_codes, k_meta, v_codes, v_meta, params, first_frame: int, S: int, k_bits: int,
                  v_bits: int, group: int, dim: int, state=None):
    """Reconstruct the frames a call of encode_frames coded, from the codes and
    the state before them.  Returns (k_hat, v_hat, state_out), fp32."""
    prm = split_params(params, dim)
    n_frames = np.asarray(k_codes).shape[0] // S
    if first_frame > 0:
        k1, k2, v1 = (np.asarray(a, np.float32) for a in state)
    kh_all, vh_all = [], []
    for f in range(n_frames):
        t = first_frame + f
        xs = slice(f * S, (f + 1) * S)
        krh = dequant(k_codes[xs], k_meta[xs], k_bits, group, dim).astype(np.float32)
        vrh = dequant(v_codes[xs], v_meta[xs], v_bits, group, dim).astype(np.float32)
        k_til = np.zeros((S, dim), np.float32) if t == 0 else predict_key(k1, k2, prm, min(t, H_K))
        k_hat = k_til + krh
        v_til = np.zeros((S, dim), np.float32) if t == 0 else predict_value(k_hat, v1, prm)
        v_hat = v_til + vrh
        kh_all.append(k_hat)
        vh_all.append(v_hat)
        k2 = k1 if t > 0 else np.zeros((S, dim), np.float32)
        k1, v1 = k_hat, v_hat
    return np.concatenate(kh_all), np.concatenate(vh_all), (k1, k2, v1)


# ----------------------------------------------------------------------------- calibration (Eq. 5)
def _ridge(Z, y, lam: float) -> np.ndarray:
    """argmin ||y - Z theta||^2 + lam ||theta||^2 (fp64 normal equations)."""
    Z = np.asarray(Z, np.float64)
    G = Z.T @ Z + lam * np.eye(Z.shape[1])
    return np.linalg.solve(G, Z.T @ np.asarray(y, np.float64))


def _rtn(x, bits: int, group: int) -> np.ndarray:
    """Plain quantization and reconstruction of tokens [N, D] (fp32)."""
    return _code_residual(np.asarray(x, np.float32), bits, group)[2]


def calibrate(k, v, S: int, k_bits: int, v_bits: int, group: int, lam: float = 1.0) -> np.ndarray:
    """Fit one head's predictors on a full-precision trace k, v [T*S, D] (T >= 3
    frames).  Returns the flat parameter vector (fp32)."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    D = k.shape[1]
    T = k.shape[0] // S
    if T < 3:
        raise ValueError("calibration needs at least three frames")
    kf = k.reshape(T, S, D).astype(np.float64)
    vf = v.reshape(T, S, D).astype(np.float64)
    kq = _rtn(k, k_bits, group).reshape(T, S, D).astype(np.float64)
    beta_k1, a_k1 = np.empty(D), np.empty(D)
    beta_k2, a_k21, a_k22 = np.empty(D), np.empty(D), np.empty(D)
    for c in range(D):
        # o = 1: frame 1 from frame 0
        th = _ridge(np.stack([kq[0, :, c], np.ones(S)], axis=1), kf[1, :, c], lam)
        a_k1[c], beta_k1[c] = th
        # o = 2: frames t >= 2 from frames t-1, t-2
        z1 = kq[1:T - 1, :, c].reshape(-1)
        z2 = kq[0:T - 2, :, c].reshape(-1)
        th = _ridge(np.stack([z1, z2, np.ones_like(z1)], axis=1), kf[2:, :, c].reshape(-1), lam)
        a_k21[c], a_k22[c], beta_k2[c] = th
    zero_v = dict(beta_v=np.zeros(D), a_v=np.zeros(D), w=np.zeros((D, D)))
    pk = join_params(beta_k1, a_k1, beta_k2, a_k21, a_k22, zero_v["beta_v"], zero_v["a_v"], zero_v["w"])
    # the keys the fitted key codec reconstructs (values coded against zero meanwhile)
    _, _, _, _, kh0, _, st = encode_frames(k[:S], v[:S], pk, 0, S, anchor_bits(k_bits, v_bits),
                                           anchor_bits(k_bits, v_bits), group)
    _, _, _, _, kh1, _, _ = encode_frames(k[S:], v[S:], pk, 1, S, k_bits, v_bits, group, st)
    khat = np.concatenate([kh0, kh1]).reshape(T, S, D).astype(np.float64)
    vq = _rtn(v, v_bits, group).reshape(T, S, D).astype(np.float64)
    beta_v, a_v, W = np.empty(D), np.empty(D), np.empty((D, D))
    # output channel c: inputs [K_hat[t] (D columns), V_q[t-1, c], 1]; the Gram
    # blocks of the key columns are shared by every c
    Kin = khat[1:].reshape(-1, D)
    n = Kin.shape[0]
    KtK = Kin.T @ Kin
    Ks = Kin.sum(axis=0)
    for c in range(D):
        z = vq[:T - 1, :, c].reshape(-1)
        y = vf[1:, :, c].reshape(-1)
        G = np.empty((D + 2, D + 2))
        G[:D, :D] = KtK
        G[:D, D] = G[D, :D] = Kin.T @ z
        G[:D, D + 1] = G[D + 1, :D] = Ks
        G[D, D] = z @ z
        G[D, D + 1] = G[D + 1, D] = z.sum()
        G[D + 1, D + 1] = n
        rhs = np.concatenate([Kin.T @ y, [z @ y, y.sum()]])
        th = np.linalg.solve(G + lam * np.eye(D + 2), rhs)
        W[c], a_v[c], beta_v[c] = th[:D], th[D], th[D + 1]
    return join_params(beta_k1, a_k1, beta_k2, a_k21, a_k22, beta_v, a_v, W)
