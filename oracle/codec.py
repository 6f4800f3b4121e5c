"""Centre fitting, nearest-centre assignment and the residual codec (one head).

What is computed, in the pages' terms:

* assign -- every token goes to its nearest centre in squared L2 distance
  (QuantWM, section 4.1, describing the centroid-residual scheme of QVG).
* fit -- Lloyd's k-means: assign, move each centre to the mean of its members,
  repeat; two iterations by default (NanoKV, Table 4: "two K-means iterations";
  centres per head, separately for K and V).
* encode -- the residual against the assigned centre (TempoKV, section 3.3,
  Eq. 2, with the centre as the prediction) is quantized per group of g
  channels by the affine min/max quantizer of TempoKV section 3.1, Eq. 1, then
  packed.  Readings of what the page leaves open (each also listed in the
  design notes):
    - zero-point: the group minimum stored as fp16 rounded toward -inf, a real
      offset, so a code q reconstructs to q*s + z (same grid family as Eq. 1);
    - scale: (max - z) / (2^b - 1) in fp32, then fp16 rounded toward +inf;
    - zero scale or zero-point values are stored as +0;
    - per element: t = (r - z) * (1/s) with one fp32 division per group, no
      fused multiply-add, q = clamp(round-half-even(t), 0, 2^b - 1);
    - a zero scale (all-equal group) stores q = 0;
    - packing: row-major per token, channel c of a row at bit b*(c mod 8/b) of
      byte c // (8/b), least significant bits first; metadata per group is the
      fp16 pair (scale, zero) in that order.
  The low-dimensional variant (NanoKV, Figure 4: coefficients of the residual
  in a reduced basis) first projects the fp32 residual on an orthonormal basis
  U (d x r): a_k = sum over i = 0..d-1, ascending, of fl32(U[i,k] * r[i]),
  accumulated in fp32 from +0 with a separate multiply and add.
* dequant -- r_hat = q*s + z, exact in fp64; reconstruct adds the centre back
  (Eq. 2) or, for coefficients, the projected centre U^T c.
"""
from __future__ import annotations

import numpy as np

from .numerics import f16_bits, f16_from_bits, fp16_round, round_to_storage


# ----------------------------------------------------------------------------- assignment
def assign(x, cent, chunk: int = 128):
    """Nearest centre of each token by the plain definition.

    D[j, c] = sum_i (x[j, i] - cent[c, i])^2 in fp64 from the stored values;
    id_j = argmin_c D[j, c], ties to the lowest index.  Returns (ids, D1, D2):
    the ids (int64) and the smallest and second-smallest distances per token
    (D2 = +inf when there is a single centre).
    """
    x64 = np.asarray(x, dtype=np.float64)
    c64 = np.asarray(cent, dtype=np.float64)
    N, C = x64.shape[0], c64.shape[0]
    ids = np.empty(N, dtype=np.int64)
    d1 = np.empty(N, dtype=np.float64)
    d2 = np.full(N, np.inf, dtype=np.float64)
    for s in range(0, N, chunk):
        diff = x64[s:s + chunk, None, :] - c64[None, :, :]
        D = (diff * diff).sum(axis=-1)
        ids[s:s + chunk] = np.argmin(D, axis=1)  # first occurrence of the minimum
        if C > 1:
            part = np.partition(D, 1, axis=1)
            d1[s:s + chunk] = part[:, 0]
            d2[s:s + chunk] = part[:, 1]
        else:
            d1[s:s + chunk] = D[:, 0]
    return ids, d1, d2


def objective(x, cent, ids) -> float:
    """k-means objective sum_j ||x_j - c_{id_j}||^2 in fp64."""
    diff = np.asarray(x, np.float64) - np.asarray(cent, np.float64)[ids]
    return float((diff * diff).sum())


def fit(x, init, n_iter: int = 2, storage: str = "bf16", history: bool = False):
    """Lloyd's k-means from the given initial centres.

    Each iteration: ids = assign(x, centres); every centre with members becomes
    the fp64 mean of its members (sum, then one division by the count), rounded
    to nearest-even in the storage dtype; a centre without members keeps its
    value.  After the last iteration a final assignment gives the ids.
    Returns (centres float32, ids) or, with history=True, also the list of
    (centres, ids) after every assignment.
    """
    x = np.asarray(x, dtype=np.float32)
    cent = np.array(init, dtype=np.float32, copy=True)
    C = cent.shape[0]
    hist = []
    for _ in range(n_iter):
        ids, _, _ = assign(x, cent)
        hist.append((cent.copy(), ids.copy()))
        counts = np.bincount(ids, minlength=C)
        for c in np.nonzero(counts)[0]:
            members = x[ids == c].astype(np.float64)
            cent[c] = round_to_storage(members.sum(axis=0) / counts[c], storage)
    ids, _, _ = assign(x, cent)
    hist.append((cent.copy(), ids.copy()))
    if history:
        return cent, ids, hist
    return cent, ids


# ----------------------------------------------------------------------------- codec
def _check_shapes(code_dim: int, bits: int, group: int):
    if bits not in (2, 4, 16):
        raise ValueError("bits must be 2, 4 or 16")
    if bits != 16 and (group <= 0 or code_dim % group):
        raise ValueError("group must divide the coded dimension")
    if bits != 16 and code_dim % (8 // bits):
        raise ValueError("coded dimension must fill whole bytes")


def residual(x, cent, ids, basis=None) -> np.ndarray:
    """fp32 residual r = fl32(x - c[id]), or its fp32 coefficients U^T r."""
    x32 = np.asarray(x, dtype=np.float32)
    c32 = np.asarray(cent, dtype=np.float32)
    r = x32 - c32[np.asarray(ids)]
    if basis is None:
        return r
    U = np.asarray(basis, dtype=np.float32)
    a = np.zeros((r.shape[0], U.shape[1]), dtype=np.float32)
    for i in range(U.shape[0]):                 # ascending channel order
        a = a + U[i][None, :] * r[:, i:i + 1]    # fp32 multiply, then fp32 add
    return a


def encode(x, cent, ids, bits: int, group: int, basis=None):
    """Encode one head's tokens.  Returns (codes uint8 [N, code_dim*bits/8],
    meta uint16 [N, code_dim/group, 2] holding fp16 bits (scale, zero)).
    bits=16 stores the fp16 (nearest-even) residual per element and no meta."""
    r = residual(x, cent, ids, basis)
    N, code_dim = r.shape
    _check_shapes(code_dim, bits, group)
    if not np.all(np.isfinite(r)):
        raise ValueError("non-finite residual")
    if bits == 16:
        h = fp16_round(r, "nearest")
        return f16_bits(h).view(np.uint8).reshape(N, code_dim * 2).copy(), None
    ng = code_dim // group
    rg = r.reshape(N, ng, group)
    mn = rg.min(axis=-1)
    mx = rg.max(axis=-1)
    z16 = fp16_round(mn, "down")
    z16[z16 == 0] = np.float16(0.0)             # a zero offset is stored as +0
    z32 = z16.astype(np.float32)
    levels = np.float32(2 ** bits - 1)
    s32 = (mx - z32) / levels
    s16 = fp16_round(s32, "up")
    s16[s16 == 0] = np.float16(0.0)
    sf = s16.astype(np.float32)
    nz = sf != 0
    inv = np.zeros_like(sf)
    inv[nz] = np.float32(1.0) / sf[nz]
    t = (rg - z32[..., None]) * inv[..., None]
    q = np.clip(np.rint(t), np.float32(0), levels)
    q[~nz] = 0
    q = q.astype(np.uint8).reshape(N, code_dim)
    per = 8 // bits
    qb = q.reshape(N, code_dim // per, per).astype(np.uint16)
    packed = np.zeros((N, code_dim // per), dtype=np.uint16)
    for k in range(per):
        packed |= qb[:, :, k] << (bits * k)
    meta = np.stack([f16_bits(s16), f16_bits(z16)], axis=-1)
    return packed.astype(np.uint8), meta


def unpack(codes, bits: int, code_dim: int) -> np.ndarray:
    """Integer codes [N, code_dim] from packed bytes (inverse of the packing)."""
    codes = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    mask = (1 << bits) - 1
    parts = [(codes >> (bits * k)) & mask for k in range(per)]
    return np.stack(parts, axis=-1).reshape(codes.shape[0], code_dim)


def dequant(codes, meta, bits: int, group: int, code_dim: int) -> np.ndarray:
    """r_hat = q*s + z per element, exact in fp64 (fp16 residuals for bits=16)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N = codes.shape[0]
    if bits == 16:
        return f16_from_bits(codes.view(np.uint16).reshape(N, code_dim)).astype(np.float64)
    q = unpack(codes, bits, code_dim).astype(np.float64)
    s = f16_from_bits(meta[..., 0]).astype(np.float64)
    z = f16_from_bits(meta[..., 1]).astype(np.float64)
    ng = code_dim // group
    rh = q.reshape(N, ng, group) * s[..., None] + z[..., None]
    return rh.reshape(N, code_dim)


def reconstruct(codes, meta, ids, cent, bits: int, group: int, basis=None) -> np.ndarray:
    """Reconstructed tokens in fp64: c[id] + r_hat (full dimension), or, with a
    basis U, coefficients U^T c[id] + a_hat (reduced dimension)."""
    c64 = np.asarray(cent, dtype=np.float64)
    if basis is not None:
        c64 = c64 @ np.asarray(basis, dtype=np.float64)
    code_dim = c64.shape[1]
    return c64[np.asarray(ids)] + dequant(codes, meta, bits, group, code_dim)


# ----------------------------------------------------------------------------- storage
def storage_bits_per_value(bits: int, group: int, meta_bits: int = 32) -> float:
    """Bits per stored element: the code plus the group's (scale, zero) share."""
    return bits + meta_bits / group


def storage_bytes(tokens: int, dim: int, k_bits: int, v_bits: int, group: int,
                  n_centroids: int = 0, code_dim: int | None = None,
                  centre_bytes: int = 2, id_bytes: int = 1) -> dict:
    """Bytes of one head's compressed K and V for ``tokens`` tokens.

    codes + fp16 (scale, zero) per group + one id per token and tensor, plus a
    centre table of C x dim per tensor when C > 0."""
    cd = dim if code_dim is None else code_dim
    codes = tokens * cd * (k_bits + v_bits) // 8
    meta = tokens * 2 * (cd // group) * 4
    ids = tokens * 2 * id_bytes if n_centroids > 0 else 0
    centres = 2 * n_centroids * dim * centre_bytes
    return {"codes": codes, "meta": meta, "ids": ids, "centres": centres,
            "total": codes + meta + ids + centres}
