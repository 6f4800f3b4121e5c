"""Shared helpers of the parity tests: move data between torch and numpy, build
oracle-encoded caches and upload them as GPU segments.  Every cache the GPU
attention reads in these tests is produced by the oracle (or drawn by the
generators), never by the HIP path."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synth


def np32(t: torch.Tensor) -> np.ndarray:
    """Values of a bf16/fp32 tensor as a float32 numpy array (exact)."""
    return t.detach().to("cpu").float().numpy()


def encode_heads(x, cent, ids, bits, group, basis=None):
    """Oracle encode of every head: codes [H, N, B], meta [H, N, G, 2]."""
    H = x.shape[0]
    codes, metas = [], []
    for h in range(H):
        c, m = oracle.encode(x[h], cent[h], ids[h], bits, group, None if basis is None else basis[h])
        codes.append(c)
        metas.append(m)
    return np.stack(codes), (None if metas[0] is None else np.stack(metas))   # 16-bit residuals: no meta


def nearest_ids(x: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """Nearest centre per token via the expanded distance in fp64 (test-input
    preparation only; parity of the assignment itself uses oracle.assign)."""
    H = x.shape[0]
    out = np.empty(x.shape[:2], np.int64)
    for h in range(H):
        xh = torch.from_numpy(x[h].astype(np.float64))
        ch = torch.from_numpy(cent[h].astype(np.float64))
        d = (xh * xh).sum(1, keepdim=True) - 2 * xh @ ch.T + (ch * ch).sum(1)[None, :]
        out[h] = d.argmin(1).numpy()
    return out


class Cache:
    """A compressed cache made by the oracle: numpy arrays per tensor, all heads."""

    def __init__(self, k, v, kc, vc, kid, vid, k_bits, v_bits, group, basis_k=None, basis_v=None):
        self.k_bits, self.v_bits, self.group = k_bits, v_bits, group
        self.kc, self.vc = kc, vc
        self.kid, self.vid = kid, vid
        self.basis_k, self.basis_v = basis_k, basis_v
        self.k_codes, self.k_meta = encode_heads(k, kc, kid, k_bits, group, basis_k)
        self.v_codes, self.v_meta = encode_heads(v, vc, vid, v_bits, group, basis_v)
        self.rank = 0 if basis_k is None else basis_k.shape[2]

    @property
    def n_tokens(self):
        return self.kid.shape[1]

    def oracle_segment(self, h: int) -> oracle.Segment:
        km = None if self.k_meta is None else self.k_meta[h]
        vm = None if self.v_meta is None else self.v_meta[h]
        return oracle.Segment(self.k_codes[h], km, self.kid[h], self.kc[h],
                              self.v_codes[h], vm, self.vid[h], self.vc[h],
                              self.k_bits, self.v_bits, self.group)

    def gpu_segment(self, cent_dtype=torch.bfloat16, head_map=None, device="cuda"):
        """Upload as a GPU segment; head_map (source head of every GPU head) tiles
        the oracle's heads over a larger head count on the device."""
        import compressed_kv_cache_kvc_amd as kvc
        idx = None if head_map is None else torch.as_tensor(np.asarray(head_map), device=device)

        def up(a, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype is not None:
                t = t.to(dtype)
            t = t.to(device)
            if idx is not None:
                t = t.index_select(0, idx)
            return t.contiguous()

        def meta(m):
            return None if m is None else up(m.view(np.int16)).view(torch.uint16)

        return kvc.Segment(
            k_codes=up(self.k_codes), k_meta=meta(self.k_meta),
            k_ids=up(self.kid.astype(np.uint8)), k_cent=up(self.kc, cent_dtype),
            v_codes=up(self.v_codes), v_meta=meta(self.v_meta),
            v_ids=up(self.vid.astype(np.uint8)), v_cent=up(self.vc, cent_dtype),
            k_bits=self.k_bits, v_bits=self.v_bits, group=self.group, rank=self.rank)


def ar1_kv(cfg, heads, n_tokens, stream_id=0):
    """bf16 K and V [heads, n_tokens, d] from the AR(1) generator, as torch tensors."""
    k = synth.AR1Stream(cfg, "k", heads=heads, stream_id=stream_id).tokens(n_tokens)
    v = synth.AR1Stream(cfg, "v", heads=heads, stream_id=stream_id).tokens(n_tokens)
    return k, v


def attn_errors(out_gpu: np.ndarray, lse_gpu: np.ndarray, out_ref: np.ndarray, lse_ref: np.ndarray):
    """(rel-L2, max-abs, max |dLSE|) of one head's checked rows."""
    diff = out_gpu.astype(np.float64) - out_ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(out_ref), 1e-300))
    mabs = float(np.max(np.abs(diff))) if diff.size else 0.0
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse_gpu)), "LSE finiteness differs"
    dl = float(np.max(np.abs(lse_gpu[fin].astype(np.float64) - lse_ref[fin]))) if fin.any() else 0.0
    return rel, mabs, dl


REL_L2 = 1e-2     # attention tolerances (per head, checked rows)
MAX_ABS = 2e-2
MAX_DLSE = 2e-2


def check_attention(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    rel, mabs, dl = attn_errors(out_gpu, lse_gpu, out_ref, lse_ref)
    assert rel <= REL_L2 and mabs <= MAX_ABS and dl <= MAX_DLSE, \
        f"{what}: rel-L2 {rel:.3e}, max-abs {mabs:.3e}, |dLSE| {dl:.3e}"
    return rel, mabs, dl


def near_tie(d1, d2, rel=1e-5):
    """Tokens whose oracle top-2 distance gap is below ``rel`` of the second distance."""
    d2s = np.where(np.isfinite(d2), d2, np.inf)
    with np.errstate(invalid="ignore", divide="ignore"):
        gap = (d2s - d1) / d2s
    return (gap < rel) | (d2s == 0)


def check_ids(ids_gpu: np.ndarray, x: np.ndarray, cent: np.ndarray, rel=1e-5, what="", ref=None):
    """Nearest-centre ids of one head against the oracle: identical except on
    near-ties (0 < (D2 - D1)/D2 < rel); exact ties (D1 == D2) must go to the
    lowest index like the oracle's.  On a near-tie the GPU's id must still be a
    valid answer: its own distance, by the plain definition in fp64, within
    rel * D2 of the smallest.  ``ref`` may pass oracle.assign(x, cent) when it
    is already known.  Returns (near-ties, ids that differ from the oracle's)."""
    ids, d1, d2 = oracle.assign(x, cent) if ref is None else ref
    exact = d1 == d2
    tie = near_tie(d1, d2, rel) & ~exact
    bad = (ids_gpu != ids) & ~tie
    assert not bad.any(), f"{what}: {int(bad.sum())} ids differ outside near-ties"
    j = np.nonzero(tie & (ids_gpu != ids))[0]
    if len(j):
        assert np.all((ids_gpu[j] >= 0) & (ids_gpu[j] < cent.shape[0])), f"{what}: id out of range on a near-tie"
        diff = x[j].astype(np.float64) - cent[ids_gpu[j]].astype(np.float64)
        dg = (diff * diff).sum(axis=1)
        worse = dg - d1[j] > rel * d2[j]
        assert not worse.any(), f"{what}: {int(worse.sum())} near-tie ids are not among the nearest centres"
    return int(tie.sum()), int(len(j))


def softmax_scale(d):
    return 1.0 / math.sqrt(d)
