"""Compressed KV cache for autoregressive video on MI355X (gfx950).

Thin Python binding of the kvc C ABI (include/kvc.h): it checks tensor shapes,
dtypes and devices, allocates the outputs and the workspace through PyTorch and
passes raw device pointers plus the current HIP stream.  Every step of the
computation runs in the HIP kernels of libkvc.so; nothing here computes.

Entry points (names follow the C ABI):
  fit_assign(x, centroids, n_iter)          -> ids            (centroids fitted in place)
  encode(x, centroids, bits, group, ...)    -> (codes, meta, ids)
  attend(q, segments)                       -> (out, lse)
  attend_noalloc(q, segments, out, lse)     -> (out, lse)     (no allocation: static scratch)
  attend_lowdim(q, basis_k, basis_v, segs)  -> (out, lse)
  lse_merge(outs, lses)                     -> (out, lse)
  assign_qsac(x, centroids, w, n_cand, group) -> ids          (query-aware key assignment)
  query_stats(q, w, n_prev)                 -> w              (running E[q_c^2], in place)
  route_frames(n_frames, n_recent, ...)     -> [bool]         (full-dim frames of a history)
  anchor_bits(k_bits, v_bits)               -> int            (anchor precision)
  query_moments(q, m, n_prev) / psac_basis(m) / psac_coeffs(...) / attend_psac(q, u, segs, coefs)
                                            (principal-subspace logit compensation)
  tempo_encode / tempo_decode               (predictive residual coding over latent frames)
  reconstructed_segment(k_hat, v_hat)       -> Segment        (decoded history as a 16-bit segment)
  streaming.StreamingCache                  (chunk-by-chunk composition: fit, encode, append, attend)
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import KvcSegment

__all__ = ["KvcError", "Segment", "fit_assign", "encode", "attend", "attend_noalloc", "attend_lowdim", "lse_merge",
           "assign_qsac", "query_stats", "route_frames", "anchor_bits", "query_moments", "psac_basis",
           "tempo_param_count", "tempo_encode", "tempo_decode", "reconstructed_segment",
           "psac_coeffs", "attend_psac", "library", "version"]


class KvcError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {message}")


def library():
    return _lib.load()


def version() -> str:
    return library().kvc_version().decode()


def _status_name(status: int) -> str:
    return library().kvc_status_string(status).decode()


def _check(status: int):
    if status != _lib.KVC_OK:
        raise KvcError(status, library().kvc_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.KVC_BF16
    if t.dtype == torch.float32:
        return _lib.KVC_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, device=None, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------ fit / assign
def fit_assign(x: torch.Tensor, centroids: torch.Tensor, n_iter: int = 2,
               ids_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Lloyd k-means per head; ``centroids`` [H, C, d] is updated in place with the
    fitted centres; returns the final ids [H, N] (uint8)."""
    _need(x, "x")
    H, N, d = x.shape
    _need(centroids, "centroids", x.device, x.dtype)
    C = centroids.shape[1]
    if tuple(centroids.shape) != (H, C, d):
        raise ValueError("centroids must be [H, C, d]")
    ids = ids_out if ids_out is not None else torch.empty(H, N, dtype=torch.uint8, device=x.device)
    _need(ids, "ids_out", x.device, torch.uint8, (H, N))
    lib = library()
    wsb = lib.kvc_fit_assign_workspace_bytes(H, N, d, C)
    ws = _workspace(wsb, x.device)
    _check(lib.kvc_fit_assign(H, N, d, _dtype_code(x), _ptr(x), C, _ptr(centroids), n_iter, _ptr(ids),
                              _ptr(ws), wsb, _stream(x.device)))
    return ids


# ------------------------------------------------------------------------------ query-aware assignment
def assign_qsac(x: torch.Tensor, centroids: torch.Tensor, w: Optional[torch.Tensor], n_cand: int, group: int,
                ids_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """QSAC ids [H, N] (uint8) of key tokens x [H, N, d] against centroids [H, C, d];
    w [H, d] fp32 channel weights or None (all ones)."""
    _need(x, "x")
    H, N, d = x.shape
    _need(centroids, "centroids", x.device, x.dtype)
    C = centroids.shape[1]
    if tuple(centroids.shape) != (H, C, d):
        raise ValueError("centroids must be [H, C, d]")
    if w is not None:
        _need(w, "w", x.device, torch.float32, (H, d))
    ids = ids_out if ids_out is not None else torch.empty(H, N, dtype=torch.uint8, device=x.device)
    _need(ids, "ids_out", x.device, torch.uint8, (H, N))
    _check(library().kvc_assign_qsac(H, N, d, _dtype_code(x), _ptr(x), C, _ptr(centroids), _ptr(w), n_cand, group,
                                     _ptr(ids), _stream(x.device)))
    return ids


def query_stats(q: torch.Tensor, w: Optional[torch.Tensor] = None, n_prev: int = 0) -> torch.Tensor:
    """Running per-channel second moments of the queries q [H, n_q, d]: w [H, d]
    fp32 is updated in place (allocated when None, with n_prev = 0) and returned."""
    _need(q, "q")
    H, n_q, d = q.shape
    if w is None:
        if n_prev:
            raise ValueError("n_prev > 0 needs the previous statistics w")
        w = torch.empty(H, d, dtype=torch.float32, device=q.device)
    _need(w, "w", q.device, torch.float32, (H, d))
    lib = library()
    wsb = lib.kvc_query_stats_workspace_bytes(H, n_q, d)
    ws = _workspace(wsb, q.device)
    _check(lib.kvc_query_stats(H, n_q, d, _dtype_code(q), _ptr(q), n_prev, _ptr(w), _ptr(ws), wsb,
                               _stream(q.device)))
    return w


# ------------------------------------------------------------------------------ routing
def route_frames(n_frames: int, n_recent: int, period: int = 0, n_sink: int = 0,
                 all_full_until: int = 0) -> list:
    """Per latent frame (oldest first): True when read at full dimension."""
    buf = (ctypes.c_uint8 * max(1, n_frames))()
    _check(library().kvc_route_frames(n_frames, n_recent, period, n_sink, all_full_until, buf))
    return [bool(buf[f]) for f in range(n_frames)]


def anchor_bits(k_bits: int, v_bits: int) -> int:
    return int(library().kvc_anchor_bits(k_bits, v_bits))


# ------------------------------------------------------------------------------ predictive residual codec
def tempo_param_count(dim: int) -> int:
    return int(library().kvc_tempo_param_count(dim))


def _tempo_state(H: int, S: int, d: int, state: Optional[torch.Tensor], first_frame: int, device):
    if state is None:
        if first_frame > 0:
            raise ValueError("frames after the anchor need the state the previous call left")
        state = torch.zeros(H, S, 3, d, dtype=torch.float32, device=device)
    _need(state, "state", device, torch.float32, (H, S, 3, d))
    return state


def tempo_encode(k: torch.Tensor, v: torch.Tensor, params: torch.Tensor, first_frame: int, frame_tokens: int,
                 k_bits: int, v_bits: int, group: int, state: Optional[torch.Tensor] = None):
    """Predictive residual coding of the frames first_frame, ... of k, v [H, n*S, d]
    (params [H, P] fp32).  Returns (k_codes, k_meta, v_codes, v_meta, state); the
    state [H, S, 3, d] fp32 is updated in place (allocated for the anchor call)."""
    _need(k, "k")
    H, N, d = k.shape
    _need(v, "v", k.device, k.dtype, (H, N, d))
    _need(params, "params", k.device, torch.float32, (H, tempo_param_count(d)))
    S = frame_tokens
    if S <= 0 or N % S:
        raise ValueError("tokens must be whole frames of frame_tokens tokens")
    state = _tempo_state(H, S, d, state, first_frame, k.device)
    dev = k.device
    kc = torch.empty(H, N, d * k_bits // 8, dtype=torch.uint8, device=dev)
    vc = torch.empty(H, N, d * v_bits // 8, dtype=torch.uint8, device=dev)
    km = torch.empty(H, N, d // group, 2, dtype=torch.uint16, device=dev)
    vm = torch.empty(H, N, d // group, 2, dtype=torch.uint16, device=dev)
    _check(library().kvc_tempo_encode(H, S, first_frame, N // S, d, _dtype_code(k), _ptr(k), _ptr(v), _ptr(params),
                                      k_bits, v_bits, group, _ptr(kc), _ptr(km), _ptr(vc), _ptr(vm), _ptr(state),
                                      _stream(dev)))
    return kc, km, vc, vm, state


def tempo_decode(k_codes: torch.Tensor, k_meta: torch.Tensor, v_codes: torch.Tensor, v_meta: torch.Tensor,
                 params: torch.Tensor, first_frame: int, frame_tokens: int, k_bits: int, v_bits: int, group: int,
                 state: Optional[torch.Tensor] = None, k_hat: Optional[torch.Tensor] = None,
                 v_hat: Optional[torch.Tensor] = None):
    """Reconstruct the frames a tempo_encode call coded.  Returns (k_hat, v_hat,
    state): fp16 [H, n*S, d] reconstructions and the state (updated in place)."""
    _need(k_codes, "k_codes")
    H, N, _ = k_codes.shape
    dev = k_codes.device
    d = k_codes.shape[2] * 8 // k_bits
    _need(params, "params", dev, torch.float32, (H, tempo_param_count(d)))
    _need(k_codes, "k_codes", dev, torch.uint8, (H, N, d * k_bits // 8))
    _need(v_codes, "v_codes", dev, torch.uint8, (H, N, d * v_bits // 8))
    _need(k_meta, "k_meta", dev, torch.uint16, (H, N, d // group, 2))
    _need(v_meta, "v_meta", dev, torch.uint16, (H, N, d // group, 2))
    S = frame_tokens
    if S <= 0 or N % S:
        raise ValueError("tokens must be whole frames of frame_tokens tokens")
    state = _tempo_state(H, S, d, state, first_frame, dev)
    k_hat = k_hat if k_hat is not None else torch.empty(H, N, d, dtype=torch.float16, device=dev)
    v_hat = v_hat if v_hat is not None else torch.empty(H, N, d, dtype=torch.float16, device=dev)
    _need(k_hat, "k_hat", dev, torch.float16, (H, N, d))
    _need(v_hat, "v_hat", dev, torch.float16, (H, N, d))
    _check(library().kvc_tempo_decode(H, S, first_frame, N // S, d, _ptr(params), k_bits, v_bits, group,
                                      _ptr(k_codes), _ptr(k_meta), _ptr(v_codes), _ptr(v_meta), _ptr(state),
                                      _ptr(k_hat), _ptr(v_hat), _stream(dev)))
    return k_hat, v_hat, state


def reconstructed_segment(k_hat: torch.Tensor, v_hat: torch.Tensor) -> "Segment":
    """A history segment holding reconstructed K and V (fp16 [H, n, d]) as 16-bit
    residuals over a zero centre table (one centre, all ids 0), which attend()
    reads unchanged."""
    H, N, d = k_hat.shape
    dev = k_hat.device
    ids = torch.zeros(H, N, dtype=torch.uint8, device=dev)
    zero = torch.zeros(H, 1, d, dtype=torch.bfloat16, device=dev)
    return Segment(k_hat.view(torch.uint8).view(H, N, 2 * d), None, ids, zero,
                   v_hat.view(torch.uint8).view(H, N, 2 * d), None, ids, zero, 16, 16, 16)


# ------------------------------------------------------------------------------ encode
def encode(x: torch.Tensor, centroids: torch.Tensor, bits: int, group: int,
           ids: Optional[torch.Tensor] = None, basis: Optional[torch.Tensor] = None,
           codes_out: Optional[torch.Tensor] = None, meta_out: Optional[torch.Tensor] = None):
    """Encode [H, N, d] tokens against [H, C, d] centres.  Returns (codes uint8
    [H, N, code_dim*bits/8], meta uint16 [H, N, code_dim/group, 2] (fp16 bits of
    scale, zero), ids uint8 [H, N]).  Without ``ids`` the assignment runs first.
    bits=16 stores the fp16 residual itself (full dimension) and returns meta None."""
    _need(x, "x")
    H, N, d = x.shape
    _need(centroids, "centroids", x.device, x.dtype)
    C = centroids.shape[1]
    if tuple(centroids.shape) != (H, C, d):
        raise ValueError("centroids must be [H, C, d]")
    rank = 0
    if basis is not None:
        _need(basis, "basis", x.device, torch.float32)
        if basis.shape[0] != H or basis.shape[1] != d:
            raise ValueError("basis must be [H, d, rank]")
        rank = basis.shape[2]
    code_dim = rank or d
    codes = codes_out if codes_out is not None else torch.empty(
        H, N, code_dim * bits // 8, dtype=torch.uint8, device=x.device)
    _need(codes, "codes_out", x.device, torch.uint8, (H, N, code_dim * bits // 8))
    if bits == 16:
        meta = None
    else:
        meta = meta_out if meta_out is not None else torch.empty(
            H, N, code_dim // group, 2, dtype=torch.uint16, device=x.device)
        _need(meta, "meta_out", x.device, torch.uint16, (H, N, code_dim // group, 2))
    lib = library()
    if ids is None:
        ids_out = torch.empty(H, N, dtype=torch.uint8, device=x.device)
        wsb = lib.kvc_encode_workspace_bytes(H, N, d, C, 0)
        ws = _workspace(wsb, x.device)
        _check(lib.kvc_encode(H, N, d, _dtype_code(x), _ptr(x), C, _ptr(centroids), None, _ptr(ids_out),
                              _ptr(basis), rank, bits, group, _ptr(codes), _ptr(meta), _ptr(ws), wsb,
                              _stream(x.device)))
        return codes, meta, ids_out
    _need(ids, "ids", x.device, torch.uint8, (H, N))
    _check(lib.kvc_encode(H, N, d, _dtype_code(x), _ptr(x), C, _ptr(centroids), _ptr(ids), None,
                          _ptr(basis), rank, bits, group, _ptr(codes), _ptr(meta), None, 0,
                          _stream(x.device)))
    return codes, meta, ids


# ------------------------------------------------------------------------------ segments
@dataclass
class Segment:
    """One run of encoded history (all heads) with its own centre tables."""
    k_codes: torch.Tensor     # [H, n, code_dim*k_bits/8] uint8
    k_meta: Optional[torch.Tensor]  # [H, n, code_dim/group, 2] uint16; None for 16-bit residuals
    k_ids: torch.Tensor       # [H, n] uint8
    k_cent: torch.Tensor      # [H, C, d]
    v_codes: torch.Tensor
    v_meta: torch.Tensor
    v_ids: torch.Tensor
    v_cent: torch.Tensor
    k_bits: int
    v_bits: int
    group: int
    rank: int = 0

    @property
    def n_tokens(self) -> int:
        return int(self.k_ids.shape[1])

    def to_c(self) -> KvcSegment:
        s = KvcSegment()
        s.n_tokens = self.n_tokens
        s.n_centroids = int(self.k_cent.shape[1])
        if int(self.v_cent.shape[1]) != s.n_centroids:
            raise ValueError("K and V centre tables of a segment must have the same number of centres")
        s.rank = self.rank
        s.k_bits, s.v_bits, s.group = self.k_bits, self.v_bits, self.group
        s.cent_dtype = _dtype_code(self.k_cent)
        for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_ids", "v_ids", "k_cent", "v_cent"):
            t = getattr(self, name)
            if t is None and name.endswith("_meta"):
                setattr(s, name, None)       # 16-bit residual segments carry no metadata
                continue
            _need(t, name)
            setattr(s, name, t.data_ptr())
        return s


def _seg_array(segments: Sequence[Segment]):
    arr = (KvcSegment * max(1, len(segments)))()
    for i, s in enumerate(segments):
        arr[i] = s.to_c()
    return arr


# ------------------------------------------------------------------------------ attention
def attend(q: torch.Tensor, segments: Sequence[Segment], out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None):
    """Attention of q [H, n_q, d] over the concatenated segments.  Returns
    (out fp32 [H, n_q, d], lse fp32 [H, n_q])."""
    _need(q, "q")
    H, n_q, d = q.shape
    out = out if out is not None else torch.empty(H, n_q, d, dtype=torch.float32, device=q.device)
    lse = lse if lse is not None else torch.empty(H, n_q, dtype=torch.float32, device=q.device)
    _need(out, "out", q.device, torch.float32, (H, n_q, d))
    _need(lse, "lse", q.device, torch.float32, (H, n_q))
    arr = _seg_array(segments)
    lib = library()
    wsb = lib.kvc_attend_workspace_bytes(H, n_q, d, _dtype_code(q), arr, len(segments))
    ws = _workspace(wsb, q.device)
    _check(lib.kvc_attend(H, n_q, d, _dtype_code(q), _ptr(q), arr, len(segments), _ptr(out), _ptr(lse),
                          _ptr(ws), wsb, _stream(q.device)))
    return out, lse


def attend_noalloc(q: torch.Tensor, segments: Sequence[Segment], out: torch.Tensor, lse: torch.Tensor):
    """attend() through kvc_attend_noalloc: the workspace is the library's static
    per-GPU scratch array, so the call allocates nothing (the caller passes the
    outputs).  Calls that overlap on one GPU race on that array."""
    _need(q, "q")
    H, n_q, d = q.shape
    _need(out, "out", q.device, torch.float32, (H, n_q, d))
    _need(lse, "lse", q.device, torch.float32, (H, n_q))
    arr = _seg_array(segments)
    _check(library().kvc_attend_noalloc(H, n_q, d, _dtype_code(q), _ptr(q), arr, len(segments), _ptr(out),
                                        _ptr(lse), _stream(q.device)))
    return out, lse


# ------------------------------------------------------------------------------ logit compensation
PSAC_RANK = 8


def query_moments(q: torch.Tensor, m: Optional[torch.Tensor] = None, n_prev: int = 0) -> torch.Tensor:
    """Running second-moment matrices [H, d, d] fp32 of the queries q [H, n_q, d]
    (updated in place; allocated when None, with n_prev = 0)."""
    _need(q, "q")
    H, n_q, d = q.shape
    if m is None:
        if n_prev:
            raise ValueError("n_prev > 0 needs the previous moments m")
        m = torch.empty(H, d, d, dtype=torch.float32, device=q.device)
    _need(m, "m", q.device, torch.float32, (H, d, d))
    _check(library().kvc_query_moments(H, n_q, d, _dtype_code(q), _ptr(q), n_prev, _ptr(m), _stream(q.device)))
    return m


def psac_basis(m: torch.Tensor, n_iter: int = 32, u_prev: Optional[torch.Tensor] = None):
    """Top-8 eigenvectors u [H, d, 8] fp32 and eigenvalues [H, 8] of m [H, d, d]."""
    _need(m, "m", dtype=torch.float32)
    H, d, _ = m.shape
    u = torch.empty(H, d, PSAC_RANK, dtype=torch.float32, device=m.device)
    lam = torch.empty(H, PSAC_RANK, dtype=torch.float32, device=m.device)
    if u_prev is not None:
        _need(u_prev, "u_prev", m.device, torch.float32, (H, d, PSAC_RANK))
    _check(library().kvc_psac_basis(H, d, _ptr(m), PSAC_RANK, n_iter, _ptr(u_prev), _ptr(u), _ptr(lam),
                                    _stream(m.device)))
    return u, lam


def psac_coeffs(x: torch.Tensor, centroids: torch.Tensor, ids: torch.Tensor, codes: torch.Tensor,
                meta: torch.Tensor, bits: int, group: int, u: torch.Tensor) -> torch.Tensor:
    """Kept coefficients [H, N, 8] fp16 (as uint16 bits) of the keys' remaining
    quantization error along u [H, d, 8]."""
    _need(x, "x")
    H, N, d = x.shape
    C = centroids.shape[1]
    _need(centroids, "centroids", x.device, x.dtype, (H, C, d))
    _need(ids, "ids", x.device, torch.uint8, (H, N))
    _need(codes, "codes", x.device, torch.uint8)
    _need(meta, "meta", x.device, torch.uint16)
    _need(u, "u", x.device, torch.float32, (H, d, PSAC_RANK))
    coef = torch.empty(H, N, PSAC_RANK, dtype=torch.uint16, device=x.device)
    _check(library().kvc_psac_coeffs(H, N, d, _dtype_code(x), _ptr(x), C, _ptr(centroids), _ptr(ids), _ptr(codes),
                                     _ptr(meta), bits, group, _ptr(u), PSAC_RANK, _ptr(coef), _stream(x.device)))
    return coef


def attend_psac(q: torch.Tensor, u: torch.Tensor, segments: Sequence[Segment], coefs: Sequence[torch.Tensor],
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """attend() with every logit corrected by (u^T q) . coef (one coefficient
    tensor [H, n, 8] per segment)."""
    _need(q, "q")
    H, n_q, d = q.shape
    _need(u, "u", q.device, torch.float32, (H, d, PSAC_RANK))
    if len(coefs) != len(segments):
        raise ValueError("one coefficient tensor per segment")
    for s, c in zip(segments, coefs):
        _need(c, "coef", q.device, torch.uint16, (H, s.n_tokens, PSAC_RANK))
    out = out if out is not None else torch.empty(H, n_q, d, dtype=torch.float32, device=q.device)
    lse = lse if lse is not None else torch.empty(H, n_q, dtype=torch.float32, device=q.device)
    _need(out, "out", q.device, torch.float32, (H, n_q, d))
    _need(lse, "lse", q.device, torch.float32, (H, n_q))
    arr = _seg_array(segments)
    cp = (ctypes.c_void_p * max(1, len(coefs)))(*[c.data_ptr() for c in coefs])
    lib = library()
    wsb = lib.kvc_attend_psac_workspace_bytes(H, n_q, d, _dtype_code(q), arr, len(segments))
    ws = _workspace(wsb, q.device)
    _check(lib.kvc_attend_psac(H, n_q, d, _dtype_code(q), _ptr(q), _ptr(u), PSAC_RANK, arr, cp, len(segments),
                               _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream(q.device)))
    return out, lse


def attend_lowdim(q: torch.Tensor, basis_k: torch.Tensor, basis_v: torch.Tensor, segments: Sequence[Segment],
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Low-dimensional attention over coefficient-coded segments; returns
    (out fp32 [H, n_q, d], lse fp32 [H, n_q])."""
    _need(q, "q")
    H, n_q, d = q.shape
    _need(basis_k, "basis_k", q.device, torch.float32)
    _need(basis_v, "basis_v", q.device, torch.float32, tuple(basis_k.shape))
    rank = basis_k.shape[2]
    out = out if out is not None else torch.empty(H, n_q, d, dtype=torch.float32, device=q.device)
    lse = lse if lse is not None else torch.empty(H, n_q, dtype=torch.float32, device=q.device)
    _need(out, "out", q.device, torch.float32, (H, n_q, d))
    _need(lse, "lse", q.device, torch.float32, (H, n_q))
    arr = _seg_array(segments)
    lib = library()
    wsb = lib.kvc_attend_lowdim_workspace_bytes(H, n_q, d, rank, arr, len(segments))
    ws = _workspace(wsb, q.device)
    _check(lib.kvc_attend_lowdim(H, n_q, d, _dtype_code(q), _ptr(q), _ptr(basis_k), _ptr(basis_v), rank, arr,
                                 len(segments), _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream(q.device)))
    return out, lse


def lse_merge(outs: Sequence[torch.Tensor], lses: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None):
    """Merge attention parts of the same queries by log-sum-exp."""
    if len(outs) != len(lses) or not outs:
        raise ValueError("need the same positive number of outputs and LSEs")
    H, n_q, d = outs[0].shape
    for i, (o, l) in enumerate(zip(outs, lses)):
        _need(o, f"outs[{i}]", outs[0].device, torch.float32, (H, n_q, d))
        _need(l, f"lses[{i}]", outs[0].device, torch.float32, (H, n_q))
    dev = outs[0].device
    out = out if out is not None else torch.empty(H, n_q, d, dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty(H, n_q, dtype=torch.float32, device=dev)
    po = (ctypes.c_void_p * len(outs))(*[o.data_ptr() for o in outs])
    pl = (ctypes.c_void_p * len(lses))(*[l.data_ptr() for l in lses])
    _check(library().kvc_lse_merge(H, n_q, d, len(outs), po, pl, _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse
