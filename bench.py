"""Benchmark of the compressed-KV hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input that
already sits in HBM: fit the K and V centres (two Lloyd iterations + final
assignment), encode K and V, and attend the current chunk's queries over the
compressed history (plus, for the larger-backbone workload, the low-dimensional
far-history read and the LSE merge; for the streaming workload, ten chunks of
fit + encode + attention over the growing history).

Prints ONE JSON line.  `value` is the compressed-history attention throughput
(TFLOP/s, 4*n_q*n_kv*d per head, multiply and add counted as 2) over the timed
steps; the line also carries the encode rate (tokens/s, GB/s), the step time,
the roofline of the attention kernel measured with HIP events on the launch
stream, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="streaming",
                    choices=["self_forcing_layer", "long_history", "larger_backbone", "streaming", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--qsac", type=int, default=0, metavar="M",
                    help="re-assign the keys after the fit with the query-aware assignment (QuantWM section 4.1) "
                         "over M candidates, weighted by the statistics of the previous chunks' queries, and "
                         "update those statistics after the attention (self_forcing_layer, streaming); 0 = off")
    ap.add_argument("--psac", action="store_true",
                    help="self_forcing_layer, streaming: compensate the keys' remaining error along the top-8 "
                         "directions of the earlier queries (QuantWM section 4.2): kept coefficients after the "
                         "encode, compensated attention, then the query moments and the basis updated")
    ap.add_argument("--route", default="", metavar="R,P,S,A",
                    help="larger_backbone: read at full dimension the R most recent latent frames, one anchor "
                         "per P older frames, the S oldest frames, or every frame while the history has at most "
                         "A frames (NanoKV appendix Table 7); the rest through the rank-r maps")
    ap.add_argument("--anchor", action="store_true",
                    help="larger_backbone: code the oldest frame, when read at full dimension, at "
                         "max(4, k_bits, v_bits) bits (TempoKV section 3.3)")
    ap.add_argument("--tempo", action="store_true",
                    help="self_forcing_layer coded by predictive residuals over its latent frames (TempoKV "
                         "section 3.3): encode, decode and attention over the decoded history")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the warmup, run one plain fp32 negation of MIB MiB (reads and writes MIB MiB) so "
                         "that a hardware-counter run can scale its byte counters against a kernel of known traffic")
    return ap.parse_args()


# ------------------------------------------------------------------------------ workloads
class Workload:
    """Inputs resident on the GPU plus a step() that runs the whole hot path."""

    def __init__(self, cfg, dev):
        import torch
        import synth
        self.cfg, self.dev, self.torch = cfg, dev, torch
        self.synth = synth
        self.phase_ms = {}
        self.events = []
        self.side = None
        self.qsac = 0                 # candidates of the query-aware key assignment (0: plain ids)
        self.psac = False             # logit compensation of the remaining key error
        self.mq = None                # running query second moments [H, d, d]
        self.u = None                 # principal query directions [H, d, 8]
        self.wq = None                # running query statistics [H, d] fp32
        self.n_seen = 0               # queries folded into wq

    def both(self, fk, fv):
        """Run fk() on the current stream and fv() on a second stream (default
        priority), both after the work already queued; the current stream then
        waits for the second.  The K and V fits are independent, so their small,
        latency-bound launches overlap."""
        torch = self.torch
        cur = torch.cuda.current_stream()
        if self.side is None:
            self.side = torch.cuda.Stream()
        self.side.wait_stream(cur)
        rk = fk()
        with torch.cuda.stream(self.side):
            rv = fv()
        for t in (rv if isinstance(rv, (list, tuple)) else [rv]):
            if isinstance(t, torch.Tensor):
                t.record_stream(cur)
        cur.wait_stream(self.side)
        return rk, rv

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def mark(self, name, a, b):
        self.events.append((name, a, b))

    def collect(self):
        acc = {}
        for name, a, b in self.events:
            acc[name] = acc.get(name, 0.0) + a.elapsed_time(b)
        self.events = []
        return acc


def fit_encode_pair(w, k, kc0, v, vc0, n_iter=2):
    """Fit the K and V centres (from kc0, vc0) side by side, then encode both:
    returns (kcodes, kmeta, kid, kc), (vcodes, vmeta, vid, vc)."""
    import compressed_kv_cache_kvc_amd as kvc
    cfg = w.cfg
    kc, vc = kc0.clone(), vc0.clone()
    e0 = w.ev()
    kid, vid = w.both(lambda: kvc.fit_assign(k, kc, n_iter=n_iter), lambda: kvc.fit_assign(v, vc, n_iter=n_iter))
    e1 = w.ev()
    w.mark("fit", e0, e1)
    if w.qsac:
        kid = kvc.assign_qsac(k, kc, w.wq, w.qsac, cfg.group)
        e1b = w.ev()
        w.mark("qsac", e1, e1b)
        e1 = e1b
    kco, kme, _ = kvc.encode(k, kc, cfg.k_bits, cfg.group, ids=kid)
    vco, vme, _ = kvc.encode(v, vc, cfg.v_bits, cfg.group, ids=vid)
    e2 = w.ev()
    w.mark("encode", e1, e2)
    if w.psac and w.u is not None:
        w.coef = kvc.psac_coeffs(k, kc, kid, kco, kme, cfg.k_bits, cfg.group, w.u)
        e3 = w.ev()
        w.mark("psac_coeffs", e2, e3)
    return (kco, kme, kid, kc), (vco, vme, vid, vc)


def attend_step(w, q, segs, coefs):
    """The attention call of a step (compensated when PSAC is on and a basis exists)."""
    import compressed_kv_cache_kvc_amd as kvc
    e0 = w.ev()
    if w.psac and w.u is not None:
        out, lse = kvc.attend_psac(q, w.u, segs, coefs)
    else:
        out, lse = kvc.attend(q, segs)
    e1 = w.ev()
    w.mark("attend", e0, e1)
    return out, lse


def update_psac_basis(w, q):
    """Fold the chunk's queries into the second moments and refresh the basis
    (warm start from the previous one)."""
    import compressed_kv_cache_kvc_amd as kvc
    e0 = w.ev()
    w.mq = kvc.query_moments(q, w.mq, n_prev=w.n_seen_m)
    e1 = w.ev()
    w.u, _ = kvc.psac_basis(w.mq, n_iter=4 if w.u is not None else 32, u_prev=w.u)
    e2 = w.ev()
    w.mark("query_moments", e0, e1)
    w.mark("psac_basis", e1, e2)
    w.n_seen_m += q.shape[1]


def update_query_stats(w, q):
    """Fold the chunk's queries into the running statistics (timed as a phase)."""
    import compressed_kv_cache_kvc_amd as kvc
    e0 = w.ev()
    w.wq = kvc.query_stats(q, w.wq, n_prev=w.n_seen)
    e1 = w.ev()
    w.mark("query_stats", e0, e1)
    w.n_seen += q.shape[1]


class SingleLayer(Workload):
    """self_forcing_layer, long_history, tiny: one history, fitted and encoded per step."""

    def __init__(self, cfg, dev):
        super().__init__(cfg, dev)
        torch, synth = self.torch, self.synth
        H, N = cfg.heads, cfg.hist
        if cfg.dtype == "f32":
            self.k, _ = synth.tiny_kv(cfg, "k")
            self.v, _ = synth.tiny_kv(cfg, "v")
            self.k, self.v = self.k.to(dev), self.v.to(dev)
        else:
            self.k = synth.AR1Stream(cfg, "k", device=dev).tokens(N)
            self.v = synth.AR1Stream(cfg, "v", device=dev).tokens(N)
        self.q = synth.queries(cfg, device=dev)
        S = cfg.n_segments
        self.bounds = [N * i // S for i in range(S + 1)]
        self.k_parts = [self.k[:, a:b].contiguous() for a, b in zip(self.bounds[:-1], self.bounds[1:])]
        self.v_parts = [self.v[:, a:b].contiguous() for a, b in zip(self.bounds[:-1], self.bounds[1:])]
        # one centre table per head over the whole history; segments are attention splits
        self.kc0 = synth.forgy_init(self.k, cfg.n_centroids, synth.seed_for(cfg.seed, 0, 0, 1)).to(dev)
        self.vc0 = synth.forgy_init(self.v, cfg.n_centroids, synth.seed_for(cfg.seed, 0, 1, 1)).to(dev)
        self.attn_flops = 4.0 * H * cfg.n_q * N * cfg.dim
        self.enc_tokens = H * N
        esz = 4 if cfg.dtype == "f32" else 2
        self.enc_bytes = sum(H * N * (cfg.dim * esz + 1) + H * N * (cfg.dim * b // 8 + 4 * cfg.dim // cfg.group)
                             for b in (cfg.k_bits, cfg.v_bits))

    def step(self):
        import compressed_kv_cache_kvc_amd as kvc
        cfg = self.cfg
        if len(self.bounds) == 2:
            (kcodes, kmeta, kid, kc), (vcodes, vmeta, vid, vc) = fit_encode_pair(
                self, self.k, self.kc0, self.v, self.vc0, n_iter=cfg.n_iter)
            segs = [kvc.Segment(kcodes, kmeta, kid, kc, vcodes, vmeta, vid, vc, cfg.k_bits, cfg.v_bits, cfg.group)]
            if self.psac:
                out, lse = attend_step(self, self.q, segs, [self.coef])
                update_psac_basis(self, self.q)
                if self.qsac:
                    update_query_stats(self, self.q)
                return out
        else:
            # one centre table per head over the whole history; each history
            # segment is encoded from its own slice (segments are attention splits)
            kc, vc = self.kc0.clone(), self.vc0.clone()
            e0 = self.ev()
            kid, vid = self.both(lambda: kvc.fit_assign(self.k, kc, n_iter=cfg.n_iter),
                                 lambda: kvc.fit_assign(self.v, vc, n_iter=cfg.n_iter))
            e1 = self.ev()
            segs = []
            for (a, b), ks, vs in zip(zip(self.bounds[:-1], self.bounds[1:]), self.k_parts, self.v_parts):
                ki, vi = kid[:, a:b].contiguous(), vid[:, a:b].contiguous()
                kco, kme, _ = kvc.encode(ks, kc, cfg.k_bits, cfg.group, ids=ki)
                vco, vme, _ = kvc.encode(vs, vc, cfg.v_bits, cfg.group, ids=vi)
                segs.append(kvc.Segment(kco, kme, ki, kc, vco, vme, vi, vc, cfg.k_bits, cfg.v_bits, cfg.group))
            e2 = self.ev()
            self.mark("fit", e0, e1)
            self.mark("encode", e1, e2)
        e0 = self.ev()
        out, lse = kvc.attend(self.q, segs)
        e1 = self.ev()
        self.mark("attend", e0, e1)
        if self.qsac:
            update_query_stats(self, self.q)
        return out

    def enable_psac(self):
        """Logit compensation; moments and basis start from a previous chunk's queries."""
        import compressed_kv_cache_kvc_amd as kvc
        if len(self.bounds) != 2 or self.cfg.dtype != "bf16":
            raise SystemExit("--psac covers the single-segment bf16 workloads (self_forcing_layer, streaming)")
        self.psac = True
        prev = self.synth.queries(self.cfg, device=self.dev, stream_id=2)
        self.mq = kvc.query_moments(prev)
        self.u, _ = kvc.psac_basis(self.mq, n_iter=32)
        self.n_seen_m = prev.shape[1]

    def enable_qsac(self, m):
        """Query-aware key assignment; the statistics start from a previous chunk's queries."""
        import compressed_kv_cache_kvc_amd as kvc
        if len(self.bounds) != 2:
            raise SystemExit("--qsac covers the single-segment workloads (self_forcing_layer, streaming, tiny)")
        self.qsac = m
        prev = self.synth.queries(self.cfg, device=self.dev, stream_id=1)
        self.wq = kvc.query_stats(prev)
        self.n_seen = prev.shape[1]


class LargerBackbone(Workload):
    """Far history (rank-32 coefficients) + recent full-dim part, merged by LSE."""

    def __init__(self, cfg, dev):
        super().__init__(cfg, dev)
        synth = self.synth
        H, N, r = cfg.heads, cfg.hist, cfg.rank
        self.k = synth.AR1Stream(cfg, "k", device=dev).tokens(N)
        self.v = synth.AR1Stream(cfg, "v", device=dev).tokens(N)
        self.q = synth.queries(cfg, device=dev)
        self.kc0 = synth.forgy_init(self.k, cfg.n_centroids, synth.seed_for(cfg.seed, 0, 0, 1)).to(dev)
        self.vc0 = synth.forgy_init(self.v, cfg.n_centroids, synth.seed_for(cfg.seed, 0, 1, 1)).to(dev)
        self.Uk = synth.orthonormal_basis(H, cfg.dim, r, synth.seed_for(cfg.seed, 0, 0, 2)).to(dev)
        self.Uv = synth.orthonormal_basis(H, cfg.dim, r, synth.seed_for(cfg.seed, 0, 1, 2)).to(dev)
        F, R = cfg.far, cfg.recent
        self.kf, self.kr = self.k[:, :F].contiguous(), self.k[:, F:].contiguous()
        self.vf, self.vr = self.v[:, :F].contiguous(), self.v[:, F:].contiguous()
        self.attn_flops = 4.0 * H * cfg.n_q * R * cfg.dim + 4.0 * H * cfg.n_q * F * r + 4.0 * H * cfg.n_q * cfg.dim * r
        self.full_tokens, self.low_tokens = R, F
        self.enc_tokens = H * N
        self.enc_bytes = sum(H * N * (cfg.dim * 2 + 1) for _ in range(2)) + \
            H * R * (cfg.dim * (cfg.k_bits + cfg.v_bits) // 8 + 8 * cfg.dim // cfg.group) + \
            H * F * (r * (cfg.k_bits + cfg.v_bits) // 8 + 8 * r // cfg.group)

    def step(self):
        import compressed_kv_cache_kvc_amd as kvc
        cfg = self.cfg
        torch = self.torch
        kc, vc = self.kc0.clone(), self.vc0.clone()
        e0 = self.ev()
        kid, vid = self.both(lambda: kvc.fit_assign(self.k, kc, n_iter=cfg.n_iter),
                             lambda: kvc.fit_assign(self.v, vc, n_iter=cfg.n_iter))
        e1 = self.ev()
        F = cfg.far
        kidf, kidr = kid[:, :F].contiguous(), kid[:, F:].contiguous()
        vidf, vidr = vid[:, :F].contiguous(), vid[:, F:].contiguous()
        krc, krm, _ = kvc.encode(self.kr, kc, cfg.k_bits, cfg.group, ids=kidr)
        vrc, vrm, _ = kvc.encode(self.vr, vc, cfg.v_bits, cfg.group, ids=vidr)
        e1b = self.ev()
        kfc, kfm, _ = kvc.encode(self.kf, kc, cfg.k_bits, cfg.group, ids=kidf, basis=self.Uk)
        vfc, vfm, _ = kvc.encode(self.vf, vc, cfg.v_bits, cfg.group, ids=vidf, basis=self.Uv)
        e2 = self.ev()
        self.mark("encode_lowdim", e1b, e2)
        recent = kvc.Segment(krc, krm, kidr, kc, vrc, vrm, vidr, vc, cfg.k_bits, cfg.v_bits, cfg.group)
        far = kvc.Segment(kfc, kfm, kidf, kc, vfc, vfm, vidf, vc, cfg.k_bits, cfg.v_bits, cfg.group, rank=cfg.rank)
        o1, l1 = kvc.attend(self.q, [recent])
        e3 = self.ev()
        o2, l2 = kvc.attend_lowdim(self.q, self.Uk, self.Uv, [far])
        e4 = self.ev()
        out, lse = kvc.lse_merge([o1, o2], [l1, l2])
        e5 = self.ev()
        self.mark("fit", e0, e1)
        self.mark("encode", e1, e2)
        self.mark("attend", e2, e3)
        self.mark("attend_lowdim", e3, e4)
        self.mark("lse_merge", e4, e5)
        return out


class RoutedBackbone(LargerBackbone):
    """larger_backbone with frame routing (NanoKV appendix Table 7): the latent
    frames chosen by the rule (recent frames, a sink, periodic anchors) are read
    at full dimension, the others through the rank-r maps; with --anchor the
    oldest frame, when read at full dimension, is coded at b_a = max(4, b_K, b_V)
    bits (TempoKV section 3.3).  Full-dimensional runs of different codecs go to
    one attention call (one launch per codec), the reduced runs to the low-dim
    call, and the two results are merged by LSE."""

    def __init__(self, cfg, dev, route, anchor):
        super().__init__(cfg, dev)
        import compressed_kv_cache_kvc_amd as kvc
        H, S = cfg.heads, cfg.frame_tokens
        n_frames = cfg.hist // S
        mask = kvc.route_frames(n_frames, *route)
        self.runs = []                 # (first token, end token, full, anchor)
        f = 0
        while f < n_frames:
            e = f
            while e < n_frames and mask[e] == mask[f]:
                e += 1
            if mask[f] and anchor and f == 0:
                self.runs.append((0, S, True, True))
                if e > 1:
                    self.runs.append((S, e * S, True, False))
            else:
                self.runs.append((f * S, e * S, mask[f], False))
            f = e
        self.anchor_bits = kvc.anchor_bits(cfg.k_bits, cfg.v_bits)
        full = sum(b - a for a, b, fu, _ in self.runs if fu)
        low = cfg.hist - full
        r = cfg.rank
        self.full_tokens, self.low_tokens = full, low
        self.attn_flops = 4.0 * H * cfg.n_q * full * cfg.dim + 4.0 * H * cfg.n_q * low * r + \
            (4.0 * H * cfg.n_q * cfg.dim * r if low else 0.0)
        self.slices = [(self.k[:, a:b].contiguous(), self.v[:, a:b].contiguous()) for a, b, _, _ in self.runs]
        self.route, self.anchor = route, anchor

    def step(self):
        import compressed_kv_cache_kvc_amd as kvc
        cfg = self.cfg
        kc, vc = self.kc0.clone(), self.vc0.clone()
        e0 = self.ev()
        kid, vid = self.both(lambda: kvc.fit_assign(self.k, kc, n_iter=cfg.n_iter),
                             lambda: kvc.fit_assign(self.v, vc, n_iter=cfg.n_iter))
        e1 = self.ev()
        full_segs, low_segs = [], []
        for (a, b, full, anc), (ks, vs) in zip(self.runs, self.slices):
            ki, vi = kid[:, a:b].contiguous(), vid[:, a:b].contiguous()
            kb, vb = (self.anchor_bits, self.anchor_bits) if anc else (cfg.k_bits, cfg.v_bits)
            if full:
                kco, kme, _ = kvc.encode(ks, kc, kb, cfg.group, ids=ki)
                vco, vme, _ = kvc.encode(vs, vc, vb, cfg.group, ids=vi)
                full_segs.append(kvc.Segment(kco, kme, ki, kc, vco, vme, vi, vc, kb, vb, cfg.group))
            else:
                kco, kme, _ = kvc.encode(ks, kc, kb, cfg.group, ids=ki, basis=self.Uk)
                vco, vme, _ = kvc.encode(vs, vc, vb, cfg.group, ids=vi, basis=self.Uv)
                low_segs.append(kvc.Segment(kco, kme, ki, kc, vco, vme, vi, vc, kb, vb, cfg.group, rank=cfg.rank))
        e2 = self.ev()
        o1, l1 = kvc.attend(self.q, full_segs)
        e3 = self.ev()
        o2, l2 = kvc.attend_lowdim(self.q, self.Uk, self.Uv, low_segs)
        e4 = self.ev()
        out, lse = kvc.lse_merge([o1, o2], [l1, l2])
        e5 = self.ev()
        self.mark("fit", e0, e1)
        self.mark("encode", e1, e2)
        self.mark("attend", e2, e3)
        self.mark("attend_lowdim", e3, e4)
        self.mark("lse_merge", e4, e5)
        return out


class Streaming(Workload):
    """Ten chunks: fit + encode each new chunk for all (layer, head) pairs, then
    attend the chunk's queries over every segment so far."""

    def __init__(self, cfg, dev):
        super().__init__(cfg, dev)
        synth = self.synth
        H, T = cfg.heads, cfg.chunk
        ks = synth.AR1Stream(cfg, "k", device=dev)
        vs = synth.AR1Stream(cfg, "v", device=dev)
        self.chunks = []
        for i in range(cfg.steps):
            k = ks.tokens(T)
            v = vs.tokens(T)
            q = synth.queries(cfg, device=dev, stream_id=i)
            kc0 = synth.forgy_init(k, cfg.n_centroids, synth.seed_for(cfg.seed, i, 0, 1)).to(dev)
            vc0 = synth.forgy_init(v, cfg.n_centroids, synth.seed_for(cfg.seed, i, 1, 1)).to(dev)
            self.chunks.append((k, v, q, kc0, vc0))
        self.attn_flops = sum(4.0 * H * cfg.n_q * T * (i + 1) * cfg.dim for i in range(cfg.steps))
        self.enc_tokens = H * T * cfg.steps
        self.enc_bytes = cfg.steps * sum(H * T * (cfg.dim * 2 + 1) + H * T * (cfg.dim * b // 8 + 4 * cfg.dim // cfg.group)
                                         for b in (cfg.k_bits, cfg.v_bits))

    def step(self):
        """One rollout: for each chunk, fit + encode it into the cache (its own
        centre tables), then attend the chunk's queries over every chunk so far.
        The cache is the package's StreamingCache, the composition the rollout
        parity test checks against the oracle."""
        import compressed_kv_cache_kvc_amd as kvc
        from compressed_kv_cache_kvc_amd.streaming import StreamingCache
        cfg = self.cfg
        cache = StreamingCache(cfg.k_bits, cfg.v_bits, cfg.group, n_iter=cfg.n_iter)
        out = None
        if self.qsac:                 # each rollout starts cold: unit weights for the first chunk
            self.wq, self.n_seen = None, 0
        if self.psac:                 # cold start: no compensation until queries have been seen
            self.mq, self.u, self.n_seen_m = None, None, 0
        coefs = []
        for (k, v, q, kc0, vc0) in self.chunks:
            e0 = self.ev()
            kid, kc, vid, vc = cache.fit(k, v, kc0, vc0)
            e1 = self.ev()
            self.mark("fit", e0, e1)
            if self.qsac:
                kid = kvc.assign_qsac(k, kc, self.wq, self.qsac, cfg.group)
                e1b = self.ev()
                self.mark("qsac", e1, e1b)
                e1 = e1b
            seg = cache.encode(k, v, kid, kc, vid, vc)
            e2 = self.ev()
            self.mark("encode", e1, e2)
            cache.push(seg)
            if self.psac:
                # one basis per rollout, fixed after the first chunk (the cold start);
                # the first chunk keeps zero coefficients (no compensation)
                if self.u is not None:
                    coefs.append(kvc.psac_coeffs(k, kc, kid, seg.k_codes, seg.k_meta, cfg.k_bits, cfg.group, self.u))
                    e3 = self.ev()
                    self.mark("psac_coeffs", e2, e3)
                else:
                    coefs.append(self.torch.zeros(cfg.heads, k.shape[1], 8, dtype=self.torch.uint16, device=self.dev))
                if self.u is not None:
                    out, lse = attend_step(self, q, cache.segments, coefs)
                else:
                    out, lse = attend_step(self, q, cache.segments, None)
                    update_psac_basis(self, q)
            else:
                out, lse = attend_step(self, q, cache.segments, None)
            if self.qsac:
                update_query_stats(self, q)
        return out

    def enable_psac(self):
        self.psac = True
        self.n_seen_m = 0

    def enable_qsac(self, m):
        self.qsac = m


class TempoLayer(Workload):
    """self_forcing_layer coded by predictive residuals over its six latent frames
    (TempoKV section 3.3): the anchor frame alone at 4 bits, then frames 1-5 at
    the layer's k_bits / v_bits; the step encodes, decodes the fp16
    reconstructions and attends over them (a 16-bit segment over a zero centre).
    Values depend on the aligned key (synth.coupled_values).  The predictor
    coefficients are seeded draws of plausible size (temporal gains below 1, a
    dense key-to-value map); their fitted values would not change the work."""

    def __init__(self, cfg, dev):
        super().__init__(cfg, dev)
        torch, synth = self.torch, self.synth
        import compressed_kv_cache_kvc_amd as kvc
        H, N, d = cfg.heads, cfg.hist, cfg.dim
        self.S = cfg.frame_tokens
        self.T = N // self.S
        self.k = synth.AR1Stream(cfg, "k", device=dev).tokens(N)
        self.v = synth.coupled_values(self.k, synth.AR1Stream(cfg, "v", device=dev).tokens(N),
                                      synth.seed_for(cfg.seed, 0, 1, 2))
        self.q = synth.queries(cfg, device=dev)
        g = torch.Generator(device="cpu").manual_seed(synth.seed_for(cfg.seed, 0, 0, 5))
        u = lambda lo, hi: lo + (hi - lo) * torch.rand(H, d, generator=g)   # noqa: E731
        z = lambda: 0.05 * torch.randn(H, d, generator=g)                   # noqa: E731
        w = 0.6 * torch.randn(H, d, d, generator=g) / math.sqrt(d)
        self.params = torch.cat([z(), u(0.6, 1.0), z(), u(0.4, 0.9), u(-0.2, 0.3), z(), u(0.0, 0.6),
                                 w.reshape(H, d * d)], dim=1).float().contiguous().to(dev)
        assert self.params.shape[1] == kvc.tempo_param_count(d)
        self.k0, self.k1 = self.k[:, :self.S].contiguous(), self.k[:, self.S:].contiguous()
        self.v0, self.v1 = self.v[:, :self.S].contiguous(), self.v[:, self.S:].contiguous()
        self.anchor_bits = kvc.anchor_bits(cfg.k_bits, cfg.v_bits)
        self.attn_flops = 4.0 * H * cfg.n_q * N * d
        self.enc_tokens = H * N
        self.enc_bytes = H * N * (d * 2 * 2) + H * self.S * 2 * (d * self.anchor_bits // 8 + 4 * d // cfg.group) + \
            H * (N - self.S) * (d * (cfg.k_bits + cfg.v_bits) // 8 + 8 * d // cfg.group)

    def step(self):
        import compressed_kv_cache_kvc_amd as kvc
        cfg, S, P = self.cfg, self.S, self.params
        ba, g = self.anchor_bits, cfg.group
        e0 = self.ev()
        a = kvc.tempo_encode(self.k0, self.v0, P, 0, S, ba, ba, g)
        b = kvc.tempo_encode(self.k1, self.v1, P, 1, S, cfg.k_bits, cfg.v_bits, g, a[4])
        e1 = self.ev()
        kh0, vh0, st = kvc.tempo_decode(a[0], a[1], a[2], a[3], P, 0, S, ba, ba, g)
        kh1, vh1, _ = kvc.tempo_decode(b[0], b[1], b[2], b[3], P, 1, S, cfg.k_bits, cfg.v_bits, g, st)
        e2 = self.ev()
        # the anchor frame and the predicted frames: two 16-bit segments, one launch
        out, lse = kvc.attend(self.q, [kvc.reconstructed_segment(kh0, vh0), kvc.reconstructed_segment(kh1, vh1)])
        e3 = self.ev()
        self.mark("tempo_encode", e0, e1)
        self.mark("tempo_decode", e1, e2)
        self.mark("attend", e2, e3)
        return out


def make_workload(cfg, dev, route=None, anchor=False):
    if cfg.name == "larger_backbone":
        if route is not None or anchor:
            return RoutedBackbone(cfg, dev, route or (cfg.recent // cfg.frame_tokens, 0, 0, 0), anchor)
        return LargerBackbone(cfg, dev)
    if cfg.name == "streaming":
        return Streaming(cfg, dev)
    return SingleLayer(cfg, dev)


# ------------------------------------------------------------------------------ CPU oracle baseline
def cpu_baseline_tempo(cfg):
    """The oracle's predictive residual codec (oracle/tempo.py) on one head of the
    layer: encode of its six frames (anchor, then five), timed as tokens/s."""
    import numpy as np
    import oracle
    import synth
    S = cfg.frame_tokens
    k = synth.AR1Stream(cfg, "k", heads=1).tokens(cfg.hist)
    v = synth.coupled_values(k, synth.AR1Stream(cfg, "v", heads=1).tokens(cfg.hist), synth.seed_for(cfg.seed, 0, 1, 2))
    kn, vn = k[0].float().numpy(), v[0].float().numpy()
    rng = np.random.default_rng(cfg.seed)
    d = cfg.dim
    P = oracle.tempo.join_params(0.05 * rng.standard_normal(d), rng.uniform(0.6, 1.0, d), 0.05 * rng.standard_normal(d),
                                 rng.uniform(0.4, 0.9, d), rng.uniform(-0.2, 0.3, d), 0.05 * rng.standard_normal(d),
                                 rng.uniform(0.0, 0.6, d), 0.6 * rng.standard_normal((d, d)) / np.sqrt(d))
    ba = oracle.tempo.anchor_bits(cfg.k_bits, cfg.v_bits)
    t0 = time.perf_counter()
    a = oracle.tempo.encode_frames(kn[:S], vn[:S], P, 0, S, ba, ba, cfg.group)
    oracle.tempo.encode_frames(kn[S:], vn[S:], P, 1, S, cfg.k_bits, cfg.v_bits, cfg.group, a[6])
    dt = time.perf_counter() - t0
    return {"tempo_encode_tokens_per_s": cfg.hist / dt,
            "tempo_sample": f"oracle predictive encode of 1 head x {cfg.hist // S} frames x {S} tokens"}


def cpu_baseline(cfg, budget_s):
    """Time the oracle (as it stands) on a bounded sample of the workload: the
    fp64 attention of all queries over the history the timed step attends, head
    after head, until the time budget is spent or every generated head is done.
    The history has the workload's segment structure (streaming: the step-10
    history of ten chunks, each with its own centre table; long history: eight
    segments sharing one table).  The codes come from the oracle's own encoder
    (timed too) with centres drawn from the tokens; ids from the expanded
    distance."""
    import numpy as np
    import torch
    import oracle
    import synth
    from threadpoolctl import threadpool_info

    if cfg.name == "streaming":
        N, bounds, own_tables = cfg.hist, [cfg.chunk * i for i in range(cfg.steps + 1)], True
        H = min(cfg.heads, 16)
    elif cfg.name == "larger_backbone":
        N, bounds, own_tables = cfg.recent, [0, cfg.recent], False
        H = min(cfg.heads, 16)
    else:
        N = cfg.hist
        bounds, own_tables = [N * i // cfg.n_segments for i in range(cfg.n_segments + 1)], False
        H = min(cfg.heads, 16)
    if cfg.dtype == "f32":
        k, _ = synth.tiny_kv(cfg, "k")
        v, _ = synth.tiny_kv(cfg, "v")
    else:
        k = synth.AR1Stream(cfg, "k", heads=H).tokens(N)
        v = synth.AR1Stream(cfg, "v", heads=H).tokens(N)
    q_all = synth.queries(cfg, heads=H)
    H = min(H, k.shape[0])
    C = cfg.n_centroids
    rng = np.random.default_rng(cfg.seed)

    def ids_of(x, c):
        xt, ct = torch.from_numpy(x.astype(np.float64)), torch.from_numpy(c.astype(np.float64))
        return ((ct * ct).sum(1)[None] - 2 * xt @ ct.T).argmin(1).numpy()

    t_att = t_enc = 0.0
    flops = 0.0
    n_enc = heads_done = nq_total = 0
    wall0 = time.perf_counter()
    for h in range(H):
        if h > 0 and time.perf_counter() - wall0 > budget_s:
            break
        kn, vn = k[h].float().numpy(), v[h].float().numpy()
        segs = []
        for si, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
            if own_tables or si == 0:
                base = (a, b) if own_tables else (0, N)
                span = base[1] - base[0]
                kc = kn[base[0]:base[1]][rng.choice(span, min(C, span), replace=False)]
                vc = vn[base[0]:base[1]][rng.choice(span, min(C, span), replace=False)]
            kid, vid = ids_of(kn[a:b], kc), ids_of(vn[a:b], vc)
            t0 = time.perf_counter()
            kcodes, kmeta = oracle.encode(kn[a:b], kc, kid, cfg.k_bits, cfg.group)
            vcodes, vmeta = oracle.encode(vn[a:b], vc, vid, cfg.v_bits, cfg.group)
            t_enc += time.perf_counter() - t0
            n_enc += 2 * (b - a)
            segs.append(oracle.Segment(kcodes, kmeta, kid, kc, vcodes, vmeta, vid, vc, cfg.k_bits, cfg.v_bits,
                                       cfg.group))
        q = q_all[h].float().numpy()
        t0 = time.perf_counter()
        oracle.attend(q, segs)
        t_att += time.perf_counter() - t0
        flops += 4.0 * len(q) * N * cfg.dim
        nq_total += len(q)
        heads_done += 1
    threads = 1
    for info in threadpool_info():
        threads = max(threads, int(info.get("num_threads", 1)))
    hist = f"{N} history tokens in {len(bounds) - 1} segment(s)"
    if cfg.name == "streaming":
        hist = f"the step-{cfg.steps} history of {N} tokens in {cfg.steps} chunks with their own centre tables"
    return {
        "value": flops / t_att / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"fp64 attention of {heads_done} head(s) x {nq_total // max(heads_done, 1)} queries over "
                  f"{hist} (d={cfg.dim}); oracle encode of the same heads' K and V ({n_enc} token rows)",
        "encode_tokens_per_s": n_enc / t_enc if t_enc > 0 else None,
        "seconds": t_att + t_enc,
        "cpu_count_affinity": len(os.sched_getaffinity(0)),
    }


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, scaled against a copy of known size), or
    None when there is none or the attention source has changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_attend_kernel_{workload}.md")
    src = os.path.join(ROOT, "compressed_kv_cache_kvc_amd", "csrc", "attend.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("attend.hip sha256") != sha or "traffic bytes per launch" not in fields:
        return None
    return int(float(fields["traffic bytes per launch"]))


def fit_kernel_rates(w, cfg):
    """The fit's two kernels on one streaming chunk's keys (720 heads x 4680
    tokens), measured after the timed steps with HIP events on the launch stream
    (median of 5): one assignment pass (n_iter = 0) against the bf16 MFMA peak
    (2*C*d FLOP per token) and HBM (the tokens and the centre tables read, the ids
    written), and the centre update (an n_iter = 1 fit less its two assignment
    passes, each timed alone) against HBM (the tokens and ids read, the centres
    written)."""
    import compressed_kv_cache_kvc_amd as kvc
    torch = w.torch
    k, _, _, kc0, _ = w.chunks[-1]
    H, N = k.shape[0], k.shape[1]

    def timed(c0, n_iter):
        ts = []
        for _ in range(5):
            c = c0.clone()
            a = w.ev()
            kvc.fit_assign(k, c, n_iter=n_iter)
            b = w.ev()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return sorted(ts)[2]

    # the second pass of an n_iter = 1 fit scores against the moved centres, whose
    # flag rate differs: time that pass on its own too
    c1 = kc0.clone()
    kvc.fit_assign(k, c1, n_iter=1)
    t_a = timed(kc0, 0)
    t_a1 = timed(c1, 0)
    t_u = max(timed(kc0, 1) - t_a - t_a1, 1e-9)
    flop = 2.0 * H * N * cfg.n_centroids * cfg.dim
    tok_b = H * N * cfg.dim * 2
    cen_b = H * cfg.n_centroids * cfg.dim * 2
    a_bytes = tok_b + cen_b + H * N
    u_bytes = tok_b + H * N + cen_b
    return {"tokens": H * N,
            "assign_ms": round(t_a * 1e3, 4), "assign_TFLOPs": round(flop / t_a / 1e12, 1),
            "assign_pct_bf16_peak": round(100.0 * flop / t_a / 1e12 / PEAK_MFMA_TFLOPS, 2),
            "assign_GBps": round(a_bytes / t_a / 1e9, 1), "assign_pct_hbm": round(100.0 * a_bytes / t_a / 1e9 / PEAK_HBM_GBS, 2),
            "update_ms": round(t_u * 1e3, 4), "update_GBps": round(u_bytes / t_u / 1e9, 1),
            "update_pct_hbm": round(100.0 * u_bytes / t_u / 1e9 / PEAK_HBM_GBS, 2)}


# ------------------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the hot path runs on "
              "one GPU; across GPUs it would be split by head, which needs no communication)", file=sys.stderr)
        sys.exit(2)
    import torch
    import compressed_kv_cache_kvc_amd as kvc
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kvc.library()
    cfg = synth.get_config(args.workload)
    route = tuple(int(v) for v in args.route.split(",")) if args.route else None
    if route is not None and len(route) != 4:
        raise SystemExit("--route takes RECENT,PERIOD,SINK,ALL_FULL_UNTIL")
    if (route is not None or args.anchor) and cfg.name != "larger_backbone":
        raise SystemExit("--route and --anchor apply to the larger_backbone workload")
    if args.tempo:
        if cfg.name != "self_forcing_layer":
            raise SystemExit("--tempo covers the self_forcing_layer workload")
        w = TempoLayer(cfg, dev)
    else:
        w = make_workload(cfg, dev, route, args.anchor)
    if args.psac:
        if not hasattr(w, "enable_psac"):
            raise SystemExit("--psac covers the single-segment workloads (self_forcing_layer, streaming)")
        w.enable_psac()
    if args.qsac:
        if not hasattr(w, "enable_qsac"):
            raise SystemExit("--qsac covers the single-segment workloads (self_forcing_layer, streaming, tiny)")
        w.enable_qsac(args.qsac)
    torch.cuda.synchronize()
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration * (1 << 18), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    w.collect()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        w.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phases = w.collect()
    K = args.steps
    ms_step = wall * 1e3 / K
    attend_ms = phases.get("attend", 0.0) / K
    lowdim_ms = phases.get("attend_lowdim", 0.0) / K
    encode_ms = phases.get("encode", 0.0) / K
    fit_ms = phases.get("fit", 0.0) / K
    attn_ms_total = attend_ms + lowdim_ms + phases.get("lse_merge", 0.0) / K
    value = w.attn_flops / (attn_ms_total * 1e-3) / 1e12

    # roofline of the full-dim attention kernel (the dominant launch)
    if cfg.name == "larger_backbone":
        fl = 4.0 * cfg.heads * cfg.n_q * w.full_tokens * cfg.dim
        launches = 1
    elif cfg.name == "streaming":
        fl = w.attn_flops
        launches = cfg.steps
    else:
        fl = w.attn_flops
        launches = 1
    achieved = fl / launches / (attend_ms / launches * 1e-3) / 1e12 if attend_ms > 0 else 0.0
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MFMA_TFLOPS, 4), "traffic": measured_traffic(cfg.name),
                "kernel": "attend_kernel", "flops_per_launch": fl / launches,
                "avg_launch_ms": attend_ms / launches}
    enc_s = encode_ms * 1e-3
    line = {
        "metric": "compressed-history attention TFLOP/s (% bf16 MFMA peak); encode tokens/s, HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if cfg.dtype == "bf16" else "f32",
        "dtype_detail": ("attention products on f16 MFMA tiles (bf16 inputs widened exactly), f32 accumulation "
                         "and softmax; codes u8" if cfg.dtype == "bf16" else "f32 throughout"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "heads": cfg.heads, "head_dim": cfg.dim, "history": cfg.hist,
                   "queries": cfg.n_q, "centroids": cfg.n_centroids, "k_bits": cfg.k_bits, "v_bits": cfg.v_bits,
                   "group": cfg.group, "segments": cfg.n_segments, "far": cfg.far, "rank": cfg.rank,
                   "steps": cfg.steps},
        "pct_mfma_peak": round(100.0 * value / PEAK_MFMA_TFLOPS, 2),
        "encode_tokens_per_s": round(w.enc_tokens / enc_s, 1) if enc_s > 0 else None,
        "encode_GBps": round(w.enc_bytes / enc_s / 1e9, 1) if enc_s > 0 else None,
        "phase_ms": {"fit": round(fit_ms, 4), "encode": round(encode_ms, 4), "attend": round(attend_ms, 4),
                     "attend_lowdim": round(lowdim_ms, 4),
                     "lse_merge": round(phases.get("lse_merge", 0.0) / K, 4)},
        "roofline": roofline,
    }
    if isinstance(w, RoutedBackbone):
        line["config"]["route"] = list(w.route)
        line["config"]["anchor_bits"] = w.anchor_bits if w.anchor else None
        line["config"]["full_dim_tokens"] = w.full_tokens
        line["config"]["far"] = w.low_tokens
    if cfg.name == "larger_backbone" and lowdim_ms > 0:
        # the far part is bound by the softmax's vector work rather than the
        # matrix cores: one exponential per score.  Transcendental instructions
        # issue at a quarter of the fp32 vector rate: 256 CUs x 4 SIMDs x 16
        # lanes / 4 per clock at 2.4 GHz
        scores = float(cfg.heads) * cfg.n_q * w.low_tokens
        exp_peak = 256 * 4 * 16 / 4 * 2.4e9
        line["lowdim"] = {"ms": round(lowdim_ms, 4),
                          "TFLOP/s": round((4.0 * cfg.heads * cfg.n_q * w.low_tokens * cfg.rank
                                            + 4.0 * cfg.heads * cfg.n_q * cfg.dim * cfg.rank) / (lowdim_ms * 1e-3) / 1e12, 2),
                          "scores_per_s": round(scores / (lowdim_ms * 1e-3), 1),
                          "exp_peak_per_s": exp_peak,
                          "exp_bound_frac": round(scores / (lowdim_ms * 1e-3) / exp_peak, 4)}
        # the low-dim encode of the far part (K and V): a = U^T r with every
        # multiply and add rounded separately (2*d*r vector operations per token,
        # no fused multiply-add, so no packed or matrix unit applies); its bound is
        # one fp32 operation per lane and clock: 256 CUs x 64 lanes x 2.4 GHz
        el = phases.get("encode_lowdim", 0.0) / K * 1e-3
        if el > 0:
            ops = 2.0 * cfg.heads * w.low_tokens * 2.0 * cfg.dim * cfg.rank
            valu_peak = 256 * 64 * 2.4e9
            line["phase_ms"]["encode_lowdim"] = round(el * 1e3, 4)
            line["encode_lowdim"] = {"ms": round(el * 1e3, 4),
                                     "tokens_per_s": round(2.0 * cfg.heads * w.low_tokens / el, 1),
                                     "valu_TOPs": round(ops / el / 1e12, 3),
                                     "valu_peak_TOPs": valu_peak / 1e12,
                                     "valu_frac": round(ops / el / valu_peak, 4)}
    if isinstance(w, TempoLayer):
        # the predictions cost 2*d*d FLOP per value token (W K_hat, multiply and add
        # rounded separately) plus 6*d for the key and the temporal terms; the
        # reference rate of separately rounded fp32 operations is one per lane and
        # clock: 256 CUs x 64 lanes x 2.4 GHz = 39.3 TFLOP/s
        te = phases.get("tempo_encode", 0.0) / K * 1e-3
        td = phases.get("tempo_decode", 0.0) / K * 1e-3
        pred_tokens = cfg.heads * (cfg.hist - w.S)
        pred_flop = pred_tokens * (2.0 * cfg.dim * cfg.dim + 6.0 * cfg.dim)
        valu_peak = 256 * 64 * 2.4e9
        line["config"]["codec"] = "tempo"
        line["config"]["anchor_bits"] = w.anchor_bits
        line["phase_ms"]["tempo_encode"] = round(te * 1e3, 4)
        line["phase_ms"]["tempo_decode"] = round(td * 1e3, 4)
        line["tempo"] = {"encode_tokens_per_s": round(w.enc_tokens / te, 1) if te else None,
                         "decode_tokens_per_s": round(w.enc_tokens / td, 1) if td else None,
                         "encode_GBps": round(w.enc_bytes / te / 1e9, 1) if te else None,
                         "prediction_TFLOPs_encode": round(pred_flop / te / 1e12, 3) if te else None,
                         "prediction_TFLOPs_decode": round(pred_flop / td / 1e12, 3) if td else None,
                         "valu_peak_TFLOPs": valu_peak / 1e12,
                         "encode_valu_frac": round(pred_flop / te / valu_peak, 4) if te else None}
    if w.psac:
        for name in ("psac_coeffs", "query_moments", "psac_basis"):
            line["phase_ms"][name] = round(phases.get(name, 0.0) / K, 4)
        line["psac"] = {"rank": 8, "attention_includes_compensation": True}
    if w.qsac:
        # keys re-assigned per step: H*N tokens (all chunks for streaming); the
        # weighted distances are 2*C*d FLOP per token, the tokens are read once
        qs = phases.get("qsac", 0.0) / K * 1e-3
        qtok = w.enc_tokens
        line["phase_ms"]["qsac"] = round(qs * 1e3, 4)
        line["phase_ms"]["query_stats"] = round(phases.get("query_stats", 0.0) / K, 4)
        line["qsac"] = {"n_cand": w.qsac, "tokens_per_s": round(qtok / qs, 1) if qs > 0 else None,
                        "distance_TFLOPs": round(2.0 * qtok * cfg.n_centroids * cfg.dim / qs / 1e12, 2) if qs else None,
                        "read_GBps": round(qtok * cfg.dim * (4 if cfg.dtype == "f32" else 2) / qs / 1e9, 1) if qs else None}
    if isinstance(w, Streaming):
        line["fit_kernels"] = fit_kernel_rates(w, cfg)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
        if isinstance(w, TempoLayer):
            line["cpu_baseline"].update(cpu_baseline_tempo(cfg))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
