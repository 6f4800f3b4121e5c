"""Frame routing of mixed-dimensional attention and the anchor precision rule.
TEST INFRASTRUCTURE ONLY (part of the oracle package).

* route_frames -- NanoKV-Fast reads part of the history at full dimension and the
  rest through the reduced maps (NanoKV, Figure 4; appendix Table 7 lists the
  deployed rules: recent frames, a sink frame, periodic anchors among the older
  frames, or the whole history during the first chunks).  Reading: frame f of a
  history of F latent frames (0 = oldest) is read at full dimension when
    F <= all_full_until, or f >= F - n_recent, or f < n_sink,
    or (period > 0 and f % period == 0);
  "one anchor per P older frames" is the first frame of every P-frame window.
* anchor_bits -- the anchor frame is quantized at b_a = max(4, b_K, b_V)
  (TempoKV, section 3.3 "Anchor frames" and appendix A.3, Table 7).

Pinned by tests/test_oracle_routing.py against the deployed rules of the
appendix table, worked by hand.
"""
from __future__ import annotations


def route_frames(n_frames: int, n_recent: int, period: int = 0, n_sink: int = 0,
                 all_full_until: int = 0) -> list[bool]:
    """Per frame (oldest first): True when read at full dimension."""
    F = n_frames
    out = []
    for f in range(F):
        full = (F <= all_full_until) or (f >= F - n_recent) or (f < n_sink) or (period > 0 and f % period == 0)
        out.append(bool(full))
    return out


def runs(mask: list[bool]) -> list[tuple[int, int, bool]]:
    """Maximal runs (first frame, end frame, full) of equal routing, in order."""
    out = []
    f = 0
    while f < len(mask):
        e = f
        while e < len(mask) and mask[e] == mask[f]:
            e += 1
        out.append((f, e, mask[f]))
        f = e
    return out


def anchor_bits(k_bits: int, v_bits: int) -> int:
    """b_a = max(4, b_K, b_V)."""
    return max(4, k_bits, v_bits)
