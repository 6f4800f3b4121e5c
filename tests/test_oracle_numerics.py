"""Pins of the oracle's rounding helpers against table-driven exact definitions.

Every finite fp16 / bf16 value is enumerated from its bit pattern and held as a
float64 (exact: both formats, and every midpoint of two neighbours, fit in
fp64's 53-bit significand).  Directed and nearest-even rounding are then
defined by searching that sorted table; ties go to the neighbour whose bit
pattern has an even last bit.
"""
import numpy as np
import pytest

from oracle import fp16_round, round_to_bf16, round_to_f32


def _table_f16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    bits, vals = bits[ok], vals[ok]
    # drop -0 so that the table is strictly increasing; +0 (bits 0) stays
    keep = ~((vals == 0) & (bits != 0))
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


def _table_bf16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals)
    bits, vals = bits[ok], vals[ok]
    keep = ~((vals == 0) & (bits != 0))
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


def _exact_round(x, table, tbits, mode):
    """Round each x to the table by definition: down = largest <= x, up =
    smallest >= x, nearest = closer neighbour, ties to the even bit pattern."""
    x = np.asarray(x, np.float64)
    hi = np.searchsorted(table, x, side="left")       # first table value >= x
    hi = np.clip(hi, 0, len(table) - 1)
    exact = table[hi] == x
    lo = np.where(exact, hi, np.clip(hi - 1, 0, len(table) - 1))
    down = table[lo]
    up = table[hi]
    if mode == "down":
        return down
    if mode == "up":
        return up
    dl = x - down
    du = up - x
    pick_up = (du < dl) | ((du == dl) & (tbits[hi] % 2 == 0) & ~exact)
    return np.where(exact, x, np.where(pick_up, up, down))


def _f16_probe_values(rng):
    table, _ = _table_f16()
    pos = table[table > 0]
    mids = (pos[1:] + pos[:-1]) / 2
    v = [rng.standard_normal(20000) * 10.0 ** rng.uniform(-8, 4, 20000),
         rng.choice(pos, 4000), -rng.choice(pos, 4000),
         rng.choice(mids, 4000), -rng.choice(mids, 4000),
         np.array([0.0, -0.0, 65504.0, -65504.0, 6.103515625e-05, 6.097555160522461e-05,
                   5.960464477539063e-08, 2.9802322387695312e-08, 1.0, 2.0, 0.5, 1024.0, 2048.0])]
    v = np.concatenate(v).astype(np.float32)
    v = v[np.abs(v.astype(np.float64)) <= 65504.0]
    # also the fp32 neighbours of table values and midpoints
    near = np.concatenate([np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))])
    near = near[np.abs(near.astype(np.float64)) <= 65504.0]
    return np.concatenate([v, near])


@pytest.mark.parametrize("mode", ["down", "up", "nearest"])
def test_fp16_rounding_matches_exact_definition(mode):
    rng = np.random.default_rng(1)
    v = _f16_probe_values(rng)
    table, tbits = _table_f16()
    want = _exact_round(v.astype(np.float64), table, tbits, mode)
    got = fp16_round(v, mode).astype(np.float64)
    bad = got != want
    assert not bad.any(), (v[bad][:5], got[bad][:5], want[bad][:5])


def test_fp16_directed_brackets_and_range():
    v = np.array([65504.0, -65504.0, 1.0 + 2.0 ** -20], np.float32)
    assert fp16_round(v, "down")[2] == np.float16(1.0)
    assert fp16_round(v, "up")[2] == np.float16(1.0 + 2.0 ** -10)
    with pytest.raises(ValueError):
        fp16_round(np.array([65504.5], np.float32), "up")
    with pytest.raises(ValueError):
        fp16_round(np.array([np.nan], np.float32), "down")


def test_bf16_rne_from_fp64_matches_exact_definition():
    rng = np.random.default_rng(2)
    table, tbits = _table_bf16()
    pos = table[(table > 0) & (table < 1e30)]
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-40, 30, 20000),
        rng.choice(mids, 5000), -rng.choice(mids, 5000),
        rng.choice(pos, 2000),
        np.nextafter(rng.choice(mids, 2000), np.inf), np.nextafter(rng.choice(mids, 2000), -np.inf),
        np.array([0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** -133, 2.0 ** -134,
                  3 * 2.0 ** -135, 2.0 ** -126 * (1 - 2.0 ** -9)]),
    ])
    want = _exact_round(x, table, tbits, "nearest")
    got = round_to_bf16(x).astype(np.float64)
    bad = got != want
    assert not bad.any(), (x[bad][:5], got[bad][:5], want[bad][:5])


def test_bf16_mean_tie_goes_to_even():
    # the mean of bf16 1.0 and its successor 1 + 2^-7 lies exactly halfway
    assert round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == np.float32(1.0)
    assert round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == np.float32(1.0 + 2.0 ** -6)


def test_f32_rne_from_fp64_matches_correctly_rounded_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.uniform(-44, 37, 50000),
                        np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 2.0 ** -149, 2.0 ** -150,
                                  3 * 2.0 ** -150, 0.0])])
    want = x.astype(np.float32)   # IEEE conversion, round to nearest even
    got = round_to_f32(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
