"""Pins for the oracle's OCP e4m3fn encoder and decoder.

The pages name the format (float8_e4m3fn, TileKernels article section 3.1)
but print no codes, so the encoder is pinned to the format definition:
hand-worked codes (tests/golden/e4m3_codes.txt), torch's own e4m3fn decode
table and cast (a library routine) inside the finite range, and brute-force
nearest-value search with ties to the even mantissa over all bf16 patterns,
every midpoint +-1 ulp and a large random fp32 sample.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.txt")


def _torch_decode_table():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return codes.to(torch.float32).numpy()


def _nearest_even_codes(x):
    """Brute-force reference: nearest e4m3 magnitude (ties -> even code), saturating."""
    table = _torch_decode_table()
    pos_vals = table[:0x7F].astype(np.float64)  # codes 0x00..0x7E, ascending
    x = np.asarray(x, np.float32)
    a = np.abs(x).astype(np.float64)
    hi = np.clip(np.searchsorted(pos_vals, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = np.abs(a - pos_vals[lo])
    d_hi = np.abs(pos_vals[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a >= 464.0, 0x7E, code).astype(np.uint8)  # past the format: saturate
    sign = np.signbit(x).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def test_golden_hand_worked_codes():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v, c = line.split()[:2]
            rows.append((float(v), int(c, 16)))
    assert len(rows) >= 15
    vals = np.array([r[0] for r in rows], np.float32)
    want = np.array([r[1] for r in rows], np.uint8)
    got = oracle.e4m3_encode(vals)
    assert [hex(c) for c in got] == [hex(c) for c in want]


def test_decode_matches_torch_table():
    table = _torch_decode_table()
    mine = oracle.e4m3_decode(np.arange(256))
    finite = ~np.isnan(table)
    assert np.array_equal(np.isnan(mine), ~finite)
    assert np.array_equal(mine[finite].view(np.uint32), table[finite].view(np.uint32))
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def test_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_all_bf16_patterns_nearest_even():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle.e4m3_encode(x), _nearest_even_codes(x))


def test_midpoints_and_neighbours():
    table = _torch_decode_table()[:0x7F].astype(np.float32)
    mids = ((table[:-1].astype(np.float64) + table[1:].astype(np.float64)) / 2).astype(np.float32)
    # every midpoint is exact in fp32 (e4m3 needs 4 significant bits)
    assert np.array_equal(mids.astype(np.float64), (table[:-1].astype(np.float64) + table[1:]) / 2)
    xs = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                         np.nextafter(mids, np.float32(0))])
    xs = np.concatenate([xs, -xs])
    assert np.array_equal(oracle.e4m3_encode(xs), _nearest_even_codes(xs))


def test_random_fp32_nearest_even():
    rng = np.random.default_rng(1234)
    n = 4_000_000
    mag = np.exp2(rng.uniform(-14.0, 9.2, n)).astype(np.float32)
    x = np.where(rng.random(n) < 0.5, -mag, mag).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(x), _nearest_even_codes(x))


def test_matches_torch_cast_inside_range():
    rng = np.random.default_rng(99)
    x = (rng.standard_normal(1_000_000) * 60).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = oracle.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("v,code", [(464.0, 0x7E), (465.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E),
                                    (-np.inf, 0xFE), (-500.0, 0xFE), (np.nan, 0x7F)])
def test_saturation_and_nan(v, code):
    assert int(oracle.e4m3_encode(np.array([v], np.float32))[0]) == code
