"""Pins for the oracle's per-group e4m3 cast (TileKernels article sections
3.1 and 3.2: amax per 128-channel group, amax clamped below at 1e-4 for
e4m3, sf = amax / 448, codes = e4m3(x * (1 / sf))).

The scale factor is checked against exact rational arithmetic (Fraction),
worked groups with power-of-two scales reduce the codes to the bare encoder,
and invariants that hold for every group (a code of magnitude 448 in every
group whose amax reaches the clamp, the dequantisation error bound, exact
scaling by powers of two) catch a dropped clamp, a wrong constant, a wrong
inverse or a lost sign.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rn32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even), normal range."""
    f64 = float(fr)  # correctly rounded to fp64 first
    c = np.float32(f64)
    # fix a possible double-rounding case by checking neighbours exactly
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    dist = [abs(Fraction(float(x)) - fr) for x in cands]
    best = min(dist)
    ties = [x for x, d in zip(cands, dist) if d == best]
    if len(ties) == 1:
        return ties[0]
    return [x for x in ties if (int(np.float32(x).view(np.uint32)) & 1) == 0][0]


def test_worked_group_scale_one():
    # amax == 448 gives sf = 448/448 = 1 exactly and inv = 1: codes are the bare encoder.
    v = np.zeros(128, np.float32)
    v[:6] = [448.0, 1.0, -2.0, 0.1, 240.0, -0.375]
    q, sf = oracle.cast_group(v)
    assert sf == np.float32(1.0)
    assert [hex(c) for c in q[:6]] == ["0x7e", "0x38", "0xc0", "0x1d", "0x77", "0xac"]
    assert np.all(q[6:] == 0)


def test_worked_group_scale_half():
    # amax == 224: sf = 0.5, inv = 2, codes of 2*v.
    v = np.zeros(128, np.float32)
    v[:4] = [224.0, 0.5, -1.0, 120.0]
    q, sf = oracle.cast_group(v)
    assert sf == np.float32(0.5)
    assert [hex(c) for c in q[:4]] == ["0x7e", "0x38", "0xc0", "0x77"]


def test_zero_group_uses_clamp():
    q, sf = oracle.cast_group(np.zeros(128, np.float32))
    want = _rn32(Fraction(float(np.float32(1e-4))) / 448)
    assert sf.view(np.uint32) == want.view(np.uint32) == np.uint32(0x346FACAD)
    assert np.all(q == 0)
    qn, _ = oracle.cast_group(-np.zeros(128, np.float32))
    assert np.all(qn == 0x80)


def test_tiny_group_clamped():
    v = np.full(128, 3e-5, np.float32)
    q, sf = oracle.cast_group(v)
    assert sf == np.float32(np.float32(1e-4) / np.float32(448))
    # 3e-5 * inv = 134.4; the e4m3 spacing in [128, 256) is 16, so the code is 128 (0x70)
    assert np.all(q == 0x70)


@pytest.mark.parametrize("seed", range(6))
def test_scale_exact_and_invariants(seed):
    rng = np.random.default_rng(seed)
    for trial in range(200):
        scale = np.float32(2.0 ** rng.uniform(-20, 12))
        v = (rng.standard_normal(128) * scale).astype(np.float32)
        if trial % 7 == 0:
            v[rng.integers(0, 128)] *= 50  # an outlier
        q, sf = oracle.cast_group(v)
        amax = np.max(np.abs(v))
        amax_c = max(amax, np.float32(1e-4))
        want_sf = _rn32(Fraction(float(amax_c)) / 448)
        assert sf.view(np.uint32) == want_sf.view(np.uint32)
        inv = _rn32(1 / Fraction(float(sf)))
        dec = oracle.e4m3_decode(q).astype(np.float64)
        # signs are kept
        assert np.all((q >= 0x80) == np.signbit(v))
        # a code of magnitude 448 wherever amax reached the clamp
        if amax >= np.float32(1e-4):
            assert np.any((q & 0x7F) == 0x7E)
        # dequantisation: |dec - v*inv| <= half the e4m3 spacing at that magnitude
        y = np.abs(v.astype(np.float64) * float(inv))
        spacing = np.where(y < 2.0 ** -6, 2.0 ** -9,
                           2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
        err = np.abs(np.abs(dec) - y)
        assert np.all(err <= spacing / 2 + y * 2.0 ** -23)


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(128).astype(np.float32)
    q0, sf0 = oracle.cast_group(v)
    for k in (-8, -3, 1, 5, 10):
        q, sf = oracle.cast_group((v * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(q, q0)
        assert sf == np.float32(sf0 * np.float32(2.0 ** k))


def test_one_over_sf_not_448_over_amax():
    # The inverse is 1/sf (the pages multiply by the inverse of SF).  Where
    # 1/sf and 448/amax differ by an ulp, build a value whose product with
    # the two inverses lands on either side of a code midpoint, and check the
    # oracle took the 1/sf side.
    rng = np.random.default_rng(11)
    mids = np.float32([1.0625, 3.125, 13.5, 54.0, 200.0, 432.0])  # e4m3 code midpoints
    found = 0
    for _ in range(2000):
        amax = np.float32(rng.uniform(0.5, 8.0))
        sf = np.float32(amax / np.float32(448))
        inv_a = np.float32(np.float32(1.0) / sf)
        inv_b = np.float32(np.float32(448) / amax)
        if inv_a == inv_b:
            continue
        for m in mids:
            v = np.float32(m / inv_a)
            for _step in range(4):
                ca = oracle.e4m3_encode(np.array([v * inv_a], np.float32))[0]
                cb = oracle.e4m3_encode(np.array([v * inv_b], np.float32))[0]
                if ca != cb:
                    g = np.zeros(128, np.float32)
                    g[0], g[1] = amax, v
                    q, s = oracle.cast_group(g)
                    assert s == sf and q[1] == ca
                    found += 1
                    break
                v = np.nextafter(v, np.float32(np.inf))
        if found >= 5:
            return
    assert found > 0
