"""Pins for the oracle's format-general cast: OCP FP4 e2m1 codes, groups of
16/32/128, power-of-two scales (round_sf), UE8M0 scale bytes, the e2m1 clamp
("DeepSeek open-sources TileKernels", section 3.1: CastOutputConfig with
round_sf and clamp_min_value = max_value * 2^-126 for float4_e2m1fn;
"CuTeDSL at Perplexity", Blackwell section: absmax over 16 or 32 elements for
NVFP4 and MXFP8/MXFP4).

The encoder is pinned by hand-worked codes (tests/golden/e2m1_codes.txt) and
by the properties that define round-to-nearest-even with saturation: every
code decodes to a value that encodes back to it, the error is at most half
the local spacing, a value exactly between two neighbours takes the even
code, and the map is monotone.  Scales are pinned by exact rational
arithmetic and, for round_sf, by minimality among powers of two.  The
format-general expand and SwiGLU reduce to the pinned e4m3/128 functions.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_codes.txt")
E2M1, E4M3 = oracle.FMT_E2M1, oracle.FMT_E4M3


def _bits_value(code):
    """e2m1 value from its bit fields (sign, 2-bit exponent with bias 1, 1-bit mantissa)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    v = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
    return -v if s else v


def test_decode_matches_bit_fields():
    for c in range(16):
        assert oracle.e2m1_decode(np.array([c]))[0] == _bits_value(c)


def test_golden_hand_worked_codes():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    vals = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    assert len(rows) >= 20
    assert np.array_equal(oracle.e2m1_encode(vals), want)


def test_round_trip_every_code():
    codes = np.arange(16, dtype=np.uint8)
    back = oracle.e2m1_encode(oracle.e2m1_decode(codes))
    assert np.array_equal(back, codes)


def test_nearest_with_ties_to_even_and_saturation():
    mags = sorted({abs(_bits_value(c)) for c in range(8)})
    grid = np.concatenate([np.linspace(-8, 8, 4097, dtype=np.float32),
                           np.array([(a + b) / 2 for a, b in zip(mags, mags[1:])], np.float32)])
    grid = np.concatenate([grid, np.nextafter(grid, np.float32(np.inf)), np.nextafter(grid, np.float32(-np.inf))])
    codes = oracle.e2m1_encode(grid)
    vals = oracle.e2m1_decode(codes)
    for x, c, v in zip(grid.tolist(), codes.tolist(), vals.tolist()):
        assert (c >= 8) == (np.signbit(np.float32(x)))
        a = abs(x)
        if a >= 6:
            assert c & 7 == 7
            continue
        lo = max(m for m in mags if m <= a)
        hi = min(m for m in mags if m >= a)
        assert abs(v) in (lo, hi)
        if lo == hi:  # representable: exact
            assert abs(v) == a
        elif a - lo < hi - a:
            assert abs(v) == lo
        elif a - lo > hi - a:
            assert abs(v) == hi
        else:  # exact midpoint: the even code
            assert (c & 1) == 0
    pos = grid[grid >= 0]
    order = np.argsort(pos, kind="stable")
    assert np.all(np.diff(oracle.e2m1_decode(oracle.e2m1_encode(pos[order]))) >= 0)


@pytest.mark.parametrize("dtype", [E4M3, E2M1])
def test_scale_is_the_exact_quotient(dtype):
    rng = np.random.default_rng(3 + dtype)
    maxv = Fraction(oracle.FMT_MAX[dtype])
    clamp = Fraction(oracle.default_clamp(dtype))
    for i in range(300):
        v = (rng.standard_normal(32) * 2.0 ** rng.integers(-30, 20)).astype(np.float32)
        _, sf = oracle.cast_group_fmt(v, dtype)
        c = max(Fraction(float(np.abs(v).max())), clamp)
        exact = c / maxv
        # sf is the fp32 nearest to the exact quotient
        up = Fraction(float(np.nextafter(sf, np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(sf, np.float32(0))))
        s = Fraction(float(sf))
        assert abs(s - exact) <= abs(up - exact) and abs(s - exact) <= abs(dn - exact)


def test_e2m1_clamp_is_max_times_2_pow_minus_126():
    assert oracle.default_clamp(E2M1) == np.float32(6 * 2.0 ** -126)
    for rnd in (False, True):
        q, sf = oracle.cast_group_fmt(np.array([0.0, -0.0] * 16, np.float32), E2M1, round_sf=rnd)
        assert sf == np.float32(2.0 ** -126)
        assert q.tolist() == [0x0, 0x8] * 16


@pytest.mark.parametrize("dtype", [E4M3, E2M1])
def test_round_sf_is_the_smallest_sufficient_power_of_two(dtype):
    rng = np.random.default_rng(11 + dtype)
    maxv = oracle.FMT_MAX[dtype]
    for i in range(400):
        v = (rng.standard_normal(32) * 2.0 ** rng.integers(-40, 40)).astype(np.float32)
        if i % 7 == 0:  # exact powers of two times the format maximum
            v[0] = np.float32(maxv * 2.0 ** rng.integers(-20, 20))
        q, sf = oracle.cast_group_fmt(v, dtype, round_sf=True)
        c = max(float(np.abs(v).max()), float(oracle.default_clamp(dtype)))
        m, e = np.frexp(np.float64(sf))
        assert m == 0.5, sf  # a power of two
        assert float(sf) * maxv >= c
        assert float(sf) / 2 * maxv < c
        # nothing saturates: every scaled value is within the format
        assert np.all(np.abs(v.astype(np.float64) / float(sf)) <= maxv)


def test_custom_clamp():
    v = np.full(32, 1e-3, np.float32)
    _, sf = oracle.cast_group_fmt(v, E4M3, clamp_min=0.5)
    assert sf == np.float32(0.5) / np.float32(448)
    _, sf = oracle.cast_group_fmt(v, E2M1, round_sf=True, clamp_min=3.0)
    assert sf == np.float32(0.5)  # 0.5 * 6 >= 3 > 0.25 * 6


def test_ue8m0_bytes_are_ieee_exponents():
    for e in range(-126, 128):
        p = np.float32(2.0 ** e)
        assert oracle.ue8m0_encode(p) == (int(p.view(np.uint32)) >> 23) & 0xFF == e + 127
        assert oracle.ue8m0_decode(e + 127) == p
    assert oracle.ue8m0_encode(np.float32(2.0 ** -127)) == 0


def test_worked_e2m1_group():
    v = np.array([6, 3, 1.5, -0.75, 0.25, 5, -6, 0.1] + [0] * 24, np.float32)
    q, sf = oracle.cast_group_fmt(v, E2M1)  # amax 6: sf = 6 / 6 = 1
    assert sf == 1.0
    assert q[:8].tolist() == [0x7, 0x5, 0x3, 0xA, 0x0, 0x6, 0xF, 0x0]


def test_dequantisation_error_bound():
    rng = np.random.default_rng(21)
    for dtype, rel in ((E4M3, 2.0 ** -4), (E2M1, 2.0 ** -2)):
        for rnd in (False, True):
            v = (rng.standard_normal(128) * 3).astype(np.float32)
            q, sf = oracle.cast_group_fmt(v, dtype, round_sf=rnd)
            dec = oracle.e2m1_decode(q) if dtype == E2M1 else oracle.e4m3_decode(q)
            err = np.abs(dec.astype(np.float64) * float(sf) - v)
            # half a step of the binade of |v|, or half the smallest step near zero
            step = np.maximum(np.abs(v).astype(np.float64) * rel * 2, float(sf) * (0.5 if dtype == E2M1 else 2.0 ** -9))
            assert np.all(err <= step / 2 * 1.0001 + 1e-30)


def test_group_size_nesting():
    """Each 128-group built from four 32-groups of equal amax: the 32-group
    cast equals the 128-group cast (same scale, same codes); 16 likewise."""
    rng = np.random.default_rng(31)
    H = 1024
    x = rng.standard_normal((4, H)).astype(np.float32)
    for g in range(H // 16):
        x[:, g * 16] = np.float32(9.5) * np.sign(x[:, g * 16] + 0.5)  # same amax in every 16-group
    xb = W.f32_to_bf16_bits(x)
    for dtype in (E4M3, E2M1):
        q128, s128, _ = oracle.expand_cast(xb, dtype=dtype, group_size=128)
        for gs in (16, 32):
            q, s, _ = oracle.expand_cast(xb, dtype=dtype, group_size=gs)
            assert np.array_equal(q, q128)
            assert np.array_equal(s, np.repeat(s128, 128 // gs, axis=1))


def test_e4m3_128_reduces_to_the_pinned_functions():
    rng = np.random.default_rng(41)
    T, H, K = 37, 512, 4
    x = W.f32_to_bf16_bits((rng.standard_normal((T, H)) * 4).astype(np.float32))
    pos = rng.permutation(T * K).astype(np.int32).reshape(T, K)
    w = rng.random((T, K), dtype=np.float32)
    a = oracle.expand_cast(x, pos, w)
    b = oracle.expand_cast_fp8(x, pos, w)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    gu = W.f32_to_bf16_bits(rng.standard_normal((19, 512)).astype(np.float32))
    rw = rng.random(19, dtype=np.float32)
    for clamp in (0.0, 1.5):
        a = oracle.swiglu_cast(gu, rw, clamp)
        b = oracle.swiglu_cast_fp8(gu, rw, clamp)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_e2m1_packing_and_ue8m0_rows():
    rng = np.random.default_rng(51)
    T, H = 9, 256
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    q, sf, _ = oracle.expand_cast(x, dtype=E2M1, group_size=32, round_sf=True)
    qb, sfb, _ = oracle.expand_cast(x, dtype=E2M1, group_size=32, round_sf=True, sf_ue8m0=True)
    assert q.shape == (T, H // 2) and sfb.dtype == np.uint8
    assert np.array_equal(q, qb)
    assert np.array_equal(sfb, ((sf.view(np.uint32) >> 23) & 0xFF).astype(np.uint8))
    codes = oracle.unpack_e2m1(q, H)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    for t in range(T):
        for g in range(H // 32):
            cg, sg = oracle.cast_group_fmt(xf[t, g * 32:(g + 1) * 32], E2M1, round_sf=True)
            assert np.array_equal(codes[t, g * 32:(g + 1) * 32], cg) and sg == sf[t, g]


def test_invalid_formats_rejected():
    x = np.zeros((2, 128), np.uint16)
    with pytest.raises(ValueError):
        oracle.expand_cast(x, sf_ue8m0=True)  # UE8M0 needs power-of-two scales
    with pytest.raises(ValueError):
        oracle.expand_cast(x, dtype=5)


def test_fmt_tolerance_rejects_planted_errors():
    from oracle.compare import fmt_tolerance_report
    rng = np.random.default_rng(61)
    gu = W.f32_to_bf16_bits(rng.standard_normal((8, 256)).astype(np.float32))
    for dtype in (E4M3, E2M1):
        q, sf = oracle.swiglu_cast(gu, dtype=dtype, group_size=32)
        assert fmt_tolerance_report(q, sf, q, sf, dtype, 32)[0]
        bad_sf = sf.copy()
        bad_sf[3, 2] *= np.float32(1 + 1e-5)
        assert not fmt_tolerance_report(q, bad_sf, q, sf, dtype, 32)[0]
        bad_q = q.copy()
        # far more than one step: e2m1 2.0 -> 6.0 in a low nibble; e4m3 two binades up
        if dtype == E2M1:
            j = int(np.argmax((q[0] & 0x7) == 0x4))
            assert (q[0, j] & 0x7) == 0x4
            bad_q[0, j] = q[0, j] | 0x7
        else:
            bad_q[0, 0] = q[0, 0] + 16
        assert not fmt_tolerance_report(bad_q, sf, q, sf, dtype, 32)[0]
        qr, sfr = oracle.swiglu_cast(gu, dtype=dtype, group_size=32, round_sf=True, sf_ue8m0=True)
        bad = sfr.copy()
        bad[1, 1] += 1  # scale doubled where no code sits at a binade edge
        assert fmt_tolerance_report(qr, sfr, qr, sfr, dtype, 32, sf_ue8m0=True, round_sf=True)[0]
        ok, _ = fmt_tolerance_report(qr, bad, qr, sfr, dtype, 32, sf_ue8m0=True, round_sf=True)
        assert not ok
