"""Planted-error tests of the SwiGLU tolerance checker (oracle/compare.py),
the comparison behind every e4m3 / 128 SwiGLU parity assertion and the
smoke check.  The agreed tolerance ("DeepSeek open-sources TileKernels",
section 3.3 evaluates exp in fp32, so an implementation with another exp
differs by a few ulp): scales within 1e-6 relative, dequantised values
within one e4m3 step at the larger code magnitude.

Each test starts from the oracle's own output (which must pass against
itself), plants one mistake, and checks the report: mistakes inside the
tolerance pass, mistakes outside fail and are counted.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.compare import swiglu_tolerance_report


@pytest.fixture(scope="module")
def ref():
    rng = np.random.default_rng(7)
    R, I = 16, 512
    gu = W.f32_to_bf16_bits(rng.standard_normal((R, 2 * I)).astype(np.float32))
    w = rng.random(R, dtype=np.float32)
    q, sf = oracle.swiglu_cast_fp8(gu, w)
    return q, sf


def _check(q, sf, ref):
    return swiglu_tolerance_report(q, sf, ref[0], ref[1])


def test_identical_outputs_pass(ref):
    ok, det = _check(ref[0].copy(), ref[1].copy(), ref)
    assert ok and det["codes_differing"] == 0 and det["max_sf_rel_err"] == 0.0


def test_scale_off_by_1e5_relative_fails(ref):
    sf = ref[1].copy()
    sf[3, 1] = np.float32(sf[3, 1] * (1 + 1e-5))
    ok, det = _check(ref[0].copy(), sf, ref)
    assert not ok and det["max_sf_rel_err"] > 1e-6


def test_scale_off_by_5e7_relative_passes(ref):
    sf = ref[1].copy()
    sf[3, 1] = np.float32(sf[3, 1] * (1 + 5e-7))
    ok, det = _check(ref[0].copy(), sf, ref)
    assert ok and 0 < det["max_sf_rel_err"] <= 1e-6


def _bump(code, steps):
    """The e4m3 code `steps` positions further from zero (same sign)."""
    return np.uint8((int(code) & 0x80) | ((int(code) & 0x7F) + steps))


def test_code_one_step_away_passes(ref):
    q = ref[0].copy()
    r, j = 5, 77
    assert 0x08 <= (q[r, j] & 0x7F) < 0x7E  # a normal code with a neighbour
    q[r, j] = _bump(q[r, j], 1)
    ok, det = _check(q, ref[1].copy(), ref)
    assert ok and det["codes_differing"] == 1 and det["codes_out_of_tol"] == 0


def test_code_two_binades_away_fails(ref):
    q = ref[0].copy()
    r, j = 6, 200
    c = int(q[r, j])
    assert 0x08 <= (c & 0x7F) < 0x6E  # room for two binades (16 codes) above
    q[r, j] = _bump(c, 16)
    ok, det = _check(q, ref[1].copy(), ref)
    assert not ok and det["codes_out_of_tol"] == 1


def test_code_sign_flip_fails(ref):
    q = ref[0].copy()
    r, j = 2, 300
    assert (q[r, j] & 0x7F) >= 0x20  # far from zero
    q[r, j] ^= 0x80
    ok, det = _check(q, ref[1].copy(), ref)
    assert not ok and det["codes_out_of_tol"] == 1


def test_transposed_group_scales_fail(ref):
    """A layout mistake: the scales of a row written in the wrong group order."""
    sf = ref[1].copy()
    sf[4] = sf[4, ::-1]
    assert not np.array_equal(sf[4], ref[1][4])
    ok, _ = _check(ref[0].copy(), sf, ref)
    assert not ok


def _tie_group(ref):
    """A (row, group, column) whose scale mantissa is below 1.5 (so one fp32 ulp is more than 7.9e-8 of it)
    and whose column holds a code of at least 208 with a neighbour above (together: the scale term exceeds the
    checker's 2^-20 rounding slack)."""
    q, sf = ref
    for r in range(sf.shape[0]):
        for g in range(sf.shape[1]):
            if np.frexp(sf[r, g])[0] * 2 >= 1.5:
                continue
            cols = np.nonzero(((q[r, g * 128:(g + 1) * 128] & 0x7F) >= 0x75)
                              & ((q[r, g * 128:(g + 1) * 128] & 0x7F) < 0x7E))[0]
            if cols.size:
                return r, g, g * 128 + int(cols[0])
    raise AssertionError("no group with a large code and a low scale mantissa")


def test_tie_rounded_the_other_way_under_a_scale_one_ulp_away_passes(ref):
    """A value at a rounding tie (x / sf = 232 between codes 224 and 240) with a scale one fp32 ulp
    larger rounds one step up: the scale and the code are each inside the tolerance, so the pair is
    too, although the dequantised difference exceeds one step at the larger scale."""
    r, g, j = _tie_group(ref)
    q, sf = ref[0].copy(), ref[1].copy()
    sf[r, g] = np.nextafter(sf[r, g], np.float32(np.inf))
    q[r, j] = _bump(q[r, j], 1)
    c_new = float(oracle.e4m3_decode(q[r, j:j + 1])[0])
    c_old = float(oracle.e4m3_decode(ref[0][r, j:j + 1])[0])
    step = abs(c_new) - abs(c_old)
    assert abs(c_new * np.float64(sf[r, g]) - c_old * np.float64(ref[1][r, g])) > step * np.float64(sf[r, g]) * (1 + 2.0 ** -20)
    ok, det = _check(q, sf, ref)
    assert ok and det["codes_differing"] == 1 and det["codes_out_of_tol"] == 0


def _two_steps(code):
    """Two codes away with both steps inside one binade (0x78 = 256 starts a binade: go up from it)."""
    return 2 if (int(code) & 0x7F) == 0x78 else -2


def test_code_two_steps_away_under_a_scale_one_ulp_away_fails(ref):
    r, g, j = _tie_group(ref)
    q, sf = ref[0].copy(), ref[1].copy()
    sf[r, g] = np.nextafter(sf[r, g], np.float32(np.inf))
    q[r, j] = _bump(q[r, j], _two_steps(q[r, j]))
    ok, det = _check(q, sf, ref)
    assert not ok and det["codes_out_of_tol"] == 1


def test_format_report_composes_the_same_way(ref):
    """The format-aware report (e4m3 / 128 / fp32 scales here) accepts the same tie and rejects two steps."""
    from oracle.compare import fmt_tolerance_report
    r, g, j = _tie_group(ref)
    for steps, want in ((1, True), (_two_steps(ref[0][r, j]), False)):
        q, sf = ref[0].copy(), ref[1].copy()
        sf[r, g] = np.nextafter(sf[r, g], np.float32(np.inf))
        q[r, j] = _bump(q[r, j], steps)
        ok, _ = fmt_tolerance_report(q, sf, ref[0], ref[1], oracle.FMT_E4M3, 128)
        assert ok is want
