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
