"""Pins of the oracle's SiLU over the whole working range of the gate
("DeepSeek open-sources TileKernels", section 3.3: the SwiGLU value is
silu(l) * u with silu(l) = l / (1 + exp(-l)), fused with the per-token cast
of section 3.2).

The cast hides values behind one e4m3 step (up to 1/16 relative), too coarse
to tell silu from a close relative (GELU x * Phi(x), or a swish
x * sigmoid(beta * x) with beta != 1).  The group scale is much finer: for a
group whose entries all equal v, amax = |v| and sf = fl(|v| / 448), so
sf * 448 gives |v| to one fp32 rounding.  So each test row holds one bf16
gate value l in every column (up = a power of two 2^k, exact, chosen to lift
|v| above the 1e-4 clamp), and the row's scale pins the oracle's fp32 silu(l)
against math.exp in float64, within a few fp32 ulp.

Every bf16 value in [-20, 20] is covered, subnormals included: about 34 000
gate values, each through both oracle entry points that evaluate the SwiGLU
(the e4m3 / 128 one and the block-scaled one).  Separately, random groups
check every dequantised value (not only the group maximum) against the
float64 formula within half an e4m3 step.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W

# Relative bound on |sf * 448 - |silu(l)| * u| / (|silu(l)| * u): expf within
# 1 ulp, then rounding of 1 + e, of the division, of the scale division (each
# 2^-24 relative): well under 8 ulp of fp32.
REL_TOL = 2.0 ** -20


def silu64(l):
    """silu in float64, from the definition."""
    l = float(l)
    if l < -700:  # exp overflows float64: silu(l) rounds to -0 anyway
        return -0.0
    return l / (1.0 + math.exp(-l))


def all_bf16_in(lo, hi):
    """Every finite bf16 bit pattern with value in [lo, hi] (uint16), with its fp32 value."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = W.bf16_bits_to_f32(bits)
    keep = np.isfinite(vals) & (vals >= lo) & (vals <= hi)
    # one pattern for zero (drop -0; +0 is pinned separately by the zero-gate test)
    keep &= ~((vals == 0) & (bits == 0x8000))
    return bits[keep], vals[keep]


def lift_exponent(s):
    """k such that |s| * 2^k lies in [2^-8, 2^-7): above the 1e-4 clamp and far from fp32 overflow."""
    if s == 0.0:
        return 0
    return int(-8 - math.floor(math.log2(abs(s))))


def rows_for(gate_bits, gate_vals, inter=128):
    """gate_up rows: row r = [l_r repeated inter times | 2^k_r repeated inter times]."""
    ks = np.array([lift_exponent(silu64(v)) for v in gate_vals], np.int64)
    assert ks.min() >= -126 and ks.max() <= 127
    up = np.ldexp(np.float32(1.0), ks).astype(np.float32)
    up_bits = W.f32_to_bf16_bits(up)
    assert np.array_equal(W.bf16_bits_to_f32(up_bits), up)  # powers of two: exact in bf16
    R = gate_bits.size
    gu = np.empty((R, 2 * inter), np.uint16)
    gu[:, :inter] = gate_bits[:, None]
    gu[:, inter:] = up_bits[:, None]
    return gu, ks


def check_scales(sf, codes, gate_vals, ks, entry):
    ref = np.array([silu64(v) for v in gate_vals], np.float64)
    lifted = np.abs(ref) * np.ldexp(1.0, ks)
    got = sf.astype(np.float64) * 448.0
    nz = ref != 0.0
    rel = np.abs(got[nz] - lifted[nz]) / lifted[nz]
    worst = int(np.argmax(rel)) if rel.size else 0
    assert rel.size and rel.max() <= REL_TOL, (
        f"{entry}: oracle silu off at l={gate_vals[nz][worst]!r}: rel err {rel.max():.3e}")
    # sign: every code of the row is the e4m3 maximum with the sign of silu(l)
    expect = np.where(ref < 0, 0xFE, 0x7E).astype(np.uint8)
    assert np.all(codes[nz] == expect[nz][:, None]), f"{entry}: group codes are not +-448"


@pytest.fixture(scope="module")
def gate_range():
    bits, vals = all_bf16_in(-20.0, 20.0)
    assert bits.size > 30000
    return bits, vals


def test_silu_every_bf16_gate_fp8_entry(gate_range):
    bits, vals = gate_range
    gu, ks = rows_for(bits, vals)
    q, sf = oracle.swiglu_cast_fp8(gu)
    check_scales(sf[:, 0], q, vals, ks, "swiglu_cast_fp8")


def test_silu_every_bf16_gate_block_scaled_entry(gate_range):
    bits, vals = gate_range
    gu, ks = rows_for(bits, vals, inter=32)
    q, sf = oracle.swiglu_cast(gu, dtype=oracle.FMT_E4M3, group_size=32)
    check_scales(sf[:, 0], q, vals, ks, "swiglu_cast")


@pytest.mark.parametrize("l,expected", [
    (1.0, 0.7310585786300049),     # 1 / (1 + e^-1)
    (-1.0, -0.2689414213699951),
    (2.0, 1.7615941559557649),
    (-4.0, -0.07194483984836625),
    (0.5, 0.3112296656009273),
])
def test_silu_hand_values(l, expected):
    """Values of l * sigmoid(l) worked by hand (not from the code under test):
    GELU gives 0.8413 at l = 1 and a swish with beta = 1.1 gives 0.7503, so
    either fails here by orders of magnitude more than the tolerance."""
    assert abs(silu64(l) - expected) <= 1e-15
    bits = W.f32_to_bf16_bits(np.array([l], np.float32))
    gu, ks = rows_for(bits, W.bf16_bits_to_f32(bits))
    q, sf = oracle.swiglu_cast_fp8(gu)
    got = float(sf[0, 0]) * 448.0 * math.ldexp(1.0, -int(ks[0]))
    assert abs(got - abs(expected)) <= REL_TOL * abs(expected)
    assert q[0, 0] == (0xFE if expected < 0 else 0x7E)


@pytest.mark.parametrize("seed", [0, 1])
def test_dequantised_values_follow_float64_silu(seed):
    """Random N(0,3) gates, N(0,1) up values, U(0,1) row weights: each code,
    dequantised with its group scale, lies within half an e4m3 step (at the
    code's magnitude, scaled) of the float64 value silu(l) * u * w, plus a
    few fp32 ulp for the fp32 evaluation."""
    rng = np.random.default_rng(seed)
    R, I = 64, 256
    gate = W.f32_to_bf16_bits((rng.standard_normal((R, I)) * 3).astype(np.float32))
    up = W.f32_to_bf16_bits(rng.standard_normal((R, I)).astype(np.float32))
    w = rng.random(R, dtype=np.float32)
    gu = np.concatenate([gate, up], axis=1)
    q, sf = oracle.swiglu_cast_fp8(gu, w)
    lv = W.bf16_bits_to_f32(gate).astype(np.float64)
    uv = W.bf16_bits_to_f32(up).astype(np.float64)
    exact = np.vectorize(silu64)(lv) * uv * w.astype(np.float64)[:, None]
    s = np.repeat(sf.astype(np.float64), 128, axis=1)
    codes = oracle.e4m3_decode(q).astype(np.float64)
    half_step = 0.5 * _e4m3_step(codes) * s
    err = np.abs(codes * s - exact)
    assert np.all(err <= half_step * (1 + 2.0 ** -10) + np.abs(exact) * 2.0 ** -20)


def _e4m3_step(c):
    c = np.abs(c)
    return np.where(c < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(c, 2.0 ** -6))) - 3))
