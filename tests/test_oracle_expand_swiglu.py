"""Pins for the oracle's expand+cast (TileKernels article section 2.2 with
the section 3.2 cast) and SwiGLU+cast (section 3.3).

Expand: the expanded rows are a permutation of token copies (each token's
cast row appears exactly K times, at the rows the map gives it), identity
mode is the per-token cast, and rows no copy lands in are untouched.
SwiGLU: w = None equals w = 1 bit for bit; power-of-two weights scale the
scales exactly; for gate >= 17, silu(gate) == gate in fp32 so the group
values are exact products (checked against the cast of numpy's exact
products); gate = 0 gives zeros; gate <= -89 gives -0; the clamp clips
both halves.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _bf16(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def _cast_rows(v):
    """Cast each 128-group of fp32 rows with the group oracle."""
    R, n = v.shape
    q = np.empty((R, n), np.uint8)
    sf = np.empty((R, n // 128), np.float32)
    for r in range(R):
        for g in range(n // 128):
            q[r, g * 128:(g + 1) * 128], sf[r, g] = oracle.cast_group(v[r, g * 128:(g + 1) * 128])
    return q, sf


def test_identity_mode_is_per_token_cast():
    rng = np.random.default_rng(0)
    x = _bf16(rng.standard_normal((9, 384)) * 3)
    q, sf, _ = oracle.expand_cast_fp8(x)
    q2, sf2 = _cast_rows(W.bf16_bits_to_f32(x))
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)


@pytest.mark.parametrize("T,E,K,H", [(64, 16, 2, 256), (50, 32, 4, 512)])
def test_expand_is_permutation_of_token_copies(T, E, K, H):
    rng = np.random.default_rng(T)
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, wt = oracle.topk_gate(s, K, renormalize=False, with_weights=True)
    counts, offsets, pos, row_token = oracle.token_map(idx, E)
    x = _bf16(rng.standard_normal((T, H)))
    q_id, sf_id, _ = oracle.expand_cast_fp8(x)
    q, sf, ow = oracle.expand_cast_fp8(x, pos, wt)
    assert np.array_equal(q, q_id[row_token])
    assert np.array_equal(sf, sf_id[row_token])
    assert np.bincount(row_token, minlength=T).tolist() == [K] * T
    for t in range(T):
        for k in range(K):
            assert ow[pos[t, k]] == wt[t, k]
            assert np.array_equal(q[pos[t, k]], q_id[t])


def test_expand_skips_negative_pos_and_keeps_other_rows():
    x = _bf16(np.arange(2 * 128).reshape(2, 128) / 7.0)
    pos = np.array([[1, -1], [3, 0]], np.int32)
    out = (np.full((4, 128), 0xAB, np.uint8), np.full((4, 1), -5.0, np.float32), None)
    q, sf, _ = oracle.expand_cast_fp8(x, pos, out=out)
    q_id, sf_id, _ = oracle.expand_cast_fp8(x)
    assert np.all(q[2] == 0xAB) and sf[2, 0] == -5.0
    assert np.array_equal(q[1], q_id[0]) and np.array_equal(q[3], q_id[1])
    assert np.array_equal(q[0], q_id[1])


def test_swiglu_weight_none_equals_one():
    rng = np.random.default_rng(1)
    gu = _bf16(rng.standard_normal((16, 512)))
    a = oracle.swiglu_cast_fp8(gu)
    b = oracle.swiglu_cast_fp8(gu, np.ones(16, np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_swiglu_power_of_two_weights_scale_exactly():
    rng = np.random.default_rng(2)
    gu = _bf16(rng.standard_normal((16, 512)))
    q1, s1 = oracle.swiglu_cast_fp8(gu)
    w = np.float32(2.0) ** rng.integers(-6, 4, 16).astype(np.float32)
    qw, sw = oracle.swiglu_cast_fp8(gu, w)
    # groups whose amax stays above the 1e-4 clamp scale exactly
    ok = (s1 * w[:, None] > np.float32(1e-4) / np.float32(448)) & (s1 > np.float32(1e-4) / np.float32(448))
    assert np.all(sw[ok] == (s1 * w[:, None])[ok])
    rows = np.all(ok, axis=1)
    assert np.array_equal(qw[rows], q1[rows])


def test_swiglu_large_gate_is_exact_product():
    # For gate >= 17, exp(-gate) < 2^-24 so 1 + exp(-gate) rounds to 1 and
    # silu(gate) == gate; bf16 x bf16 products are exact in fp32.
    rng = np.random.default_rng(3)
    R, I = 8, 256
    gate = rng.uniform(17, 60, (R, I)).astype(np.float32)
    up = rng.standard_normal((R, I)).astype(np.float32)
    gu = np.concatenate([_bf16(gate), _bf16(up)], axis=1)
    gate_b, up_b = W.bf16_bits_to_f32(gu[:, :I]), W.bf16_bits_to_f32(gu[:, I:])
    q, sf = oracle.swiglu_cast_fp8(gu)
    q2, sf2 = _cast_rows((gate_b * up_b).astype(np.float32))
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)
    # the halves are not interchangeable: swapping them changes the result
    qs, _ = oracle.swiglu_cast_fp8(np.concatenate([gu[:, I:], gu[:, :I]], axis=1))
    assert not np.array_equal(qs, q)


def test_swiglu_zero_and_very_negative_gate():
    R, I = 2, 128
    up = np.linspace(-3, 3, I).astype(np.float32)
    gu = np.concatenate([_bf16(np.zeros((R, I))), _bf16(np.tile(up, (R, 1)))], axis=1)
    q, sf = oracle.swiglu_cast_fp8(gu)
    assert np.all((q & 0x7F) == 0)
    gu = np.concatenate([_bf16(np.full((R, I), -100.0)), _bf16(np.tile(up, (R, 1)))], axis=1)
    q, sf = oracle.swiglu_cast_fp8(gu)
    # l / inf = -0; -0 * u keeps the product sign
    assert np.all((q & 0x7F) == 0)
    assert np.array_equal(q[0] == 0x80, up > 0)


def test_swiglu_odd_part_identity():
    # silu(l) - silu(-l) = l: compare dequantised rows for +l and -l with u = 1.
    rng = np.random.default_rng(4)
    I = 128
    l = rng.uniform(0.1, 6.0, I).astype(np.float32)
    lb = W.bf16_bits_to_f32(_bf16(l))
    ones = np.ones(I, np.float32)
    gp = np.concatenate([_bf16(lb), _bf16(ones)])[None, :]
    gn = np.concatenate([_bf16(-lb), _bf16(ones)])[None, :]
    qp, sp = oracle.swiglu_cast_fp8(gp)
    qn, sn = oracle.swiglu_cast_fp8(gn)
    vp = oracle.e4m3_decode(qp[0]).astype(np.float64) * sp[0, 0]
    vn = oracle.e4m3_decode(qn[0]).astype(np.float64) * sn[0, 0]
    # each dequantised value is within 1/16 relative (+ one subnormal step)
    tol = np.abs(vp) / 16 + np.abs(vn) / 16 + 2.0 ** -9 * (sp[0, 0] + sn[0, 0])
    assert np.all(np.abs((vp - vn) - lb) <= tol)
    assert np.all(vp > 0) and np.all(vn <= 0)


def test_swiglu_clamp():
    rng = np.random.default_rng(5)
    R, I, c = 4, 128, 20.0
    gate = rng.uniform(17, 40, (R, I)).astype(np.float32)
    up = (rng.standard_normal((R, I)) * 30).astype(np.float32)
    gu = np.concatenate([_bf16(gate), _bf16(up)], axis=1)
    g = np.minimum(W.bf16_bits_to_f32(gu[:, :I]), np.float32(c))
    u = np.clip(W.bf16_bits_to_f32(gu[:, I:]), -np.float32(c), np.float32(c))
    q, sf = oracle.swiglu_cast_fp8(gu, clamp_value=c)
    q2, sf2 = _cast_rows((g * u).astype(np.float32))
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)
