"""Pins for the oracle's combine (the weighted reduce back to token order:
"CuTeDSL at Perplexity", MoE dispatch and combine; the "Fused
Expand/Reduce" step of the TileKernels routing chain, section 2).

out[t] = bf16(sum over k in k order of w[t,k] * y_rows[pos[t,k]]), fp32
products and sums.  Pinned by: the bf16 encoder against torch's own cast;
K = 1 is an exact gather; small-integer data whose fp32 sums are exact
against numpy; a cancellation case that only the k-ordered fp32 sum gives;
skipped positions; invariance under a consistent permutation of rows and
positions; w = None equals w = 1.
"""
import numpy as np
import torch

import oracle
import workloads as W


def _bf16(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.float32(2.0) ** rng.integers(-60, 60, 200_000)).astype(np.float32)
    # exact ties: low 16 bits == 0x8000, both parities of the kept bit occur
    ties = ((rng.standard_normal(4000).astype(np.float32).view(np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, np.inf, -np.inf])])
    assert np.all(np.isfinite(x[:-2]))
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), want)


def test_k1_is_exact_gather():
    rng = np.random.default_rng(1)
    y = _bf16(rng.standard_normal((40, 256)))
    pos = rng.permutation(40)[:30].astype(np.int32).reshape(30, 1)
    out = oracle.combine(y, pos)
    assert np.array_equal(out, y[pos[:, 0]])


def test_small_integers_are_exact():
    rng = np.random.default_rng(2)
    T, K, H = 50, 8, 128
    R = T * K
    y = rng.integers(-4, 5, (R, H)).astype(np.float32)
    w = np.float32(2.0) ** rng.integers(-2, 2, (T, K)).astype(np.float32)
    pos = rng.permutation(R).astype(np.int32).reshape(T, K)
    out = oracle.combine(_bf16(y), pos, w)
    exact = np.einsum("tk,tkh->th", w.astype(np.float64), y[pos].astype(np.float64))
    assert np.array_equal(W.bf16_bits_to_f32(out).astype(np.float64), exact)


def test_sum_runs_in_k_order():
    # 2^25 + 1 rounds back to 2^25 in fp32, so (2^25 + 1) - 2^25 == 0, while
    # any order that cancels first gives 1.
    y = _bf16([[2.0 ** 25], [1.0], [-(2.0 ** 25)]])
    pos = np.array([[0, 1, 2]], np.int32)
    assert W.bf16_bits_to_f32(oracle.combine(y, pos))[0, 0] == 0.0
    pos = np.array([[0, 2, 1]], np.int32)
    assert W.bf16_bits_to_f32(oracle.combine(y, pos))[0, 0] == 1.0


def test_skipped_positions_and_default_weight():
    rng = np.random.default_rng(3)
    y = _bf16(rng.standard_normal((20, 128)))
    pos = np.array([[3, -1, 7], [-1, -1, -1], [25, 2, 4]], np.int32)  # 25 >= R: skipped too
    out = oracle.combine(y, pos)
    assert np.array_equal(out[1], np.zeros(128, np.uint16))
    ref = oracle.combine(y, np.array([[3, 7], [-1, -1], [2, 4]], np.int32))
    assert np.array_equal(out[[0, 2]], ref[[0, 2]])
    assert np.array_equal(oracle.combine(y, pos, np.ones((3, 3), np.float32)), out)


def test_row_permutation_invariance():
    rng = np.random.default_rng(4)
    T, K, H = 30, 4, 256
    R = T * K
    y = _bf16(rng.standard_normal((R, H)))
    pos = rng.permutation(R).astype(np.int32).reshape(T, K)
    w = rng.random((T, K), dtype=np.float32)
    perm = rng.permutation(R)
    inv = np.argsort(perm)
    out = oracle.combine(y, pos, w)
    out2 = oracle.combine(y[perm], inv[pos].astype(np.int32), w)
    assert np.array_equal(out, out2)
