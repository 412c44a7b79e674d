"""Pins for the oracle's top-k gating, weights and token map.

Top-k (TileKernels article section 2.1: K rounds of max, lowest index among
equal maxima, winner masked to -inf) is pinned to a brute-force stable sort
of (-score, index) on many tiny inputs with forced ties (including -0/+0),
to numpy's argmax (first index on ties) at K = 1 and to the full sort at
K = E.  The token map (section 2 group counting + token-expert mapping; the
Perplexity local kernel) is pinned to a lexicographic sort of
(expert, token, k) triples and to its invariants.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _brute_topk(s, K):
    out = []
    for row in s:
        order = sorted(range(len(row)), key=lambda i: (-float(row[i]), i))
        out.append(order[:K])
    return np.array(out, np.int64)


@pytest.mark.parametrize("E,K", [(4, 1), (4, 2), (8, 3), (16, 2), (16, 8), (13, 5), (16, 16)])
def test_topk_brute_force_random(E, K):
    rng = np.random.default_rng(E * 100 + K)
    s = rng.standard_normal((300, E)).astype(np.float32)
    idx, _ = oracle.topk_gate(s, K)
    assert np.array_equal(idx, _brute_topk(s, K))


@pytest.mark.parametrize("E,K", [(4, 2), (8, 4), (16, 6), (16, 16), (5, 5)])
def test_topk_forced_ties(E, K):
    rng = np.random.default_rng(E + K)
    vals = np.array([-1.0, 0.0, -0.0, 0.5, 1.0], np.float32)
    s = vals[rng.integers(0, len(vals), (500, E))]
    idx, _ = oracle.topk_gate(s, K)
    assert np.array_equal(idx, _brute_topk(s, K))


def test_topk_signed_zero_is_a_tie():
    s = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    idx, _ = oracle.topk_gate(s, 3)
    assert idx.tolist() == [[0, 1, 3]]
    s = np.array([[0.0, -0.0, -1.0, -0.0]], np.float32)
    idx, _ = oracle.topk_gate(s, 3)
    assert idx.tolist() == [[0, 1, 3]]


def test_topk_k1_is_argmax():
    rng = np.random.default_rng(5)
    s = rng.integers(-3, 3, (1000, 64)).astype(np.float32)
    idx, _ = oracle.topk_gate(s, 1)
    assert np.array_equal(idx[:, 0], np.argmax(s, axis=1))


def test_topk_k_equals_e_is_full_sort():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((50, 32)).astype(np.float32)
    idx, _ = oracle.topk_gate(s, 32)
    assert np.array_equal(idx, np.argsort(-s, axis=1, kind="stable"))


def test_topk_neg_inf_and_nan():
    # NaN reads as -inf.  Once only -inf is left, the lowest -inf index wins,
    # even one already taken (the masked winner is -inf too).
    s = np.array([[np.nan, 2.0, -np.inf, 1.0]], np.float32)
    idx, _ = oracle.topk_gate(s, 4)
    assert idx.tolist() == [[1, 3, 0, 0]]


def test_weights_renormalised():
    w = W.WORKLOADS["dsv3"]
    s = W.make_scores(w, num_tokens=512)
    idx, wt = oracle.topk_gate(s, 8, renormalize=True)
    g = np.take_along_axis(s, idx, axis=1).astype(np.float64)
    exact = g / g.sum(axis=1, keepdims=True)
    assert np.all(np.abs(wt - exact) <= 4 * np.spacing(exact.astype(np.float32)))
    assert np.all(np.abs(wt.astype(np.float64).sum(axis=1) - 1.0) <= 8 * 2.0 ** -23)
    assert np.all(np.diff(wt, axis=1) <= 0)
    # raw gather without renormalisation
    _, raw = oracle.topk_gate(s, 8, renormalize=False, with_weights=True)
    assert np.array_equal(raw, g.astype(np.float32))


def _brute_map(idx, E):
    T, K = idx.shape
    triples = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K) if 0 <= idx[t, k] < E)
    pos = -np.ones((T, K), np.int32)
    for r, (e, t, k) in enumerate(triples):
        pos[t, k] = r
    counts = np.bincount([e for e, _, _ in triples], minlength=E).astype(np.int32)
    return counts, pos


@pytest.mark.parametrize("T,E,K", [(1, 4, 1), (37, 16, 2), (64, 16, 2), (200, 8, 8), (333, 64, 6)])
def test_map_brute_force(T, E, K):
    rng = np.random.default_rng(T + E + K)
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = oracle.topk_gate(s, K)
    counts, offsets, pos, row_token = oracle.token_map(idx, E)
    bc, bpos = _brute_map(idx, E)
    assert np.array_equal(counts, bc)
    assert np.array_equal(pos, bpos)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert counts.sum() == T * K
    assert np.array_equal(np.sort(pos.ravel()), np.arange(T * K))
    for e in range(E):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) >= 0)
        assert all(e in idx[t] for t in seg)


def test_map_duplicates_and_out_of_range():
    idx = np.array([[3, 3, -1], [5, 0, 3], [2, 7, 0]], np.int64)
    counts, offsets, pos, row_token = oracle.token_map(idx, 6)
    bc, bpos = _brute_map(idx, 6)
    assert np.array_equal(counts, bc) and np.array_equal(pos, bpos)
    assert pos[0, 2] == -1 and pos[2, 1] == -1
    assert offsets[-1] == 7
    assert np.all(row_token[7:] == -1)


def test_map_empty_tokens():
    counts, offsets, pos, row_token = oracle.token_map(np.zeros((0, 4), np.int64), 8)
    assert np.all(counts == 0) and np.all(offsets == 0) and pos.size == 0


def test_large_workload_is_skewed():
    w = W.WORKLOADS["large"]
    s = W.make_scores(w)
    idx, _ = oracle.topk_gate(s, w.num_topk)
    counts, offsets, _, _ = oracle.token_map(idx, w.num_experts)
    assert counts.sum() == w.num_tokens * w.num_topk
    assert (counts == 0).sum() >= 8
    # an empty expert repeats its offset
    z = np.nonzero(counts == 0)[0]
    assert np.all(offsets[z] == offsets[z + 1])


def test_topk_repeats_only_expert_zero():
    """The one case where a token's ids repeat (fewer than K scores above -inf, NaN counting as -inf): every
    further round's maximum is -inf, every entry ties at -inf, so the lowest index, 0, is picked again
    ("DeepSeek open-sources TileKernels", section 2.1, masking).  No other id ever repeats, which the fused
    routing's count kernel relies on; rows with enough finite scores never repeat."""
    rng = np.random.default_rng(0)
    repeats = 0
    for _ in range(200):
        T, E = 32, int(rng.choice([1, 2, 3, 8, 16, 64, 256]))
        K = int(rng.integers(1, min(E, 16) + 1))
        s = rng.standard_normal((T, E)).astype(np.float32)
        s[rng.random((T, E)) < rng.random()] = -np.inf
        s[rng.random((T, E)) < 0.05] = np.nan
        s[rng.random((T, E)) < 0.05] = np.inf
        idx, _ = oracle.topk_gate(s, K)
        finite_or_inf = (s > -np.inf).sum(axis=1)  # NaN compares False: counts as -inf
        for t in range(T):
            vals, counts = np.unique(idx[t], return_counts=True)
            rep = vals[counts > 1]
            if finite_or_inf[t] >= K:
                assert rep.size == 0
            elif rep.size:
                repeats += 1
                assert np.array_equal(rep, [0])
    assert repeats > 100
