"""Property-based pins of the oracle (hypothesis, shrinking to a minimal
counterexample on failure), each against a definition written out here in
plain Python:

- top-k ("DeepSeek open-sources TileKernels", section 2.1): the K rounds of
  "maximum, lowest index among equal maxima, mask to -inf" equal the stable
  sort of (-score, index) over the entries above -inf, with NaN read as -inf,
  and, for the rounds after those entries run out, index 0 (every entry is
  then -inf, so the lowest index holding the maximum is 0);
- token map (section 2; "CuTeDSL at Perplexity", local kernel): counts,
  exclusive offsets and the rank of each (t, k) copy among the copies of its
  expert in row-major order, with ids outside [0, E) uncounted and at -1;
- e4m3 encoder (OCP E4M3FN, named in section 3.1): the nearest finite e4m3
  value, ties to the even code, finite values past 448 saturated, sign kept.
"""
import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st
from hypothesis.extra.numpy import arrays

import oracle

SPECIAL = [0.0, -0.0, 1.0, -1.0, 0.5, 2.0, float("inf"), float("-inf"), float("nan"), 1e-30, -3.25]


@st.composite
def score_rows(draw):
    T = draw(st.integers(1, 6))
    E = draw(st.integers(1, 24))
    K = draw(st.integers(1, min(E, 16)))
    elems = st.one_of(st.sampled_from(SPECIAL), st.floats(-4, 4, width=32))
    s = draw(arrays(np.float32, (T, E), elements=elems))
    return s, K


def _topk_definition(row, K):
    key = [(-float("inf") if v != v else float(v)) for v in row]
    live = sorted((i for i in range(len(row)) if key[i] != float("-inf")), key=lambda i: (-key[i], i))
    picks = live[:K]
    return picks + [0] * (K - len(picks))


@settings(max_examples=400, deadline=None, derandomize=True)
@given(score_rows())
def test_topk_equals_stable_sort_definition(case):
    s, K = case
    idx, _ = oracle.topk_gate(s, K)
    for t in range(s.shape[0]):
        assert list(idx[t]) == _topk_definition(s[t], K)


@st.composite
def id_rows(draw):
    T = draw(st.integers(0, 20))
    K = draw(st.integers(1, 5))
    E = draw(st.integers(1, 12))
    ids = draw(arrays(np.int64, (T, K), elements=st.integers(-3, E + 3)))
    return ids, E


@settings(max_examples=400, deadline=None, derandomize=True)
@given(id_rows())
def test_token_map_equals_rank_definition(case):
    ids, E = case
    T, K = ids.shape
    counts, offsets, pos, row_token = oracle.token_map(ids, E)
    want_counts = [sum(1 for t in range(T) for k in range(K) if ids[t, k] == e) for e in range(E)]
    assert list(counts) == want_counts
    assert list(offsets) == [sum(want_counts[:e]) for e in range(E + 1)]
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            if not 0 <= e < E:
                assert pos[t, k] == -1
                continue
            before = sum(1 for tt in range(T) for kk in range(K)
                         if ids[tt, kk] == e and (tt, kk) < (t, k))
            assert pos[t, k] == offsets[e] + before
            assert row_token[pos[t, k]] == t
    assert all(r == -1 for r in row_token[offsets[E]:])


def _e4m3_grid():
    """Magnitudes of the 127 non-negative finite codes, from the bit fields:
    subnormals m * 2^-9, normals (1 + m/8) * 2^(e - 7); code 0x7F is NaN."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return vals


GRID = _e4m3_grid()


def _e4m3_definition(x):
    sign = 0x80 if np.signbit(x) else 0
    a = min(abs(float(x)), 448.0)
    best = min(range(len(GRID)), key=lambda c: (abs(GRID[c] - a), c & 1))  # nearest, ties to even code
    return sign | best


@settings(max_examples=1000, deadline=None, derandomize=True)
@given(st.one_of(st.floats(-600, 600, width=32), st.sampled_from([0.0, -0.0, 448.0, -464.0, 464.0, 2.0 ** -10])))
def test_e4m3_encode_equals_nearest_even_definition(x):
    got = int(oracle.e4m3_encode(np.array([x], np.float32))[0])
    assert got == _e4m3_definition(np.float32(x)), (x, hex(got))
