"""Pins for the oracle's aligned, expert-local token map and padded expand
(TileKernels article section 2.2: positions < 0 are skipped and the expand
zero-fills invalid rows in the same grid; "CuTeDSL at Perplexity", local
kernel: optional padded buffers for the grouped GEMM, and the
tensor-parallel dispatch that routes only the rank's experts).

align = 1 over all experts is the plain map; segment starts are multiples
of align and each segment holds its count plus less than align padding
rows; a local range equals the full map restricted to its experts
(brute-force triple sort on a sub-range); the padded expand equals the
plain expand on routed rows and zeros elsewhere.
"""
import numpy as np
import pytest

import oracle


def _routing(T, E, K, seed):
    rng = np.random.default_rng(seed)
    idx, wt = oracle.topk_gate(rng.standard_normal((T, E)).astype(np.float32), K, with_weights=True)
    return idx, wt


def test_align_one_full_range_is_plain_map():
    idx, _ = _routing(300, 32, 4, 0)
    c0, o0, p0, r0 = oracle.token_map(idx, 32)
    c1, o1, p1, r1 = oracle.token_map_aligned(idx, 0, 32, 1)
    assert np.array_equal(c0, c1) and np.array_equal(o0, o1)
    assert np.array_equal(p0, p1) and np.array_equal(r0, r1)


@pytest.mark.parametrize("align", [2, 16, 128])
def test_segments_are_aligned_and_padded(align):
    idx, _ = _routing(517, 64, 6, align)
    counts, offsets, pos, row_token = oracle.token_map_aligned(idx, 0, 64, align)
    c0, _, _, _ = oracle.token_map(idx, 64)
    assert np.array_equal(counts, c0)
    assert np.all(offsets % align == 0)
    size = np.diff(offsets)
    assert np.all(size >= counts) and np.all(size - counts < align)
    assert np.all((size == 0) == (counts == 0))
    for e in range(64):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(seg[:counts[e]] >= 0) and np.all(np.diff(seg[:counts[e]]) >= 0)
        assert np.all(seg[counts[e]:] == -1)
        assert all(e in idx[t] for t in seg[:counts[e]])
    assert np.all(row_token[offsets[-1]:] == -1)
    valid = pos.ravel()
    assert np.array_equal(np.sort(valid), np.sort(np.nonzero(row_token >= 0)[0]))


@pytest.mark.parametrize("begin,end,align", [(0, 16, 1), (16, 48, 1), (40, 64, 8), (63, 64, 4)])
def test_local_range_is_restricted_map(begin, end, align):
    idx, _ = _routing(400, 64, 8, begin + end)
    counts, offsets, pos, row_token = oracle.token_map_aligned(idx, begin, end, align)
    local = (idx >= begin) & (idx < end)
    assert np.all((pos >= 0) == local)
    # brute force: sort the local (expert, t, k) triples; rank within expert
    T, K = idx.shape
    triples = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K) if local[t, k])
    seen = {}
    for e, t, k in triples:
        j = e - begin
        r = seen.get(j, 0)
        assert pos[t, k] == offsets[j] + r
        seen[j] = r + 1
    assert sum(seen.values()) == counts.sum() == local.sum()


def test_padded_expand_zero_fills():
    rng = np.random.default_rng(5)
    T, E, K, H = 90, 16, 4, 256
    idx, wt = _routing(T, E, K, 5)
    x = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    counts, offsets, pos, row_token = oracle.token_map_aligned(idx, 4, 12, 32)
    q, sf, ow = oracle.expand_cast_fp8_padded(x, pos, row_token, wt)
    q_id, sf_id, _ = oracle.expand_cast_fp8(x)
    routed = row_token >= 0
    assert np.array_equal(q[routed], q_id[row_token[routed]])
    assert np.array_equal(sf[routed], sf_id[row_token[routed]])
    assert np.all(q[~routed] == 0) and np.all(sf[~routed] == 0) and np.all(ow[~routed] == 0)
    for t in range(T):
        for k in range(K):
            if pos[t, k] >= 0:
                assert ow[pos[t, k]] == wt[t, k]


def test_rows_bound_is_enough():
    idx, _ = _routing(1000, 8, 8, 9)
    for align in (1, 3, 64, 256):
        counts, offsets, _, _ = oracle.token_map_aligned(idx, 0, 8, align)
        assert offsets[-1] <= oracle.padded_rows_bound(1000, 8, 8, align)
