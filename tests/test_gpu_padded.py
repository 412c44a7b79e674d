"""GPU parity of the padded, expert-local map and expand against the oracle,
bit for bit: counts, padded offsets, positions (-1 outside the local range),
row->token map with -1 padding and tail, and the padded expand (routed rows
cast as in the plain expand, every other row zero-filled by the same
launch).  DeepSeek-V3-shaped layer (4096 tokens, 256 experts, K = 8) and the
large skewed workload at full size, over several local ranges and
alignments; both expand kernels (K >= 4 and K < 4), more than 512 local
experts, ids outside the range, an all-to-one-expert batch, a row count
above the bound, and empty batches.  Outputs are prefilled with garbage so
that an unwritten row shows."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

_CACHE = {}


def _log(msg):
    sys.__stderr__.write(f"[gpu-padded] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def d_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def d_i64(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int64)).cuda()


def d_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def h(t):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t.cpu().numpy()


def bits_equal(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), np.asarray(b, np.float32).view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


def routed(name):
    if name not in _CACHE:
        w = W.WORKLOADS[name]
        idx, wt = oracle.topk_gate(W.make_scores(w), w.num_topk, renormalize=w.renormalize,
                                   with_weights=True)
        _CACHE[name] = (w, idx, wt, W.make_x(w))
    return _CACHE[name]


def _map(idx, begin, end, align, num_rows=None):
    T, K = idx.shape
    if num_rows is None:
        num_rows = oracle.padded_rows_bound(T, K, end - begin, align)
    _log(f"aligned map T={T} K={K} range=[{begin},{end}) align={align} rows={num_rows}")
    rt = torch.full((num_rows,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    g = moe.moe_token_map_aligned(d_i64(idx), begin, end, align, num_rows=num_rows,
                                  out=(torch.empty(end - begin, dtype=torch.int32, device="cuda"),
                                       torch.empty(end - begin + 1, dtype=torch.int32, device="cuda"),
                                       torch.empty((T, K), dtype=torch.int32, device="cuda"), rt))
    torch.cuda.synchronize()
    o = oracle.token_map_aligned(idx, begin, end, align, num_rows=num_rows)
    for name, a, b in zip(("counts", "offsets", "pos", "row_token"), g, o):
        assert bits_equal(h(a), b), name
    return o


def _expand(x, pos, row_token, wt):
    R, H = row_token.size, x.shape[1]
    _log(f"padded expand T={x.shape[0]} H={H} K={pos.shape[1]} R={R} weights={wt is not None}")
    q = torch.full((R, H), 0xA5, dtype=torch.uint8, device="cuda")
    sf = torch.full((R, H // 128), 7.0, dtype=torch.float32, device="cuda")
    ow = torch.full((R,), 7.0, dtype=torch.float32, device="cuda") if wt is not None else None
    moe.moe_expand_cast_fp8_padded(d_bf16(x), d_i32(pos), d_i32(row_token),
                                   d_f32(wt) if wt is not None else None, out=(q, sf, ow))
    torch.cuda.synchronize()
    gq, gsf = h(q), h(sf)
    gow = h(ow) if ow is not None else None
    del q, sf, ow
    eq, esf, eow = oracle.expand_cast_fp8_padded(x, pos, row_token, wt)
    assert bits_equal(gsf, esf)
    assert bits_equal(gq, eq)
    if wt is not None:
        assert bits_equal(gow, eow)


@pytest.mark.parametrize("begin,end,align", [(0, 256, 1), (0, 256, 128), (64, 128, 128),
                                             (255, 256, 16), (0, 256, 4096), (37, 200, 3)])
def test_aligned_map_dsv3(begin, end, align):
    _, idx, _, _ = routed("dsv3")
    _map(idx, begin, end, align)


@pytest.mark.parametrize("begin,end,align", [(0, 256, 128), (96, 160, 64)])
def test_aligned_map_large(begin, end, align):
    _, idx, _, _ = routed("large")
    _map(idx, begin, end, align)


def test_aligned_map_many_local_experts_and_bad_ids():
    rng = np.random.default_rng(41)
    T, K, E = 3000, 16, 1024
    idx, _ = oracle.topk_gate(rng.standard_normal((T, E)).astype(np.float32), K)
    idx[::5, 0] = -7
    idx[1, 1] = np.iinfo(np.int64).max
    idx[2, 2] = np.iinfo(np.int64).min
    _map(idx, 100, 800, 32)  # 700 local experts: the 512-thread rank kernel
    _map(idx, 0, 1024, 1)


def test_aligned_map_single_workgroup():
    """At most one chunk (2048 copies): the single-workgroup map, with more than
    512 local experts too."""
    rng = np.random.default_rng(43)
    idx, _ = oracle.topk_gate(rng.standard_normal((100, 1024)).astype(np.float32), 16)
    idx[::9, 3] = -1
    _map(idx, 100, 800, 32)
    _map(idx, 0, 1024, 1)
    _map(idx[:5], 0, 1024, 128)


def test_aligned_map_hot_expert_and_extra_rows():
    rng = np.random.default_rng(42)
    T, K, E = 5000, 4, 64
    idx = np.full((T, K), 9, np.int64)
    idx[:, 1] = rng.integers(0, E, T)
    bound = oracle.padded_rows_bound(T, K, 16, 256)
    _map(idx, 0, 16, 256, num_rows=bound + 1000)  # tail rows past the bound are -1 too


def test_aligned_map_zero_tokens():
    EL, R = 32, 100
    _log("aligned map T=0")
    counts = torch.full((EL,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((EL + 1,), 7, dtype=torch.int32, device="cuda")
    rt = torch.full((R,), 7, dtype=torch.int32, device="cuda")
    moe.moe_token_map_aligned(torch.empty((0, 4), dtype=torch.int64, device="cuda"), 10, 10 + EL, 4,
                              num_rows=R, out=(counts, offsets,
                                               torch.empty((0, 4), dtype=torch.int32, device="cuda"), rt))
    torch.cuda.synchronize()
    assert h(counts).tolist() == [0] * EL and h(offsets).tolist() == [0] * (EL + 1)
    assert h(rt).tolist() == [-1] * R


@pytest.mark.parametrize("begin,end,align", [(0, 256, 128), (64, 128, 128), (200, 256, 1)])
def test_padded_expand_dsv3(begin, end, align):
    _, idx, wt, x = routed("dsv3")
    _, _, pos, rt = oracle.token_map_aligned(idx, begin, end, align)
    _expand(x, pos, rt, wt)


def test_padded_expand_large_local_range():
    _, idx, wt, x = routed("large")
    _, _, pos, rt = oracle.token_map_aligned(idx, 96, 160, 128)
    _expand(x, pos, rt, wt)


@pytest.mark.parametrize("K,H", [(1, 7168), (2, 1024), (3, 128), (4, 4096), (6, 2048)])
def test_padded_expand_topk_and_hidden(K, H):
    rng = np.random.default_rng(K * 1000 + H)
    T, E = 777, 32
    idx, wt = oracle.topk_gate(rng.standard_normal((T, E)).astype(np.float32), K, with_weights=True)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    _, _, pos, rt = oracle.token_map_aligned(idx, 8, 24, 16)
    _expand(x, pos, rt, wt)
    _expand(x, pos, rt, None)


def test_padded_expand_zero_tokens_fills_all_rows():
    R, H = 300, 1024
    _log("padded expand T=0")
    q = torch.full((R, H), 0xA5, dtype=torch.uint8, device="cuda")
    sf = torch.full((R, H // 128), 7.0, dtype=torch.float32, device="cuda")
    ow = torch.full((R,), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_expand_cast_fp8_padded(torch.empty((0, H), dtype=torch.bfloat16, device="cuda"),
                                   torch.empty((0, 8), dtype=torch.int32, device="cuda"),
                                   torch.full((R,), -1, dtype=torch.int32, device="cuda"),
                                   torch.empty((0, 8), dtype=torch.float32, device="cuda"), out=(q, sf, ow))
    torch.cuda.synchronize()
    assert not h(q).any() and not h(sf).any() and not h(ow).any()


def test_aligned_pipeline_matches_plain_on_routed_rows():
    """Map and padded expand on the GPU end to end; each routed row equals the
    plain expand's row of the same copy."""
    _, idx, wt, x = routed("dsv3")
    _log("aligned pipeline dsv3 [0,256) align 128")
    xd, idx_d, wt_d = d_bf16(x), d_i64(idx), d_f32(wt)
    _, _, pos_a, rt_a = moe.moe_token_map_aligned(idx_d, 0, 256, 128)
    qa, sfa, owa = moe.moe_expand_cast_fp8_padded(xd, pos_a, rt_a, wt_d)
    _, _, pos_p, _ = moe.moe_token_map(idx_d, 256)
    qp, sfp, owp = moe.moe_expand_cast_fp8(xd, pos_p, wt_d)
    torch.cuda.synchronize()
    pa, pp = h(pos_a).ravel(), h(pos_p).ravel()
    assert bits_equal(h(qa)[pa], h(qp)[pp])
    assert bits_equal(h(sfa)[pa], h(sfp)[pp])
    assert bits_equal(h(owa)[pa], h(owp)[pp])
