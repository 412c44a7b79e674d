"""GPU parity of the combine (weighted reduce to token order) against the
oracle, bit for bit: every bf16 output equals the oracle's k-ordered fp32
sum rounded to nearest even.  Full DeepSeek-V3-shaped layer (4096 tokens,
K = 8, H = 7168) with renormalised weights; the large skewed workload on a
token sample at its full size; K in {1, 2, 3, 4, 6, 8, 16} (templated and
generic paths), H = 8, skipped rows, no weights and the k-order
cancellation case."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _log(msg):
    sys.__stderr__.write(f"[gpu-combine] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def h_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(y, pos, w=None):
    out = moe.moe_combine(d_bf16(y), torch.from_numpy(np.ascontiguousarray(pos, np.int32)).cuda(),
                          None if w is None else torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda())
    torch.cuda.synchronize()
    return h_bits(out)


def test_combine_dsv3_full():
    w = W.WORKLOADS["dsv3"]
    T, E, K, H = w.num_tokens, w.num_experts, w.num_topk, w.hidden
    idx, wt = oracle.topk_gate(W.make_scores(w), K, renormalize=True)
    _, _, pos, _ = oracle.token_map(idx, E)
    rng = np.random.default_rng(31)
    y = W.f32_to_bf16_bits(rng.standard_normal((T * K, H), dtype=np.float32))
    _log(f"combine dsv3 T={T} K={K} H={H}")
    assert np.array_equal(_run(y, pos, wt), oracle.combine(y, pos, wt))


def test_combine_large_sampled():
    w = W.WORKLOADS["large"]
    T, E, K, H = w.num_tokens, w.num_experts, w.num_topk, w.hidden
    idx, _ = oracle.topk_gate(W.make_scores(w), K)
    _, _, pos, _ = oracle.token_map(idx, E)
    R = T * K
    gen = torch.Generator(device="cuda").manual_seed(5)
    y_d = torch.randn((R, H), device="cuda", generator=gen).to(torch.bfloat16)
    wt = np.random.default_rng(32).random((T, K), dtype=np.float32)
    pos_d = torch.from_numpy(pos).cuda()
    _log(f"combine large T={T} K={K} H={H} R={R}")
    out = h_bits(moe.moe_combine(y_d, pos_d, torch.from_numpy(wt).cuda()))
    sample = np.random.default_rng(33).choice(T, 2048, replace=False)
    rows = pos[sample].reshape(-1)
    y_s = h_bits(y_d[torch.from_numpy(rows.astype(np.int64)).cuda()])
    pos_s = np.arange(rows.size, dtype=np.int32).reshape(-1, K)
    assert np.array_equal(out[sample], oracle.combine(y_s, pos_s, wt[sample]))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 6, 8, 16])
def test_combine_topk_sizes(K):
    rng = np.random.default_rng(K)
    T, H = 333, 1024
    R = T * K + 17
    y = W.f32_to_bf16_bits((rng.standard_normal((R, H)) * 3).astype(np.float32))
    pos = rng.permutation(R)[:T * K].astype(np.int32).reshape(T, K)
    pos[rng.random((T, K)) < 0.1] = -1
    pos[0, 0] = R + 3  # out of range: skipped
    wt = rng.standard_normal((T, K)).astype(np.float32)
    _log(f"combine K={K} T={T} H={H}")
    assert np.array_equal(_run(y, pos, wt), oracle.combine(y, pos, wt))
    assert np.array_equal(_run(y, pos), oracle.combine(y, pos))


def test_combine_small_hidden_and_order():
    y = W.f32_to_bf16_bits(np.array([[2.0 ** 25] * 8, [1.0] * 8, [-(2.0 ** 25)] * 8], np.float32))
    for p in ([[0, 1, 2]], [[0, 2, 1]], [[-1, -1, -1]]):
        pos = np.array(p, np.int32)
        _log(f"combine order case {p}")
        assert np.array_equal(_run(y, pos), oracle.combine(y, pos))


def test_combine_zero_tokens():
    out = moe.moe_combine(torch.empty((4, 64), dtype=torch.bfloat16, device="cuda"),
                          torch.empty((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


@pytest.mark.parametrize("H", [520, 1000, 7176])
def test_combine_rows_not_whole_waves(H):
    """Widths whose row is not a whole number of 64-lane waves (hidden % 512
    != 0): a wave spans two tokens, the per-lane kernel with K = 8 unrolled,
    skipped and out-of-range positions included."""
    rng = np.random.default_rng(H)
    T, K = 257, 8
    R = T * K
    y = W.f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    pos = rng.permutation(R).astype(np.int32).reshape(T, K)
    pos[rng.random((T, K)) < 0.1] = -1
    pos[3, 5] = R  # out of range: skipped
    wt = rng.standard_normal((T, K)).astype(np.float32)
    _log(f"combine H={H} T={T} K={K}")
    assert np.array_equal(_run(y, pos, wt), oracle.combine(y, pos, wt))


def test_combine_no_rows():
    """Tokens but no rows: every position is out of range and the sums are zero."""
    T, K, H = 50, 8, 1024
    y = np.zeros((0, H), np.uint16)
    pos = np.full((T, K), 3, np.int32)
    pos[::2] = -1
    _log("combine with an empty row set")
    got = _run(y, pos, np.ones((T, K), np.float32))
    assert np.array_equal(got, oracle.combine(y, pos, np.ones((T, K), np.float32)))
    assert not got.any()
