"""moe_token_map_noalloc (the token map for callers that cannot allocate:
its count table is the library's fixed device array) through the C ABI,
against moe_token_map with a caller workspace, bit for bit: two calls in a
row with the second smaller, the two-launch path at its largest table
(256 chunks x 1024 experts = the whole 1 MiB array), the one-workgroup path,
and T = 0.  Every output is prefilled with garbage so that an unwritten
element fails."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _log(msg):
    sys.__stderr__.write(f"[gpu-no-alloc] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _garbage_outputs(T, K, E, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)

    def junk(n):
        return torch.randint(-(1 << 30), 1 << 30, (n,), generator=g, dtype=torch.int32, device="cuda")
    return junk(E), junk(E + 1), junk(T * K).view(T, K) if T * K else junk(0).view(T, K), junk(T * K)


def _ids(T, E, K, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = moe.moe_topk_gate(torch.from_numpy(s).cuda(), K)
    return idx


def _both(idx, E, seed):
    T, K = idx.shape
    ref = moe.moe_token_map(idx, E, out=_garbage_outputs(T, K, E, seed))
    got = moe.moe_token_map_noalloc(idx, E, out=_garbage_outputs(T, K, E, seed + 1))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


def _assert_equal(ref, got):
    for name, a, b in zip(("counts", "offsets", "pos", "row_token"), ref, got):
        assert np.array_equal(a, b), name


def test_two_calls_in_a_row_second_smaller():
    """The DeepSeek-V3 routing (32768 copies, 16 chunks of the two-launch map), then 1000 tokens over 200
    experts (8 chunks): the second call's table is smaller than what the first left in the array."""
    w = W.WORKLOADS["dsv3"]
    _log("dsv3 routing, then a smaller one")
    idx = moe.moe_topk_gate(torch.from_numpy(W.make_scores(w)).cuda(), w.num_topk, renormalize=True)[0]
    ref, got = _both(idx, w.num_experts, 1)
    _assert_equal(ref, got)
    o = oracle.token_map(idx.cpu().numpy(), w.num_experts)
    _assert_equal(o, got)
    idx2 = _ids(1000, 200, 8, 2)
    ref, got = _both(idx2, 200, 3)
    _assert_equal(ref, got)
    _assert_equal(oracle.token_map(idx2.cpu().numpy(), 200), got)


def test_largest_table():
    """32768 tokens x K = 16 over 1024 experts: 256 chunks of 2048 copies, a 1 MiB count table."""
    T, E, K = 32768, 1024, 16
    assert moe.moe_token_map_workspace_bytes(T, K, E) == 1 << 20
    _log(f"largest table T={T} E={E} K={K}")
    idx = _ids(T, E, K, 4)
    ref, got = _both(idx, E, 5)
    _assert_equal(ref, got)


@pytest.mark.parametrize("T,E,K", [(64, 16, 2), (200, 256, 8), (0, 64, 4)])
def test_small_and_empty(T, E, K):
    """One-workgroup map (no count table) and T = 0 (counts and offsets zeroed)."""
    _log(f"small T={T} E={E} K={K}")
    idx = _ids(T, E, K, 6) if T else torch.empty((0, K), dtype=torch.int64, device="cuda")
    ref, got = _both(idx, E, 7)
    _assert_equal(ref, got)


def test_stream_ordered_repeats_on_a_side_stream():
    """Calls in one stream's order share the array without racing: five maps of different sizes issued
    back to back on a side stream, each checked against the workspace version."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    shapes = [(4096, 256, 8), (300, 64, 4), (20000, 512, 8), (2500, 256, 8), (50, 1024, 16)]
    idxs = [_ids(T, E, K, 10 + i) for i, (T, E, K) in enumerate(shapes)]
    torch.cuda.synchronize()
    _log("five maps back to back on a side stream")
    outs = []
    for idx, (T, E, K) in zip(idxs, shapes):
        outs.append(moe.moe_token_map_noalloc(idx, E, stream=side))
    side.synchronize()
    for idx, (T, E, K), got in zip(idxs, shapes, outs):
        ref = moe.moe_token_map(idx, E)
        torch.cuda.synchronize()
        _assert_equal([t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got])
