"""GPU parity of moe_dispatch (top-k -> map -> expand + cast in one call)
against the oracle's top-k, map and expand composed, bit for bit, in both
forms: the single launch (every workgroup routing every token itself up to 32
tokens, a grid barrier above), the top-k kernel followed by the single launch's
map and copies (no barrier), and the split launches.
Decode-sized DeepSeek-V3-shaped batches (the first T tokens of that layer,
T from 1 to 256), the first 2048 tokens of the layer through the single
launch (T*K at its 16384 limit), every top-k register width (E from 16 to 1024),
K from 1 to 16, H from 128 to 7168, tie-heavy and NaN scores, fewer finite
scores than K, one workspace reused across calls of different grid sizes
(the barrier counters must hold whole epochs, the time-out word stay zero),
a non-default stream, T = 0, and renormalised weights at every K up to 16."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

SINGLE, SPLIT, AUTO = moe.MOE_DISPATCH_SINGLE_LAUNCH, moe.MOE_DISPATCH_SPLIT, moe.MOE_DISPATCH_AUTO
TOPK_COPY = moe.MOE_DISPATCH_TOPK_THEN_COPY


def _log(msg):
    sys.__stderr__.write(f"[gpu-dispatch] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


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


def expected(scores, x, K, renormalize, with_weights):
    E = scores.shape[1]
    idx, wt = oracle.topk_gate(scores, K, renormalize=renormalize, with_weights=with_weights)
    counts, offsets, pos, rt = oracle.token_map(idx, E)
    q, sf, ow = oracle.expand_cast_fp8(x, pos, wt)
    return {"topk_idx": idx, "topk_weights": wt, "counts": counts, "offsets": offsets, "pos": pos,
            "row_token": rt, "out": q, "out_sf": sf, "out_weights": ow}


def check(scores, x, K, mode, renormalize=False, with_weights=None, workspace=None, stream=None):
    T, E = scores.shape
    want_w = renormalize if with_weights is None else with_weights
    _log(f"dispatch T={T} E={E} K={K} H={x.shape[1]} mode={mode} renorm={renormalize} weights={want_w}")
    g = moe.moe_dispatch(torch.from_numpy(np.ascontiguousarray(scores)).cuda(), d_bf16(x), K,
                         renormalize=renormalize, with_weights=with_weights, mode=mode, workspace=workspace,
                         stream=stream)
    torch.cuda.synchronize()
    e = expected(scores, x, K, renormalize, want_w)
    for name, ref in e.items():
        if ref is None:
            assert g[name] is None, name
            continue
        assert bits_equal(h(g[name]), ref), name


def dsv3_prefix(T):
    w = W.WORKLOADS["dsv3"]
    return W.make_scores(w, T), W.make_x(w, T)


# up to 4 tokens the single launch routes locally in four-wave workgroups, 5 to 32 in sixteen-wave ones (two
# tokens per wave above 16; no grid barrier), from 33 through the grid barrier
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 16, 17, 31, 32, 33, 36, 64, 256])
@pytest.mark.parametrize("mode", [SINGLE, SPLIT, TOPK_COPY])
def test_dispatch_dsv3_decode(T, mode):
    s, x = dsv3_prefix(T)
    check(s, x, 8, mode, renormalize=True)


@pytest.mark.parametrize("mode", [AUTO, SPLIT, moe.MOE_DISPATCH_ROUTE_FUSED])
def test_dispatch_dsv3_full_layer(mode):
    """The whole DeepSeek-V3 layer (4096 tokens, 32768 routed rows, hidden 7168) in the forms that take it."""
    s, x = dsv3_prefix(4096)
    check(s, x, 8, mode, renormalize=True)


@pytest.mark.parametrize("mode", [SINGLE, TOPK_COPY])
def test_dispatch_dsv3_largest_single_launch(mode):
    s, x = dsv3_prefix(2048)
    check(s, x, 8, mode, renormalize=True)


@pytest.mark.parametrize("E,K,H", [(16, 2, 256), (100, 6, 128), (64, 1, 1024), (512, 16, 2048),
                                   (1024, 8, 4096), (1000, 16, 7168)])
@pytest.mark.parametrize("T", [3, 16, 30, 45])
def test_dispatch_shapes(E, K, H, T):
    rng = np.random.default_rng(E * 31 + K + T)
    s = rng.standard_normal((T, E)).astype(np.float32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    for mode in (SINGLE, SPLIT, AUTO, TOPK_COPY):
        check(s, x, K, mode, with_weights=True)
    check(s, x, K, SINGLE)  # no weights
    check(s, x, K, TOPK_COPY)


@pytest.mark.parametrize("T", [4, 16, 24, 40])
def test_dispatch_ties_nan_and_short_rows(T):
    rng = np.random.default_rng(77)
    E, K, H = 64, 8, 512
    s = rng.choice(np.array([-1.0, 0.0, -0.0, 0.5, 1.0], np.float32), (T, E))
    s[0, :] = np.nan
    s[1, 3:] = -np.inf  # fewer finite scores than K: index 0 repeats
    s[2, ::2] = np.nan
    x = W.f32_to_bf16_bits((rng.standard_normal((T, H)) * 10).astype(np.float32))
    check(s, x, K, SINGLE, with_weights=True)
    check(s, x, K, SPLIT, with_weights=True)
    check(s, x, K, TOPK_COPY, with_weights=True)


def test_dispatch_workspace_reuse_and_stream():
    E, K, H = 256, 8, 7168
    ws = torch.zeros(moe.moe_dispatch_workspace_bytes(300, K, E), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    for T in (64, 5, 200, 1, 64):
        s, x = dsv3_prefix(T)
        check(s, x, K, SINGLE, renormalize=True, workspace=ws)
        with torch.cuda.stream(side):
            check(s, x, K, SINGLE, renormalize=True, workspace=ws, stream=side)
        torch.cuda.synchronize()
        words = h(ws[:2048].view(torch.int32)).view(np.uint32)
        assert words[2] == 0, words[:3]  # no barrier wait timed out
        assert not (words % (1 << 16)).any(), np.nonzero(words % (1 << 16))  # whole epochs only


@pytest.mark.parametrize("mode", [AUTO, SINGLE, SPLIT, TOPK_COPY, moe.MOE_DISPATCH_ROUTE_FUSED])
def test_dispatch_zero_tokens(mode):
    """No tokens: every mode returns MOE_OK and zeroes counts and offsets (prefilled with garbage here)."""
    E = 32
    _log(f"dispatch T=0 mode={mode}")
    s = torch.empty((0, E), dtype=torch.float32, device="cuda")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    g = moe.moe_dispatch(s, x, 4, mode=mode)
    g["counts"].fill_(-5)
    g["offsets"].fill_(-5)
    g = moe.moe_dispatch(s, x, 4, mode=mode, out=g)
    torch.cuda.synchronize()
    assert h(g["counts"]).tolist() == [0] * E and h(g["offsets"]).tolist() == [0] * (E + 1)


@pytest.mark.parametrize("E,K", [(32, 1), (16, 16), (64, 9), (256, 15), (256, 16), (512, 16), (1000, 13),
                                 (1024, 16)])
@pytest.mark.parametrize("T", [20, 40])
def test_renormalised_weights_every_width(E, K, T):
    """Renormalised weights at every K up to 16 (the weight sum runs in round order over the first K lanes),
    through the top-k kernel, the fused and local routing and every moe_dispatch form. Positive scores, a third of
    the rows tie-heavy (four values)."""
    rng = np.random.default_rng(E * 17 + K + T)
    s = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, E))))).astype(np.float32)
    s[::3] = np.ceil(s[::3] * 4) / 4
    x = W.f32_to_bf16_bits(rng.standard_normal((T, 256)).astype(np.float32))
    ei, ew = oracle.topk_gate(s, K, renormalize=True, with_weights=True)
    _log(f"renormalised top-k T={T} E={E} K={K}")
    idx, wt = moe.moe_topk_gate(torch.from_numpy(s).cuda(), K, renormalize=True)
    torch.cuda.synchronize()
    assert bits_equal(h(idx), ei) and bits_equal(h(wt), ew)
    route_modes = [moe.MOE_ROUTE_FUSED, moe.MOE_ROUTE_SPLIT] + ([moe.MOE_ROUTE_LOCAL] if T <= 32 else [])
    for rmode in route_modes:
        _log(f"renormalised route T={T} E={E} K={K} mode={rmode}")
        r = moe.moe_route(torch.from_numpy(s).cuda(), K, renormalize=True, mode=rmode)
        torch.cuda.synchronize()
        assert bits_equal(h(r["topk_idx"]), ei) and bits_equal(h(r["topk_weights"]), ew), rmode
    for mode in (SINGLE, TOPK_COPY, SPLIT, AUTO):
        check(s, x, K, mode, renormalize=True)
