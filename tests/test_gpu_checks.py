"""The device-side input checks (moe_check_scores, moe_check_topk_idx,
moe_check_pos) through the C ABI: clean workload inputs give no flags,
planted violations give exactly the expected bits (computed on the host from
the definitions: finite / positive scores, ids in [0, E) and distinct per
row, positions in [-1, R) and distinct), flags accumulate, the pos bitmap is
cleared per call, and MOE_FP8_DEBUG makes the calls raise before any output
is written."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import workloads as W

pytestmark = pytest.mark.gpu

NONFINITE, NONPOS, ID_RANGE, ID_DUP, POS_RANGE, POS_DUP = 0x01, 0x02, 0x04, 0x08, 0x10, 0x20


def _log(msg):
    sys.__stderr__.write(f"[gpu-checks] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _bits(flags):
    torch.cuda.synchronize()
    return int(flags.item()) & 0xFFFFFFFF


def _want_scores(s, require_positive):
    fin = np.isfinite(s)
    return (NONFINITE if (~fin).any() else 0) | (NONPOS if require_positive and (s[fin] <= 0).any() else 0)


def _want_idx(idx, E):
    bits = ID_RANGE if ((idx < 0) | (idx >= E)).any() else 0
    srt = np.sort(idx, axis=1)
    if (srt[:, 1:] == srt[:, :-1]).any():
        bits |= ID_DUP
    return bits


def _want_pos(pos, R):
    p = pos.ravel()
    bits = POS_RANGE if ((p < -1) | (p >= R)).any() else 0
    v = p[(p >= 0) & (p < R)]
    if len(np.unique(v)) != len(v):
        bits |= POS_DUP
    return bits


@pytest.mark.parametrize("name", ["tiny", "mid", "dsv3"])
def test_clean_workloads_pass(name):
    w = W.WORKLOADS[name]
    _log(f"clean {name}")
    s = torch.from_numpy(W.make_scores(w)).cuda()
    idx, _ = moe.moe_topk_gate(s, w.num_topk, renormalize=w.renormalize, with_weights=True)
    _, _, pos, _ = moe.moe_token_map(idx, w.num_experts)
    f = moe.moe_check_scores(s, require_positive=w.renormalize)
    moe.moe_check_topk_idx(idx, w.num_experts, flags=f)
    moe.moe_check_pos(pos, w.num_tokens * w.num_topk, flags=f)
    assert _bits(f) == 0


def test_large_scores_flagged_only_when_positivity_required():
    w = W.WORKLOADS["large"]
    _log("large scores (N(0,1) + log-Zipf bias: negative values)")
    s = torch.from_numpy(W.make_scores(w, num_tokens=4096)).cuda()
    assert _bits(moe.moe_check_scores(s)) == 0
    assert _bits(moe.moe_check_scores(s, require_positive=True)) == NONPOS


@pytest.mark.parametrize("seed", range(12))
def test_planted_violations(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.choice([1, 37, 1000, 5000]))
    E = int(rng.choice([16, 256, 1024]))
    K = int(rng.choice([1, 2, 8, 16]))
    K = min(K, E)
    _log(f"planted seed={seed} T={T} E={E} K={K}")
    # scores: positive, then plant NaN / inf / zero / negative values
    s = rng.random((T, E), dtype=np.float32) + np.float32(0.01)
    for val in (np.nan, np.inf, -np.inf, 0.0, -0.0, -1.5):
        if rng.random() < 0.3:
            s[rng.integers(T), rng.integers(E)] = val
    # ids: distinct per row (a random permutation prefix), then plant range / duplicate faults
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int64)
    if rng.random() < 0.4:
        idx[rng.integers(T), rng.integers(K)] = int(rng.choice([-1, E, E + 7, -(1 << 40)]))
    if K > 1 and rng.random() < 0.4:
        t = rng.integers(T)
        idx[t, 1] = idx[t, 0]
    # positions: a permutation of [0, R) with some -1, then plant range / duplicate faults
    R = T * K
    pos = rng.permutation(R).astype(np.int32).reshape(T, K)
    pos[rng.random((T, K)) < 0.05] = -1
    if rng.random() < 0.4:
        pos[rng.integers(T), rng.integers(K)] = int(rng.choice([-2, R, R + 100, -(1 << 31)]))
    if R > 1 and rng.random() < 0.4:
        a, b = rng.choice(R, 2, replace=False)
        pos.flat[b] = pos.flat[a] if pos.flat[a] >= 0 else 0
        pos.flat[a] = pos.flat[b]
    for rp in (False, True):
        got = _bits(moe.moe_check_scores(torch.from_numpy(s).cuda(), require_positive=rp))
        assert got == _want_scores(s, rp), (rp, got)
    assert _bits(moe.moe_check_topk_idx(torch.from_numpy(idx).cuda(), E)) == _want_idx(idx, E)
    assert _bits(moe.moe_check_pos(torch.from_numpy(pos).cuda(), R)) == _want_pos(pos, R)


def test_flags_accumulate_and_bitmap_is_cleared_per_call():
    dev = torch.device("cuda")
    pos_dup = torch.tensor([[0, 1], [1, 2]], dtype=torch.int32, device=dev)
    pos_ok = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    assert _bits(moe.moe_check_pos(pos_dup, 4, workspace=ws)) == POS_DUP
    # same workspace, its bitmap still holds the first call's rows: the call clears it
    assert _bits(moe.moe_check_pos(pos_ok, 4, workspace=ws)) == 0
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.moe_check_scores(torch.tensor([[float("nan"), 1.0]], device=dev), flags=f)
    moe.moe_check_topk_idx(torch.tensor([[3, 3]], dtype=torch.int64, device=dev), 8, flags=f)
    moe.moe_check_pos(torch.tensor([[5, -1]], dtype=torch.int32, device=dev), 2, flags=f)
    assert _bits(f) == NONFINITE | ID_DUP | POS_RANGE
    # -1 entries only, and zero rows with every entry -1: nothing to flag
    assert _bits(moe.moe_check_pos(torch.full((3, 2), -1, dtype=torch.int32, device=dev), 0)) == 0


def test_checks_on_a_side_stream():
    dev = torch.device("cuda")
    side = torch.cuda.Stream()
    s = torch.rand((512, 256), device=dev)
    s[100, 7] = float("inf")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f = moe.moe_check_scores(s, stream=side)
    side.synchronize()
    assert int(f.item()) == NONFINITE


def test_debug_mode_raises_before_writing(monkeypatch):
    dev = torch.device("cuda")
    w = W.WORKLOADS["tiny"]
    s = torch.from_numpy(W.make_scores(w)).cuda()
    x = torch.from_numpy(W.make_x(w).view(np.int16)).cuda().view(torch.bfloat16)
    idx, wts = moe.moe_topk_gate(s, w.num_topk, with_weights=True)
    _, _, pos, _ = moe.moe_token_map(idx, w.num_experts)
    ref = moe.moe_expand_cast_fp8(x, pos, wts)
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_FP8_DEBUG", "1")
    assert moe.debug_enabled()
    # clean inputs: same results as without the checks
    idx2, wts2 = moe.moe_topk_gate(s, w.num_topk, with_weights=True)
    _, _, pos2, _ = moe.moe_token_map(idx2, w.num_experts)
    got = moe.moe_expand_cast_fp8(x, pos2, wts2)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(pos2, pos)
    assert torch.equal(got[0].view(torch.uint8), ref[0].view(torch.uint8)) and torch.equal(got[1], ref[1])
    # violations raise before the call writes its outputs
    R, H = pos.numel(), w.hidden
    q = torch.full((R, H), 7, dtype=torch.uint8, device=dev)
    sf = torch.full((R, H // 128), 7.0, device=dev)
    ow = torch.full((R,), 7.0, device=dev)
    bad = pos.clone()
    bad[0, 1] = bad[0, 0]
    with pytest.raises(ValueError, match="MOE_CHECK_POS_DUPLICATE"):
        moe.moe_expand_cast_fp8(x, bad, wts, out=(q, sf, ow))
    torch.cuda.synchronize()
    assert (q == 7).all() and (sf == 7.0).all() and (ow == 7.0).all()
    s_nan = s.clone()
    s_nan[3, 2] = float("nan")
    with pytest.raises(ValueError, match="MOE_CHECK_NONFINITE_SCORE"):
        moe.moe_topk_gate(s_nan, w.num_topk)
    with pytest.raises(ValueError, match="MOE_CHECK_NONFINITE_SCORE"):
        moe.moe_dispatch(s_nan, x, w.num_topk)
    with pytest.raises(ValueError, match="MOE_CHECK_NONPOSITIVE_SCORE"):
        moe.moe_topk_gate(s, w.num_topk, renormalize=True)  # N(0,1) scores: some are negative
    bad_idx = idx.clone()
    bad_idx[5, 0] = w.num_experts
    with pytest.raises(ValueError, match="MOE_CHECK_ID_RANGE"):
        moe.moe_token_map(bad_idx, w.num_experts)
    monkeypatch.setenv("MOE_FP8_DEBUG", "0")
    assert not moe.debug_enabled()
    moe.moe_token_map(bad_idx, w.num_experts)  # the map's own rule: pos = -1 for that copy
    torch.cuda.synchronize()


def test_debug_mode_refuses_graph_capture(monkeypatch):
    w = W.WORKLOADS["tiny"]
    s = torch.from_numpy(W.make_scores(w)).cuda()
    idx = torch.empty((w.num_tokens, w.num_topk), dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_FP8_DEBUG", "1")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="graph capture"):
        with torch.cuda.graph(g):
            moe.moe_topk_gate(s, w.num_topk, out=(idx, None))
    monkeypatch.setenv("MOE_FP8_DEBUG", "0")
    # the device is usable afterwards
    got, _ = moe.moe_topk_gate(s, w.num_topk)
    torch.cuda.synchronize()
    assert got.shape == (w.num_tokens, w.num_topk)


NONFINITE_ACT, DISPATCH_TIMEOUT = 0x40, 0x80


@pytest.mark.parametrize("pattern", [0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x7F81])
def test_activation_check_flags_nonfinite(pattern):
    """One NaN (quiet, negative, signalling) or infinity planted in an otherwise finite row set."""
    w = W.WORKLOADS["dsv3"]
    x = W.make_x(w, num_tokens=64)
    _log(f"activations with 0x{pattern:04X}")
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    assert _bits(moe.moe_check_activations(xd)) == 0
    bad = x.copy()
    bad[37, 5001] = pattern
    bd = torch.from_numpy(bad.view(np.int16)).cuda().view(torch.bfloat16)
    assert _bits(moe.moe_check_activations(bd)) == NONFINITE_ACT
    # a ragged count that ends just before the planted value sees nothing
    flat = bd.reshape(-1)
    n = 37 * x.shape[1] + 5001
    assert _bits(moe.moe_check_activations(flat[:n])) == 0
    assert _bits(moe.moe_check_activations(flat[:n + 1])) == NONFINITE_ACT


def test_debug_mode_rejects_nonfinite_activations(monkeypatch):
    monkeypatch.setenv("MOE_FP8_DEBUG", "1")
    rng = np.random.default_rng(3)
    x = W.f32_to_bf16_bits(rng.standard_normal((8, 256)).astype(np.float32))
    x[2, 7] = 0x7F80
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    with pytest.raises(ValueError, match="MOE_CHECK_NONFINITE_ACTIVATION"):
        moe.moe_expand_cast_fp8(xd)
    gu = W.f32_to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    gu[1, 3] = 0x7FC0
    with pytest.raises(ValueError, match="MOE_CHECK_NONFINITE_ACTIVATION"):
        moe.swiglu_cast_fp8(torch.from_numpy(gu.view(np.int16)).cuda().view(torch.bfloat16))


@pytest.mark.parametrize("mode", [moe.MOE_DISPATCH_SINGLE_LAUNCH, moe.MOE_DISPATCH_SPLIT])
def test_dispatch_check_clean_after_calls(mode):
    """A completed dispatch leaves the time-out word clear; the check reports nothing."""
    w = W.WORKLOADS["dsv3"]
    T = 8
    s = torch.from_numpy(W.make_scores(w, T)).cuda()
    x = torch.from_numpy(W.make_x(w, T).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.zeros(moe.moe_dispatch_workspace_bytes(T, w.num_topk, w.num_experts), dtype=torch.uint8,
                     device="cuda")
    _log(f"dispatch check, mode {mode}")
    for _ in range(3):
        moe.moe_dispatch(s, x, w.num_topk, renormalize=True, mode=mode, workspace=ws)
    assert _bits(moe.moe_check_dispatch(ws)) == 0


def test_dispatch_timeout_word_is_reported(monkeypatch):
    """The word a timed-out barrier wait sets (uint32 2 of the header), planted from the host: the check
    reports it, and in debug mode moe_dispatch raises after the call (split form: no barrier runs)."""
    w = W.WORKLOADS["dsv3"]
    T = 4
    s = torch.from_numpy(W.make_scores(w, T)).cuda()
    x = torch.from_numpy(W.make_x(w, T).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.zeros(moe.moe_dispatch_workspace_bytes(T, w.num_topk, w.num_experts), dtype=torch.uint8,
                     device="cuda")
    ws.view(torch.int32)[2] = 1
    _log("planted dispatch time-out word")
    assert _bits(moe.moe_check_dispatch(ws)) == DISPATCH_TIMEOUT
    monkeypatch.setenv("MOE_FP8_DEBUG", "1")
    with pytest.raises(RuntimeError, match="MOE_CHECK_DISPATCH_TIMEOUT"):
        moe.moe_dispatch(s, x, w.num_topk, renormalize=True, mode=moe.MOE_DISPATCH_SPLIT, workspace=ws)
    ws.view(torch.int32)[2] = 0
    moe.moe_dispatch(s, x, w.num_topk, renormalize=True, mode=moe.MOE_DISPATCH_SPLIT, workspace=ws)
    torch.cuda.synchronize()
