"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bit-exact: top-k ids and renormalised weights, counts, offsets, positions,
row->token map, expanded e4m3 codes, scales and weights.  SwiGLU + cast:
scales within 1e-6 relative and dequantised values within one e4m3 step
(oracle.compare).  Workloads at their full sizes (the launch configuration
the benchmark times), plus ragged, tie-heavy, out-of-range, empty and
maximum-size cases, guard bytes around outputs, a non-default stream and
run-to-run determinism.
"""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W
from oracle.compare import swiglu_tolerance_report

pytestmark = pytest.mark.gpu

_CACHE = {}


def _log(msg):
    sys.__stderr__.write(f"[gpu-parity] {msg}\n")
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


def inputs(name):
    if name not in _CACHE:
        w = W.WORKLOADS[name]
        d = {"w": w}
        if w.num_tokens:
            d["scores"] = W.make_scores(w)
            d["x"] = W.make_x(w)
        if w.swiglu_rows:
            d["gate_up"] = W.make_gate_up(w)
            d["row_weights"] = W.make_row_weights(w)
        _CACHE[name] = d
    return _CACHE[name]


def oracle_routing(name):
    key = ("routing", name)
    if key not in _CACHE:
        d = inputs(name)
        w = d["w"]
        idx, wt = oracle.topk_gate(d["scores"], w.num_topk, renormalize=w.renormalize)
        _CACHE[key] = (idx, wt) + oracle.token_map(idx, w.num_experts)
    return _CACHE[key]


# --------------------------------------------------------------------------- cast / fp8


def test_e4m3_conversion_every_bf16_value():
    """Groups whose amax is 448 have sf = 1 and inv = 1, so the codes are the
    hardware conversion of the raw values: every finite bf16 with |v| <= 448."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    b16 = bits[keep].astype(np.uint16)
    per = 127
    ngroups = -(-b16.size // per)
    groups = np.zeros((ngroups, 128), np.uint16)
    groups[:, 0] = 0x43E0  # 448.0 in bf16
    flat = np.zeros(ngroups * per, np.uint16)
    flat[:b16.size] = b16
    groups[:, 1:] = flat.reshape(ngroups, per)
    G = 8
    rows = -(-ngroups // G)
    x = np.zeros((rows * G, 128), np.uint16)
    x[:ngroups] = groups
    x = x.reshape(rows, G * 128)
    _log(f"identity cast of all bf16 values: x {x.shape}")
    q, sf, _ = moe.moe_expand_cast_fp8(d_bf16(x))
    torch.cuda.synchronize()
    oq, osf, _ = oracle.expand_cast_fp8(x)
    assert bits_equal(h(sf), osf)
    assert bits_equal(h(q), oq)


def test_identity_cast_wide_magnitudes():
    rng = np.random.default_rng(21)
    T, H = 333, 1536
    scale = np.float32(2.0) ** rng.integers(-40, 40, (T, 1)).astype(np.float32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * scale)
    x[5, :] = 0          # all-zero row
    x[6, :128] = 0x8000  # -0 group
    x[7, 128:256] = 0x0001  # subnormal bf16 group
    _log(f"identity cast wide magnitudes T={T} H={H}")
    q, sf, _ = moe.moe_expand_cast_fp8(d_bf16(x))
    torch.cuda.synchronize()
    oq, osf, _ = oracle.expand_cast_fp8(x)
    assert bits_equal(h(sf), osf)
    assert bits_equal(h(q), oq)


@pytest.mark.parametrize("H", [128, 256, 1024, 2048, 4096, 7168, 8192, 16384, 20480])
def test_identity_cast_hidden_sizes(H):
    rng = np.random.default_rng(H)
    T = 19
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * 3)
    _log(f"identity cast T={T} H={H}")
    q, sf, _ = moe.moe_expand_cast_fp8(d_bf16(x))
    torch.cuda.synchronize()
    oq, osf, _ = oracle.expand_cast_fp8(x)
    assert bits_equal(h(sf), osf) and bits_equal(h(q), oq)


@pytest.mark.parametrize("K", [1, 4])
@pytest.mark.parametrize("T", [16384, 16385])
def test_expand_across_the_load_kind_threshold(T, K):
    """Inputs up to 128 MiB take the expand instance with ordinary loads, larger ones the streaming-load
    instance: both sides of the boundary (hidden 4096, so 16384 rows are exactly 128 MiB), for the flat kernel
    (K = 1, identity cast) and the split-copy kernel (K = 4, with weights)."""
    rng = np.random.default_rng(T + K)
    H, E = 4096, 64
    x = W.f32_to_bf16_bits((rng.standard_normal((T, H)) * 2).astype(np.float32))
    _log(f"expand load-kind threshold T={T} H={H} K={K}")
    if K == 1:
        q, sf, _ = moe.moe_expand_cast_fp8(d_bf16(x))
        torch.cuda.synchronize()
        oq, osf, _ = oracle.expand_cast_fp8(x)
    else:
        s = rng.standard_normal((T, E)).astype(np.float32)
        idx, wt = oracle.topk_gate(s, K, with_weights=True)
        _, _, pos, _ = oracle.token_map(idx, E)
        q, sf, ow = moe.moe_expand_cast_fp8(d_bf16(x), d_i32(pos), d_f32(wt))
        torch.cuda.synchronize()
        oq, osf, oow = oracle.expand_cast_fp8(x, pos, wt)
        assert bits_equal(h(ow), oow)
    assert bits_equal(h(sf), osf)
    assert bits_equal(h(q.view(torch.uint8)), oq)


# --------------------------------------------------------------------------- top-k


@pytest.mark.parametrize("name", ["tiny", "mid", "dsv3", "large"])
def test_topk_workloads(name):
    d = inputs(name)
    w = d["w"]
    _log(f"topk {name} T={w.num_tokens} E={w.num_experts} K={w.num_topk} renorm={w.renormalize}")
    idx, wt = moe.moe_topk_gate(d_f32(d["scores"]), w.num_topk, renormalize=w.renormalize)
    torch.cuda.synchronize()
    oidx, owt = oracle_routing(name)[:2]
    assert bits_equal(h(idx), oidx)
    if w.renormalize:
        assert bits_equal(h(wt), owt)


@pytest.mark.parametrize("E", [1, 3, 16, 64, 65, 100, 128, 255, 256, 257, 512, 1000, 1024])
def test_topk_ties_and_shapes(E):
    rng = np.random.default_rng(E)
    T = 37
    vals = np.array([-1.0, 0.0, -0.0, 0.5, 1.0, -np.inf, 2.0], np.float32)
    s = vals[rng.integers(0, len(vals), (T, E))]
    s[::5] = rng.standard_normal((len(s[::5]), E)).astype(np.float32)
    s[3, :] = np.nan if E > 1 else 0.0
    s[4, : E // 2] = np.nan
    for K in sorted({1, min(E, 2), min(E, 8), min(E, 16)}):
        _log(f"topk ties T={T} E={E} K={K}")
        idx, wt = moe.moe_topk_gate(d_f32(s), K, with_weights=True)
        torch.cuda.synchronize()
        oidx, owt = oracle.topk_gate(s, K, with_weights=True)
        assert bits_equal(h(idx), oidx), (E, K)
        assert bits_equal(h(wt), owt), (E, K)


def test_topk_unaligned_scores_and_renormalise():
    rng = np.random.default_rng(3)
    T, E, K = 129, 256, 8
    s = (1 / (1 + np.exp(-rng.standard_normal((T, E))))).astype(np.float32)
    flat = torch.empty(T * E + 1, dtype=torch.float32, device="cuda")
    flat[1:] = d_f32(s).reshape(-1)
    s_dev = flat[1:].view(T, E)  # 4-byte but not 16-byte aligned: scalar-load path
    assert s_dev.data_ptr() % 16 != 0
    _log("topk unaligned scores, renormalize")
    idx, wt = moe.moe_topk_gate(s_dev, K, renormalize=True)
    torch.cuda.synchronize()
    oidx, owt = oracle.topk_gate(s, K, renormalize=True)
    assert bits_equal(h(idx), oidx) and bits_equal(h(wt), owt)


# --------------------------------------------------------------------------- token map


def _check_map(idx_np, E, with_row_token=True):
    T, K = idx_np.shape
    _log(f"token map T={T} K={K} E={E}")
    counts, offsets, pos, rt = moe.moe_token_map(d_i64(idx_np), E, with_row_token=with_row_token)
    torch.cuda.synchronize()
    oc, oo, op, ort = oracle.token_map(idx_np, E)
    assert bits_equal(h(counts), oc)
    assert bits_equal(h(offsets), oo)
    assert bits_equal(h(pos), op)
    if with_row_token:
        assert bits_equal(h(rt), ort)


@pytest.mark.parametrize("name", ["tiny", "mid", "dsv3", "large"])
def test_token_map_workloads(name):
    w = inputs(name)["w"]
    _check_map(oracle_routing(name)[0], w.num_experts)


@pytest.mark.parametrize("T,K,E", [(1, 1, 1), (1, 8, 256), (100, 16, 1024), (128, 16, 600), (256, 8, 256),
                                   (257, 8, 256), (5000, 8, 256), (70000, 8, 256),
                                   (3000, 16, 1024), (777, 6, 64), (4096, 2, 16), (8192, 8, 256),
                                   (8193, 8, 256)])
def test_token_map_shapes(T, K, E):
    rng = np.random.default_rng(T + K + E)
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = oracle.topk_gate(s, K)
    _check_map(idx, E)


def test_token_map_duplicates_out_of_range_and_skew():
    rng = np.random.default_rng(8)
    T, K, E = 3001, 8, 256
    idx = rng.integers(-3, E + 3, (T, K)).astype(np.int64)  # duplicates and out-of-range ids
    idx[::7] = 5  # a hot expert
    idx[1, 0] = np.iinfo(np.int64).max
    idx[2, 0] = np.iinfo(np.int64).min
    _check_map(idx, E)
    _check_map(idx, E, with_row_token=False)


def test_token_map_zero_tokens_zeroes_counts():
    E = 64
    counts = torch.full((E,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), 7, dtype=torch.int32, device="cuda")
    pos = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    _log("token map T=0")
    moe.moe_token_map(torch.empty((0, 4), dtype=torch.int64, device="cuda"), E,
                      with_row_token=False, out=(counts, offsets, pos, None))
    torch.cuda.synchronize()
    assert h(counts).tolist() == [0] * E and h(offsets).tolist() == [0] * (E + 1)


# --------------------------------------------------------------------------- expand


@pytest.mark.parametrize("name", ["tiny", "mid", "dsv3", "large"])
def test_expand_workloads(name):
    d = inputs(name)
    w = d["w"]
    oidx, owt, oc, oo, opos, ort = oracle_routing(name)
    R = w.num_tokens * w.num_topk
    _log(f"expand {name} T={w.num_tokens} H={w.hidden} K={w.num_topk} R={R} weights={owt is not None}")
    q, sf, ow = moe.moe_expand_cast_fp8(d_bf16(d["x"]), d_i32(opos),
                                        d_f32(owt) if owt is not None else None)
    torch.cuda.synchronize()
    gq, gsf = h(q), h(sf)
    del q, sf
    eq, esf, eow = oracle.expand_cast_fp8(d["x"], opos, owt)
    assert bits_equal(gsf, esf)
    assert bits_equal(gq, eq)
    if owt is not None:
        assert bits_equal(h(ow), eow)
    if name == "mid":  # identity mode equals the expanded rows of each token
        _log("identity cast mid")
        iq, isf, _ = moe.moe_expand_cast_fp8(d_bf16(d["x"]))
        torch.cuda.synchronize()
        iq = h(iq)
        assert np.array_equal(gq[opos[:, 3]], iq)


def test_expand_negative_pos_leaves_rows_untouched():
    rng = np.random.default_rng(9)
    T, K, H = 50, 4, 512
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    pos = rng.permutation(T * K).astype(np.int32).reshape(T, K)
    pos[rng.random((T, K)) < 0.2] = -1
    pos[0, 0] = T * K + 5  # out of range: skipped too
    q = torch.full((T * K, H), 0xAB, dtype=torch.uint8, device="cuda")
    sf = torch.full((T * K, H // 128), -5.0, dtype=torch.float32, device="cuda")
    _log("expand with skipped rows")
    moe.moe_expand_cast_fp8(d_bf16(x), d_i32(pos), out=(q, sf, None))
    torch.cuda.synchronize()
    oq = np.full((T * K, H), 0xAB, np.uint8)
    osf = np.full((T * K, H // 128), -5.0, np.float32)
    oracle.expand_cast_fp8(x, pos, out=(oq, osf, None))
    assert bits_equal(h(q), oq) and bits_equal(h(sf), osf)


def test_expand_guard_bytes_and_stream():
    rng = np.random.default_rng(10)
    T, K, H, E = 300, 8, 7168, 256
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, wt = oracle.topk_gate(s, K, renormalize=False, with_weights=True)
    _, _, pos, _ = oracle.token_map(idx, E)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    R, G, pad = T * K, H // 128, 4096
    qbuf = torch.full((R * H + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((R * G + 2 * pad,), 3.0, dtype=torch.float32, device="cuda")
    wbuf = torch.full((R + 2 * pad,), 3.0, dtype=torch.float32, device="cuda")
    q = qbuf[pad:pad + R * H].view(R, H)
    sf = sbuf[pad:pad + R * G].view(R, G)
    ow = wbuf[pad:pad + R]
    stream = torch.cuda.Stream()
    xd, pd, wd = d_bf16(x), d_i32(pos), d_f32(wt)
    torch.cuda.synchronize()
    _log("expand on a side stream with guard bytes")
    with torch.cuda.stream(stream):
        moe.moe_expand_cast_fp8(xd, pd, wd, out=(q, sf, ow))
    stream.synchronize()
    qb, sb, wb = h(qbuf), h(sbuf), h(wbuf)
    assert np.all(qb[:pad] == 0x5A) and np.all(qb[-pad:] == 0x5A)
    assert np.all(sb[:pad] == 3.0) and np.all(sb[-pad:] == 3.0)
    assert np.all(wb[:pad] == 3.0) and np.all(wb[-pad:] == 3.0)
    eq, esf, eow = oracle.expand_cast_fp8(x, pos, wt)
    assert bits_equal(qb[pad:-pad].reshape(R, H), eq)
    assert bits_equal(sb[pad:-pad].reshape(R, G), esf)
    assert bits_equal(wb[pad:-pad], eow)


def test_zero_tokens_are_noops():
    _log("T=0 no-ops")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, sf, _ = moe.moe_expand_cast_fp8(x)
    idx, _ = moe.moe_topk_gate(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 2)
    sq, ssf = moe.swiglu_cast_fp8(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert q.numel() == 0 and idx.numel() == 0 and sq.numel() == 0


# --------------------------------------------------------------------------- pipeline


def test_full_gpu_pipeline_dsv3_deterministic():
    d = inputs("dsv3")
    w = d["w"]
    s_d, x_d = d_f32(d["scores"]), d_bf16(d["x"])
    outs = []
    for rep in range(2):
        _log(f"dsv3 GPU pipeline run {rep}")
        idx, wt = moe.moe_topk_gate(s_d, w.num_topk, renormalize=True)
        counts, offsets, pos, rt = moe.moe_token_map(idx, w.num_experts)
        q, sf, ow = moe.moe_expand_cast_fp8(x_d, pos, wt)
        torch.cuda.synchronize()
        outs.append([h(t) for t in (idx, wt, counts, offsets, pos, rt, q, sf, ow)])
    for a, b in zip(outs[0], outs[1]):
        assert bits_equal(a, b)
    oidx, owt, oc, oo, opos, ort = oracle_routing("dsv3")
    eq, esf, eow = oracle.expand_cast_fp8(d["x"], opos, owt)
    for got, want in zip(outs[0], (oidx, owt, oc, oo, opos, ort, eq, esf, eow)):
        assert bits_equal(got, want)


# --------------------------------------------------------------------------- SwiGLU


def _check_swiglu(gu, rw=None, clamp=0.0, exact=False):
    R, two_i = gu.shape
    _log(f"swiglu R={R} I={two_i // 2} weights={rw is not None} clamp={clamp}")
    q, sf = moe.swiglu_cast_fp8(d_bf16(gu), d_f32(rw) if rw is not None else None, clamp)
    torch.cuda.synchronize()
    gq, gsf = h(q), h(sf)
    oq, osf = oracle.swiglu_cast_fp8(gu, rw, clamp)
    ok, det = swiglu_tolerance_report(gq, gsf, oq, osf)
    _log(f"  {det}")
    assert ok, det
    if exact:
        assert bits_equal(gq, oq) and bits_equal(gsf, osf)
    return det


def test_swiglu_workload():
    d = inputs("swiglu")
    _check_swiglu(d["gate_up"], d["row_weights"])


def test_swiglu_large_step_sampled():
    """The benchmark step's SwiGLU at its full size and launch configuration:
    the 262144 routed rows of the large batch (I = 2048, U(0,1) row weights,
    the same seeded input the step draws), one call over all rows.  Rows are
    independent, so the oracle checks a sample: the first and last 1024 rows
    and 2048 drawn at random."""
    w = W.WORKLOADS["large"]
    R, I = w.num_tokens * w.num_topk, 2048
    gu = W.make_gate_up(w, rows=R, inter=I)
    rw = W.make_row_weights(w, rows=R)
    _log(f"swiglu full step R={R} I={I}")
    q, sf = moe.swiglu_cast_fp8(d_bf16(gu), d_f32(rw))
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([np.arange(1024), np.arange(R - 1024, R), rng.choice(R, 2048, replace=False)]))
    sel = torch.from_numpy(rows).cuda()
    gq, gsf = h(q.view(torch.uint8)[sel]), h(sf[sel])
    del q, sf
    oq, osf = oracle.swiglu_cast_fp8(gu[rows], rw[rows])
    ok, det = swiglu_tolerance_report(gq, gsf, oq, osf)
    _log(f"  {rows.size} sampled rows: {det}")
    assert ok, det


def test_swiglu_tiny_with_and_without_weights():
    d = inputs("tiny")
    _check_swiglu(d["gate_up"], d["row_weights"])
    _check_swiglu(d["gate_up"], None)


def test_swiglu_clamp_and_wide_range():
    rng = np.random.default_rng(12)
    R, I = 257, 1024
    gu = W.f32_to_bf16_bits((rng.standard_normal((R, 2 * I)) * 12).astype(np.float32))
    _check_swiglu(gu, rng.random(R, dtype=np.float32), clamp=7.0)
    _check_swiglu(gu, None)


def test_swiglu_exact_regions():
    # gate >= 17: silu(gate) == gate; products of bf16 are exact -> bit-exact
    rng = np.random.default_rng(13)
    R, I = 64, 512
    gate = rng.uniform(17, 80, (R, I)).astype(np.float32)
    up = rng.standard_normal((R, I)).astype(np.float32)
    gu = np.concatenate([W.f32_to_bf16_bits(gate), W.f32_to_bf16_bits(up)], axis=1)
    _check_swiglu(gu, exact=True)
    # gate == 0 and gate <= -89 give signed zeros everywhere
    gz = np.concatenate([np.zeros((R, I), np.uint16), W.f32_to_bf16_bits(up)], axis=1)
    _check_swiglu(gz, exact=True)
    gneg = np.concatenate([W.f32_to_bf16_bits(np.full((R, I), -120.0, np.float32)),
                           W.f32_to_bf16_bits(up)], axis=1)
    _check_swiglu(gneg, exact=True)


@pytest.mark.parametrize("group", [16, 32])
def test_e4m3_entry_points_small_groups(group):
    """moe_expand_cast_fp8 and swiglu_cast_fp8 with groups of 16 or 32 (the block-scaled kernels in the
    e4m3 / fp32-scale format) against the oracle's same functions at that group size."""
    rng = np.random.default_rng(700 + group)
    T, E, K, H = 333, 64, 6, 1024
    _log(f"e4m3 entry points, groups of {group}")
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, wt = oracle.topk_gate(s, K, with_weights=True)
    _, _, pos, _ = oracle.token_map(idx, E)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    q, sf, ow = moe.moe_expand_cast_fp8(d_bf16(x), d_i32(pos), d_f32(wt), group_size=group)
    qi, sfi, _ = moe.moe_expand_cast_fp8(d_bf16(x), group_size=group)
    R, I = 301, 640
    gu = W.f32_to_bf16_bits(rng.standard_normal((R, 2 * I)).astype(np.float32))
    rw = rng.random(R, dtype=np.float32)
    sq, ssf = moe.swiglu_cast_fp8(d_bf16(gu), d_f32(rw), group_size=group)
    torch.cuda.synchronize()
    eq, esf, eow = oracle.expand_cast_fp8(x, pos, wt, group_size=group)
    assert bits_equal(h(q.view(torch.uint8)), eq) and bits_equal(h(sf), esf) and bits_equal(h(ow), eow)
    eqi, esfi, _ = oracle.expand_cast_fp8(x, None, None, group_size=group)
    assert bits_equal(h(qi.view(torch.uint8)), eqi) and bits_equal(h(sfi), esfi)
    oq, osf = oracle.swiglu_cast_fp8(gu, rw, group_size=group)
    ok, det = swiglu_tolerance_report(h(sq.view(torch.uint8)), h(ssf), oq, osf, group=group)
    assert ok, det


def test_very_wide_rows():
    """Hidden 32768 for the expand (32 chunks of 1024 channels per row, 256 groups) and I = 16384 for the
    SwiGLU (8 passes of a 256-thread row workgroup), against the oracle."""
    rng = np.random.default_rng(811)
    T, E, K, H = 37, 64, 8, 32768
    _log(f"very wide rows H={H}")
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, wt = oracle.topk_gate(s, K, with_weights=True)
    _, _, pos, _ = oracle.token_map(idx, E)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    q, sf, ow = moe.moe_expand_cast_fp8(d_bf16(x), d_i32(pos), d_f32(wt))
    R, I = 29, 16384
    gu = W.f32_to_bf16_bits(rng.standard_normal((R, 2 * I)).astype(np.float32))
    sq, ssf = moe.swiglu_cast_fp8(d_bf16(gu), None)
    torch.cuda.synchronize()
    eq, esf, eow = oracle.expand_cast_fp8(x, pos, wt)
    assert bits_equal(h(q.view(torch.uint8)), eq) and bits_equal(h(sf), esf) and bits_equal(h(ow), eow)
    oq, osf = oracle.swiglu_cast_fp8(gu, None)
    ok, det = swiglu_tolerance_report(h(sq.view(torch.uint8)), h(ssf), oq, osf)
    assert ok, det
