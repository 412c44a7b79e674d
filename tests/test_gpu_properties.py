"""Property-based GPU parity (hypothesis): generated inputs through the C ABI
against the oracle, bit for bit.  The strategies reach the corners the
seeded workloads rarely touch: NaN, +-inf, +-0 and heavy ties in the scores
(every expert count from 1 to 1024, so both the vector and the scalar load
paths), ids outside [0, E) and repeated ids for the map up to multi-chunk
sizes, and bf16 activations with zeros, subnormals and values near the
bf16 range for the expand."""
import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from hypothesis.extra.numpy import arrays

import moe_routing_fp8_amd as moe
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

SPECIAL = [0.0, -0.0, 1.0, -1.0, 0.5, float("inf"), float("-inf"), float("nan"), 3.0e38, -1e-40]
# derandomize: the same examples on every run, so a test run is reproducible
SETTINGS = settings(max_examples=100, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _log(msg):
    sys.__stderr__.write(f"[gpu-properties] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@st.composite
def topk_case(draw):
    E = draw(st.sampled_from([1, 2, 3, 7, 16, 63, 64, 65, 100, 128, 255, 256, 257, 511, 512, 700, 1024]))
    T = draw(st.integers(1, 40))
    K = draw(st.integers(1, min(E, 16)))
    elems = st.one_of(st.sampled_from(SPECIAL), st.floats(-2, 2, width=32))
    s = draw(arrays(np.float32, (T, E), elements=elems))
    return s, K


@SETTINGS
@given(topk_case())
def test_topk_matches_oracle(case):
    s, K = case
    T, E = s.shape
    idx, w = moe.moe_topk_gate(torch.from_numpy(s).cuda(), K, with_weights=True)
    torch.cuda.synchronize()
    ei, ew = oracle.topk_gate(s, K, with_weights=True)
    assert np.array_equal(idx.cpu().numpy(), ei), (T, E, K)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), ew.view(np.uint32)), (T, E, K)


@st.composite
def map_case(draw):
    E = draw(st.sampled_from([1, 5, 16, 256, 600, 1024]))
    K = draw(st.integers(1, 16))
    T = draw(st.sampled_from([1, 3, 64, 200, 257, 1500, 3000]))
    lo, hi = draw(st.sampled_from([(0, E - 1), (-2, E + 2), (0, min(E - 1, 3))]))  # in range / out of range / hot
    seed = draw(st.integers(0, 2 ** 32 - 1))
    ids = np.random.default_rng(seed).integers(lo, hi + 1, (T, K), dtype=np.int64)
    return ids, E


@SETTINGS
@given(map_case())
def test_token_map_matches_oracle(case):
    ids, E = case
    counts, offsets, pos, row_token = moe.moe_token_map(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    ec, eo, ep, er = oracle.token_map(ids, E)
    assert np.array_equal(counts.cpu().numpy(), ec) and np.array_equal(offsets.cpu().numpy(), eo)
    assert np.array_equal(pos.cpu().numpy(), ep) and np.array_equal(row_token.cpu().numpy(), er)


BF16_SPECIAL = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F, 0x4380, 0x43E0,
                0x43E8, 0x3C00]  # zeros, subnormals, smallest normal, +-1, +-max, 256, 448, 464, 2^-7


@st.composite
def expand_case(draw):
    T = draw(st.integers(1, 24))
    H = 128 * draw(st.integers(1, 12))
    K = draw(st.integers(1, 8))
    E = draw(st.sampled_from([8, 16, 256]))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * np.float32(draw(st.sampled_from(
        [1.0, 1e-3, 1e3, 1e-30]))))
    mask = rng.random((T, H)) < draw(st.sampled_from([0.0, 0.05, 0.5]))
    x[mask] = rng.choice(np.array(BF16_SPECIAL, np.uint16), int(mask.sum()))
    s = rng.standard_normal((T, E)).astype(np.float32)
    return x, s, K


@SETTINGS
@given(expand_case())
def test_expand_matches_oracle(case):
    x, s, K = case
    E = s.shape[1]
    K = min(K, E)
    idx, w = oracle.topk_gate(s, K, with_weights=True)
    _, _, pos, _ = oracle.token_map(idx, E)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    q, sf, ow = moe.moe_expand_cast_fp8(xd, torch.from_numpy(pos).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    eq, esf, eow = oracle.expand_cast_fp8(x, pos, w)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), eq)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), esf.view(np.uint32))
    assert np.array_equal(ow.cpu().numpy().view(np.uint32), eow.view(np.uint32))


GATE_SPECIAL = [0x0000, 0x8000, 0x4188, 0x41A0, 0xC2B2, 0xC2C8, 0x42C8, 0x3F80, 0xBF80, 0x0001, 0x4700, 0xC700]
# zeros, 17, 20, -89, -100, 100, +-1, a subnormal, +-32768


@st.composite
def swiglu_case(draw):
    R = draw(st.integers(1, 40))
    I = 128 * draw(st.integers(1, 8))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    gu = W.f32_to_bf16_bits(rng.standard_normal((R, 2 * I)).astype(np.float32) * np.float32(
        draw(st.sampled_from([1.0, 8.0, 1e-3]))))
    mask = rng.random((R, 2 * I)) < draw(st.sampled_from([0.0, 0.1, 0.6]))
    gu[mask] = rng.choice(np.array(GATE_SPECIAL, np.uint16), int(mask.sum()))
    w = None
    if draw(st.booleans()):
        w = rng.random(R, dtype=np.float32)
        w[rng.random(R) < 0.2] = 0.0
    clamp = draw(st.sampled_from([0.0, 7.0, 0.75]))
    return gu, w, clamp


@SETTINGS
@given(swiglu_case())
def test_swiglu_within_tolerance_of_oracle(case):
    from oracle.compare import swiglu_tolerance_report

    gu, w, clamp = case
    gud = torch.from_numpy(gu.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.from_numpy(w).cuda() if w is not None else None
    q, sf = moe.swiglu_cast_fp8(gud, wd, clamp_value=clamp)
    torch.cuda.synchronize()
    eq, esf = oracle.swiglu_cast_fp8(gu, w, clamp_value=clamp)
    ok, det = swiglu_tolerance_report(q.view(torch.uint8).cpu().numpy(), sf.cpu().numpy(), eq, esf)
    assert ok, det


@st.composite
def format_case(draw):
    dtype = draw(st.sampled_from(["e4m3", "e2m1"]))
    group = draw(st.sampled_from([16, 32, 128]))
    round_sf = draw(st.booleans())
    ue8m0 = round_sf and draw(st.booleans())
    T = draw(st.integers(1, 16))
    H = 128 * draw(st.integers(1, 6))
    K = draw(st.integers(1, 6))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * np.float32(
        draw(st.sampled_from([1.0, 1e-3, 1e3, 1e-38]))))
    mask = rng.random((T, H)) < draw(st.sampled_from([0.0, 0.05, 0.5]))
    x[mask] = rng.choice(np.array(BF16_SPECIAL, np.uint16), int(mask.sum()))
    s = rng.standard_normal((T, 16)).astype(np.float32)
    return x, s, K, dtype, group, round_sf, ue8m0


@SETTINGS
@given(format_case())
def test_block_scaled_expand_matches_oracle(case):
    x, s, K, dtype, group, round_sf, ue8m0 = case
    idx, w = oracle.topk_gate(s, K, with_weights=True)
    _, _, pos, _ = oracle.token_map(idx, 16)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    q, sf, ow = moe.moe_expand_cast(xd, torch.from_numpy(pos).cuda(), torch.from_numpy(w).cuda(), dtype=dtype,
                                    group_size=group, round_sf=round_sf, sf_ue8m0=ue8m0)
    torch.cuda.synchronize()
    fmt = oracle.FMT_E2M1 if dtype == "e2m1" else oracle.FMT_E4M3
    eq, esf, eow = oracle.expand_cast(x, pos, w, dtype=fmt, group_size=group, round_sf=round_sf, sf_ue8m0=ue8m0)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), eq)
    assert np.array_equal(sf.cpu().numpy().view(np.uint8), esf.view(np.uint8))
    assert np.array_equal(ow.cpu().numpy().view(np.uint32), eow.view(np.uint32))


@st.composite
def combine_case(draw):
    T = draw(st.integers(1, 30))
    K = draw(st.integers(1, 16))
    H = 8 * draw(st.integers(1, 200))
    R = draw(st.integers(1, 3 * T * K))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    pos = rng.integers(-2, R + 2, (T, K)).astype(np.int32)  # out-of-range entries are skipped; repeats allowed
    y = W.f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32) * np.float32(
        draw(st.sampled_from([1.0, 1e-20, 1e20]))))
    w = rng.standard_normal((T, K)).astype(np.float32) if draw(st.booleans()) else None
    return y, pos, w


@SETTINGS
@given(combine_case())
def test_combine_matches_oracle(case):
    y, pos, w = case
    yd = torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.from_numpy(w).cuda() if w is not None else None
    out = moe.moe_combine(yd, torch.from_numpy(pos).cuda(), wd)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), oracle.combine(y, pos, w))


@st.composite
def padded_case(draw):
    T = draw(st.integers(1, 300))
    E = draw(st.sampled_from([8, 64, 256]))
    K = draw(st.integers(1, min(8, E)))
    begin = draw(st.integers(0, E - 1))
    end = draw(st.integers(begin + 1, E))
    align = draw(st.sampled_from([1, 2, 16, 128]))
    extra = draw(st.integers(0, 40))
    H = 128 * draw(st.integers(1, 3))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    return T, E, K, begin, end, align, extra, H, seed


@SETTINGS
@given(padded_case())
def test_aligned_map_and_padded_expand_match_oracle(case):
    T, E, K, begin, end, align, extra, H, seed = case
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.topk_gate(s, K, with_weights=True)
    rows = oracle.padded_rows_bound(T, K, end - begin, align) + extra
    counts, offsets, pos, row_token = moe.moe_token_map_aligned(torch.from_numpy(idx).cuda(), begin, end, align,
                                                                num_rows=rows)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    q, sf, ow = moe.moe_expand_cast_fp8_padded(torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16), pos,
                                               row_token, torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    ec, eo, ep, er = oracle.token_map_aligned(idx, begin, end, align, num_rows=rows)
    assert np.array_equal(counts.cpu().numpy(), ec) and np.array_equal(offsets.cpu().numpy(), eo)
    assert np.array_equal(pos.cpu().numpy(), ep) and np.array_equal(row_token.cpu().numpy(), er)
    eq, esf, eow = oracle.expand_cast_fp8_padded(x, ep, er, w)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), eq)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), esf.view(np.uint32))
    assert np.array_equal(ow.cpu().numpy().view(np.uint32), eow.view(np.uint32))


@st.composite
def dispatch_case(draw):
    mode = draw(st.sampled_from([moe.MOE_DISPATCH_SINGLE_LAUNCH, moe.MOE_DISPATCH_SPLIT, moe.MOE_DISPATCH_AUTO,
                                 moe.MOE_DISPATCH_ROUTE_FUSED, moe.MOE_DISPATCH_TOPK_THEN_COPY]))
    T = draw(st.integers(1, 64))
    E = draw(st.sampled_from([4, 16, 64, 256, 1000]))
    K = draw(st.integers(1, min(8, E)))
    H = 128 * draw(st.sampled_from([1, 2, 8, 56]))
    renorm = draw(st.booleans())
    ties = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 32 - 1))
    return mode, T, E, K, H, renorm, ties, seed


# tie-heavy score sets: with renormalisation positive values only (a zero or non-finite sum has no
# single IEEE NaN bit pattern to compare), without it +-0, NaN and -inf as well
TIES_RENORM = np.array([0.25, 0.5, 0.75, 1.0], np.float32)
TIES_PLAIN = np.array([1.0, 0.5, 0.0, -0.0, -1.0, np.nan, -np.inf], np.float32)


@SETTINGS
@given(dispatch_case())
def test_dispatch_forms_match_oracle(case):
    mode, T, E, K, H, renorm, ties, seed = case
    rng = np.random.default_rng(seed)
    if ties:
        s = rng.choice(TIES_RENORM if renorm else TIES_PLAIN, (T, E))
    else:
        s = rng.standard_normal((T, E)).astype(np.float32)
        if renorm:
            s = (1.0 / (1.0 + np.exp(-s.astype(np.float64)))).astype(np.float32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    out = moe.moe_dispatch(torch.from_numpy(s).cuda(), torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16),
                           K, renormalize=renorm, with_weights=True, mode=mode)
    torch.cuda.synchronize()
    ei, ew = oracle.topk_gate(s, K, renormalize=renorm, with_weights=True)
    ec, eo, ep, er = oracle.token_map(ei, E)
    eq, esf, eow = oracle.expand_cast_fp8(x, ep, ew)
    assert np.array_equal(out["topk_idx"].cpu().numpy(), ei)
    assert np.array_equal(out["topk_weights"].cpu().numpy().view(np.uint32), ew.view(np.uint32))
    assert np.array_equal(out["counts"].cpu().numpy(), ec) and np.array_equal(out["offsets"].cpu().numpy(), eo)
    assert np.array_equal(out["pos"].cpu().numpy(), ep) and np.array_equal(out["row_token"].cpu().numpy(), er)
    assert np.array_equal(out["out"].view(torch.uint8).cpu().numpy(), eq)
    assert np.array_equal(out["out_sf"].cpu().numpy().view(np.uint32), esf.view(np.uint32))
    assert np.array_equal(out["out_weights"].cpu().numpy().view(np.uint32), eow.view(np.uint32))


@st.composite
def route_case(draw):
    """Scores with NaN, +-inf, +-0 and ties over every top-k register width, T spanning one to many
    workgroups and super-chunks of the fused routing."""
    E = draw(st.sampled_from([1, 3, 16, 64, 65, 100, 256, 257, 512, 700, 1024]))
    T = draw(st.sampled_from([1, 2, 15, 16, 17, 33, 100, 255, 256, 257, 600]))
    K = draw(st.integers(1, min(E, 16)))
    elems = st.one_of(st.sampled_from(SPECIAL), st.floats(-2, 2, width=32))
    s = draw(arrays(np.float32, (T, E), elements=elems))
    mode = draw(st.sampled_from([moe.MOE_ROUTE_FUSED, moe.MOE_ROUTE_AUTO, moe.MOE_ROUTE_LOCAL]))
    if mode == moe.MOE_ROUTE_LOCAL and T > 32:  # the local form takes at most 32 tokens
        mode = moe.MOE_ROUTE_AUTO
    return s, K, mode


@SETTINGS
@given(route_case())
def test_route_matches_oracle(case):
    s, K, mode = case
    T, E = s.shape
    ws = torch.zeros(moe.moe_route_workspace_bytes(T, K, E), dtype=torch.uint8, device="cuda")
    r = moe.moe_route(torch.from_numpy(s).cuda(), K, with_weights=True, mode=mode, workspace=ws)
    torch.cuda.synchronize()
    ei, ew = oracle.topk_gate(s, K, with_weights=True)
    ec, eo, ep, er = oracle.token_map(ei, E)
    assert np.array_equal(r["topk_idx"].cpu().numpy(), ei)
    assert np.array_equal(r["topk_weights"].cpu().numpy().view(np.uint32), ew.view(np.uint32))
    assert np.array_equal(r["counts"].cpu().numpy(), ec) and np.array_equal(r["offsets"].cpu().numpy(), eo)
    assert np.array_equal(r["pos"].cpu().numpy(), ep) and np.array_equal(r["row_token"].cpu().numpy(), er)
