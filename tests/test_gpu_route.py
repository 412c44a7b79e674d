"""GPU parity of moe_route (top-k gating, group counting and the token map
with the top-k and the counting fused, two launches: "DeepSeek open-sources
TileKernels", section 2, the routing chain; "CuTeDSL at Perplexity", MoE
dispatch) and of moe_dispatch's MOE_DISPATCH_ROUTE_FUSED form, against the
oracle's top-k and map composed, bit for bit.

Covered: the mid batch, the DeepSeek-V3 layer and the large batch in full;
every top-k register width and both workgroup sizes (E from 8 to 1024); K
from 1 to 16; token counts around the workgroup size and around the
super-chunk group sizes (1, 15, 16, 17, 129, 256, 257 ...); the largest batch
the fused form takes (one token more is refused, and routed by the split form
under AUTO); renormalised, raw and absent weights; unaligned scores; ties and
NaN scores; one workspace reused across fused calls of different grid sizes
and expert counts, split calls and the single-launch dispatch (the table the
next call adds into must be zero after every fused call); a side stream while
the current stream is the default one; the split form; T = 0."""
import math
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

FUSED, SPLIT, AUTO = moe.MOE_ROUTE_FUSED, moe.MOE_ROUTE_SPLIT, moe.MOE_ROUTE_AUTO
LOCAL = moe.MOE_ROUTE_LOCAL
EPOCH = 1 << 16
WORD_PARITY, WORD_USED, WORD_EXTENT0 = 288, 296, 304  # header words of the fused form
TABLES = 2048  # two super-chunk tables of 64 x 1024 int32 after the header, alternating between calls
TABLE_INTS = 64 * 1024
MAX_BLOCKS = 4096


def _log(msg):
    sys.__stderr__.write(f"[gpu-route] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def h(t):
    return t.cpu().numpy()


def bits_equal(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), np.asarray(b, np.float32).view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


def expected(scores, K, renormalize, with_weights):
    idx, wt = oracle.topk_gate(scores, K, renormalize=renormalize, with_weights=with_weights)
    counts, offsets, pos, rt = oracle.token_map(idx, scores.shape[1])
    return {"topk_idx": idx, "topk_weights": wt, "counts": counts, "offsets": offsets, "pos": pos, "row_token": rt}


def check(res, exp, what):
    for key, want in exp.items():
        got = res.get(key)
        if want is None:
            assert got is None, (what, key)
            continue
        assert bits_equal(h(got), want), (what, key)


def header_ok(ws, copies=None):
    """After a fused call: the parity names the other table than the one used, that other table (the next
    call adds into it) is zero, and the one used holds this call's copies (its super-chunk counts)."""
    words = h(ws[:2048].view(torch.int32)).view(np.uint32)
    used = int(words[WORD_USED]) & 1
    assert int(words[WORD_PARITY]) & 1 == used ^ 1
    tables = h(ws[TABLES:TABLES + 2 * TABLE_INTS * 4].view(torch.int32)).reshape(2, TABLE_INTS)
    assert not tables[used ^ 1].any()
    assert not tables[used][int(words[WORD_EXTENT0 + used]):].any()
    if copies is not None:
        assert int(tables[used].sum()) == copies


def fresh_ws(T, K, E):
    return torch.zeros(max(moe.moe_route_workspace_bytes(T, K, E), 256), dtype=torch.uint8, device="cuda")


def tokens_per_block(E):
    return 16 if E <= 512 else 8


def fits_fused(T, E):
    """At most 4096 workgroups in at most 64 super-chunks of ceil(sqrt(G)) workgroups (above 256 workgroups
    at most 8192 / E)."""
    if T <= 0:
        return False
    G = -(-T // tokens_per_block(E))
    if G > MAX_BLOCKS:
        return False
    group = math.isqrt(G - 1) + 1
    if G > 256:  # one slot workgroup per super-chunk: its LDS holds group x E <= 8192
        group = min(group, 8192 // E)
    return -(-G // group) <= 64


def largest_fused(E):
    T = MAX_BLOCKS * tokens_per_block(E)
    while not fits_fused(T, E):
        T -= tokens_per_block(E)
    return T


def run(scores_np, K, renormalize=False, with_weights=None, mode=FUSED, ws=None, stream=None):
    s = torch.from_numpy(np.ascontiguousarray(scores_np, np.float32)).cuda()
    T, E = scores_np.shape
    if ws is None:
        ws = fresh_ws(T, K, E)
    res = moe.moe_route(s, K, renormalize=renormalize, with_weights=with_weights, mode=mode, workspace=ws,
                        stream=stream)
    torch.cuda.synchronize()
    return res, ws


@pytest.mark.parametrize("name", ["mid", "dsv3", "large"])
def test_route_workloads(name):
    """Each batch in full through the fused form (the large batch: 2048 workgroups in 64 super-chunks)."""
    w = W.WORKLOADS[name]
    T, E, K = w.num_tokens, w.num_experts, w.num_topk
    assert fits_fused(T, E)
    _log(f"workload {name} T={T} E={E} K={K}")
    scores = W.make_scores(w)
    exp = expected(scores, K, w.renormalize, w.renormalize)
    res, ws = run(scores, K, renormalize=w.renormalize, mode=FUSED)
    check(res, exp, name)
    header_ok(ws, T * K)


# (T, E, K): every top-k register width (P = 1, 2, 4, 8 with 1024-thread workgroups, 16 with 512), E not a
# multiple of 4 (scalar score loads), K from 1 to 16, T around the workgroup size (16 or 8) and the super-chunk
# group sizes (one workgroup; groups of 1 up to 16 workgroups, a ragged last group)
SHAPES = [(1, 8, 1), (15, 64, 2), (16, 64, 8), (17, 100, 6), (129, 128, 8), (256, 256, 8), (257, 256, 8),
          (300, 257, 6), (1000, 256, 12), (2048, 512, 8), (1023, 513, 16), (2000, 1024, 16), (4095, 256, 8),
          (777, 1024, 3), (3000, 96, 12), (4096, 64, 16), (4000, 64, 5), (2048, 1000, 7)]


@pytest.mark.parametrize("T,E,K", SHAPES)
def test_route_shapes(T, E, K):
    if not fits_fused(T, E):
        pytest.skip(f"T={T}: more workgroups than compute units")
    _log(f"shape T={T} E={E} K={K}")
    rng = np.random.default_rng(T * 7919 + E * 31 + K)
    scores = rng.standard_normal((T, E)).astype(np.float32)
    exp = expected(scores, K, False, True)
    res, ws = run(scores, K, with_weights=True, mode=FUSED)
    check(res, exp, (T, E, K))
    header_ok(ws, T * K)


def test_route_renormalised_unaligned_ties_and_nan():
    """Scores at a 4-byte offset (scalar loads), heavy ties, NaNs and positive scores renormalised."""
    T, E, K = 3000, 256, 8
    rng = np.random.default_rng(11)
    base = rng.integers(1, 6, (T, E + 1)).astype(np.float32) / 4.0  # few distinct values: many ties
    base[rng.random((T, E + 1)) < 0.02] = np.nan
    flat = torch.from_numpy(base.reshape(-1)).cuda()
    s = flat[1:1 + T * E].view(T, E)  # 4-byte aligned, not 16
    scores = base.reshape(-1)[1:1 + T * E].reshape(T, E)
    _log("renormalised, unaligned, ties, NaN")
    exp = expected(scores, K, True, True)
    ws = fresh_ws(T, K, E)
    res = moe.moe_route(s, K, renormalize=True, mode=FUSED, workspace=ws)
    torch.cuda.synchronize()
    check(res, exp, "ties")
    header_ok(ws, T * K)


def test_route_without_weights_or_row_token():
    T, E, K = 2500, 256, 8
    scores = np.random.default_rng(3).standard_normal((T, E)).astype(np.float32)
    exp = expected(scores, K, False, False)
    s = torch.from_numpy(scores).cuda()
    ws = fresh_ws(T, K, E)
    _log("no weights, no row_token")
    res = moe.moe_route(s, K, with_weights=False, with_row_token=False, mode=FUSED, workspace=ws)
    torch.cuda.synchronize()
    exp["row_token"] = None
    check(res, exp, "no weights")
    header_ok(ws, T * K)


@pytest.mark.parametrize("E", [64, 256, 1024])
def test_route_largest_batch_that_fits(E):
    """The largest batch the fused form takes (65536 tokens at E = 64, 32768 at 256, 4096 at 1024) at K = 16;
    one token more is refused by MOE_ROUTE_FUSED and routed by the split form under AUTO."""
    K = 16
    T = largest_fused(E)
    assert fits_fused(T, E) and not fits_fused(T + 1, E)
    _log(f"largest batch T={T} E={E} K={K}")
    scores = np.random.default_rng(17).standard_normal((T + 1, E)).astype(np.float32)
    exp = expected(scores[:T], K, False, True)
    res, ws = run(scores[:T], K, with_weights=True, mode=FUSED)
    check(res, exp, "largest")
    header_ok(ws, T * K)
    del res
    s = torch.from_numpy(scores).cuda()
    with pytest.raises(moe.MoeError):
        moe.moe_route(s, K, mode=FUSED, workspace=fresh_ws(T + 1, K, E))
    res = moe.moe_route(s, K, with_weights=True, mode=AUTO, workspace=fresh_ws(T + 1, K, E))
    torch.cuda.synchronize()
    check(res, expected(scores, K, False, True), "one more, split")


def test_route_workspace_reuse_across_shapes_and_dispatch():
    """One workspace, zeroed once, serves fused calls of different grid sizes and expert counts (a large
    table extent followed by small ones and back), split calls and the single-launch dispatch in between:
    every result is exact and the tables are left ready after every fused call."""
    K, H = 8, 1024
    ws = fresh_ws(8192, 16, 1024)
    rng = np.random.default_rng(23)
    calls = [(4096, 256, 8), (100, 256, 8), (4096, 1024, 16), (1, 64, 8), (2049, 256, 8), (4096, 512, 2),
             (17, 1024, 16), (2500, 256, 8), (4000, 1024, 16), (300, 8, 3)]
    for i, (T, E, Kc) in enumerate(calls):
        scores = rng.standard_normal((T, E)).astype(np.float32)
        mode = SPLIT if i % 4 == 3 else FUSED
        _log(f"reuse call {i}: T={T} E={E} K={Kc} mode={mode}")
        exp = expected(scores, Kc, False, True)
        res, _ = run(scores, Kc, with_weights=True, mode=mode, ws=ws)
        check(res, exp, ("reuse", i, T, E))
        if mode == FUSED:
            header_ok(ws, T * Kc)
        if i % 3 == 1:  # a single-launch dispatch on the same workspace
            Td, Ed = 8, 256
            sd = rng.standard_normal((Td, Ed)).astype(np.float32)
            x = W.f32_to_bf16_bits(rng.standard_normal((Td, H)).astype(np.float32))
            xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
            out = moe.moe_dispatch(torch.from_numpy(sd).cuda(), xd, K, with_weights=True,
                                   mode=moe.MOE_DISPATCH_SINGLE_LAUNCH, workspace=ws)
            torch.cuda.synchronize()
            assert bits_equal(h(out["pos"]), oracle.token_map(oracle.topk_gate(sd, K)[0], Ed)[2])
            if mode == FUSED:
                header_ok(ws, T * Kc)  # the single launch leaves the fused form's words and tables alone


def test_route_split_and_auto_match():
    T, E, K = 4096, 256, 8
    scores = np.random.default_rng(29).standard_normal((T, E)).astype(np.float32)
    exp = expected(scores, K, False, True)
    for mode in (SPLIT, AUTO):
        _log(f"mode {mode}")
        res, _ = run(scores, K, with_weights=True, mode=mode)
        check(res, exp, mode)


def test_route_side_stream_with_default_current():
    """stream= a side stream while the current stream stays the default one: outputs and the zeroed
    workspace are made on the side stream, so nothing races."""
    T, E, K = 4096, 256, 8
    scores = np.random.default_rng(31).standard_normal((T, E)).astype(np.float32)
    exp = expected(scores, K, False, True)
    s = torch.from_numpy(scores).cuda()
    side = torch.cuda.Stream()
    _log("side stream")
    for _ in range(3):
        res = moe.moe_route(s, K, with_weights=True, mode=FUSED, stream=side)
        side.synchronize()
        check(res, exp, "side")


def test_route_zero_tokens():
    E, K = 256, 8
    for mode in (FUSED, SPLIT, AUTO, LOCAL):
        counts = torch.full((E,), 7, dtype=torch.int32, device="cuda")
        offsets = torch.full((E + 1,), 7, dtype=torch.int32, device="cuda")
        out = {"topk_idx": torch.empty((0, K), dtype=torch.int64, device="cuda"), "topk_weights": None,
               "counts": counts, "offsets": offsets, "pos": torch.empty((0, K), dtype=torch.int32, device="cuda"),
               "row_token": torch.empty(0, dtype=torch.int32, device="cuda")}
        moe.moe_route(torch.empty((0, E), dtype=torch.float32, device="cuda"), K, mode=mode, out=out,
                      workspace=fresh_ws(0, K, E))
        torch.cuda.synchronize()
        assert not h(counts).any() and not h(offsets).any()


def test_dispatch_route_launch_form():
    """moe_dispatch's MOE_DISPATCH_ROUTE_FUSED form (routing in one launch, then the expand) against the oracle's
    top-k, map and expand, on the first 1024 tokens of the DeepSeek-V3 layer; AUTO picks the same outputs."""
    w = W.WORKLOADS["dsv3"]
    T = 1024
    scores = W.make_scores(w, num_tokens=T)
    x = W.make_x(w, num_tokens=T)
    K = w.num_topk
    idx, wt = oracle.topk_gate(scores, K, renormalize=True)
    counts, offsets, pos, rt = oracle.token_map(idx, w.num_experts)
    q, sf, ow = oracle.expand_cast_fp8(x, pos, wt)
    sd = torch.from_numpy(scores).cuda()
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    for mode in (moe.MOE_DISPATCH_ROUTE_FUSED, moe.MOE_DISPATCH_AUTO):
        _log(f"dispatch mode {mode} T={T}")
        ws = torch.zeros(moe.moe_dispatch_workspace_bytes(T, K, w.num_experts), dtype=torch.uint8, device="cuda")
        out = moe.moe_dispatch(sd, xd, K, renormalize=True, mode=mode, workspace=ws)
        torch.cuda.synchronize()
        for key, want in (("topk_idx", idx), ("topk_weights", wt), ("counts", counts), ("offsets", offsets),
                          ("pos", pos), ("row_token", rt), ("out_sf", sf), ("out_weights", ow)):
            assert bits_equal(h(out[key]), want), (mode, key)
        assert np.array_equal(h(out["out"].view(torch.uint8)), q), mode
        header_ok(ws, T * K)


def test_auto_takes_the_fused_form_where_it_is_faster():
    """AUTO takes the fused form from 129 tokens (1032 copies) up to four workgroups of 16 tokens per compute
    unit (16384 tokens on 256 compute units: the DeepSeek-V3 layer's 4096 among them) and the split form for
    one token more and for 128 tokens (1024 copies); which form ran shows in the parity word, which only the
    fused form flips."""
    K, E = 8, 256
    rng = np.random.default_rng(41)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for T, fused in ((4096, cus >= 64), (64 * cus, True), (64 * cus + 1, False), (128, False), (129, True)):
        scores = rng.standard_normal((T, E)).astype(np.float32)
        ws = fresh_ws(T, K, E)
        _log(f"AUTO T={T}: expect fused={fused}")
        res, _ = run(scores, K, with_weights=True, mode=AUTO, ws=ws)
        check(res, expected(scores, K, False, True), ("auto", T))
        parity = int(h(ws[:2048].view(torch.int32))[WORD_PARITY]) & 1
        assert parity == (1 if fused else 0), (T, parity)


def test_fused_form_under_graph_replay():
    """The fused routing captured once into a HIP graph (20 calls), replayed with new scores copied into the
    captured input between replays and eager fused calls on another workspace in between: every replay
    equals the oracle for its inputs (the tables alternate from replay to replay through the workspace's own
    words; the library records no memset)."""
    T, E, K = 2048, 256, 8
    s = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = fresh_ws(T, K, E)
    s.copy_(torch.from_numpy(np.random.default_rng(50).standard_normal((T, E)).astype(np.float32)))
    out = moe.moe_route(s, K, with_weights=True, mode=FUSED, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_route(s, K, with_weights=True, mode=FUSED, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            moe.moe_route(s, K, with_weights=True, mode=FUSED, workspace=ws, out=out)
    other_ws = fresh_ws(T, K, E)
    for rep in range(4):
        scores = np.random.default_rng(60 + rep).standard_normal((T, E)).astype(np.float32)
        s.copy_(torch.from_numpy(scores))
        _log(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        check(out, expected(scores, K, False, True), ("replay", rep))
        header_ok(ws, T * K)
        # eager work between replays, on another workspace
        other, _ = run(np.random.default_rng(70 + rep).standard_normal((T // 2, E)).astype(np.float32), K,
                       mode=FUSED, ws=other_ws)
    del g


@pytest.mark.parametrize("T,E,K", [(1, 3, 2), (40, 16, 8), (300, 256, 8), (2049, 64, 16)])
def test_route_fewer_finite_scores_than_k(T, E, K):
    """Rows with fewer scores above -inf than K: once only -inf is left, every round picks expert 0 again, so a
    token's ids repeat; the fused form ranks the repeats by lane as the map does."""
    rng = np.random.default_rng(T + E + K)
    scores = np.full((T, E), -np.inf, np.float32)
    finite = rng.integers(0, K, T)  # 0 .. K-1 finite scores per row
    for t in range(T):
        cols = rng.choice(E, size=finite[t], replace=False)
        scores[t, cols] = rng.standard_normal(finite[t]).astype(np.float32)
    scores[rng.random((T, E)) < 0.01] = np.nan  # NaN ranks as -inf
    _log(f"fewer finite than K: T={T} E={E} K={K}")
    exp = expected(scores, K, False, True)
    assert (exp["topk_idx"] == 0).sum(axis=1).max() > 1  # repeats do occur
    res, ws = run(scores, K, with_weights=True, mode=FUSED)
    check(res, exp, (T, E, K))
    header_ok(ws, T * K)


@pytest.mark.parametrize("T", [1, 3, 4, 5, 16, 17, 31, 32])
@pytest.mark.parametrize("E,K", [(3, 2), (64, 6), (256, 8), (1024, 16)])
def test_local_form_matches_oracle(T, E, K):
    """The local form (one launch, every workgroup routing the whole batch: four-wave workgroups up to 4 tokens,
    sixteen-wave ones above, two tokens per wave above 16) against the oracle, with ties, NaN and -inf rows among
    normal scores, renormalised weights, raw weights and none; AUTO (the local form up to 16 tokens, the split
    form above) gives the same results."""
    rng = np.random.default_rng(T * 131 + E)
    s = rng.standard_normal((T, E)).astype(np.float32)
    s[0, ::2] = np.nan
    if T > 2:
        s[1, 1:] = -np.inf  # fewer finite scores than K: index 0 repeats
        s[2] = np.float32(0.5)  # all tied
    pos_scores = np.abs(s) + np.float32(0.01)  # renormalisation needs positive scores
    pos_scores[np.isnan(pos_scores)] = np.float32(0.5)
    _log(f"local T={T} E={E} K={K}")
    for mode in (LOCAL, AUTO):
        res, ws = run(pos_scores, K, renormalize=True, with_weights=True, mode=mode)
        check(res, expected(pos_scores, K, True, True), ("local renorm", mode))
        assert not h(ws[:2048].view(torch.int32)).any()  # the header is not touched
    res, _ = run(s, K, with_weights=True, mode=LOCAL)
    check(res, expected(s, K, False, True), "local raw weights")
    sd = torch.from_numpy(s).cuda()
    r = moe.moe_route(sd, K, with_weights=False, with_row_token=False, mode=LOCAL, workspace=fresh_ws(T, K, E))
    torch.cuda.synchronize()
    exp = expected(s, K, False, False)
    exp["row_token"] = None
    check(r, exp, "local no weights")


def test_local_form_refuses_more_than_32_tokens():
    s = torch.zeros((33, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_route(s, 2, mode=LOCAL, workspace=fresh_ws(33, 2, 16))
