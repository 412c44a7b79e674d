"""Calls on independent buffers run concurrently on different streams (the
C ABI's stream-ordering contract): the split path (top-k, map, expand,
SwiGLU) issued on two streams with interleaved launches, and two
single-launch decode dispatches at once (each grid a few workgroups, so both
are resident together), each checked against the oracle bit for bit (SwiGLU
within its tolerance)."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W
from oracle.compare import swiglu_tolerance_report

pytestmark = pytest.mark.gpu


def _log(msg):
    sys.__stderr__.write(f"[gpu-streams] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _inputs(seed, T, E, H, R, I):
    rng = np.random.default_rng(seed)
    s = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, E))))).astype(np.float32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gu = W.f32_to_bf16_bits(rng.standard_normal((R, 2 * I)).astype(np.float32))
    rw = rng.random(R, dtype=np.float32)
    return s, x, gu, rw


def _dev(a, bf16=False):
    t = torch.from_numpy(a.view(np.int16) if bf16 else a).cuda()
    return t.view(torch.bfloat16) if bf16 else t


def test_split_path_on_two_streams():
    T, E, K, H, I = 1500, 256, 8, 2048, 512
    R = T * K
    cases = [_inputs(seed, T, E, H, R, I) for seed in (21, 22)]
    dev_in = [(_dev(s), _dev(x, True), _dev(gu, True), _dev(rw)) for s, x, gu, rw in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = [{} for _ in streams]
    _log(f"split path on two streams T={T} H={H}")
    # interleave the launches of the two pipelines
    for j, (st, (s, x, gu, rw)) in enumerate(zip(streams, dev_in)):
        with torch.cuda.stream(st):
            outs[j]["idx"], outs[j]["w"] = moe.moe_topk_gate(s, K, renormalize=True, stream=st)
    for j, st in enumerate(streams):
        with torch.cuda.stream(st):
            outs[j]["map"] = moe.moe_token_map(outs[j]["idx"], E, stream=st)
    for j, (st, (s, x, gu, rw)) in enumerate(zip(streams, dev_in)):
        with torch.cuda.stream(st):
            outs[j]["exp"] = moe.moe_expand_cast_fp8(x, outs[j]["map"][2], outs[j]["w"], stream=st)
            outs[j]["sw"] = moe.swiglu_cast_fp8(gu, rw, stream=st)
    for st in streams:
        st.synchronize()
    for j, (s, x, gu, rw) in enumerate(cases):
        ei, ew = oracle.topk_gate(s, K, renormalize=True)
        ec, eo, ep, er = oracle.token_map(ei, E)
        eq, esf, eow = oracle.expand_cast_fp8(x, ep, ew)
        o = outs[j]
        assert np.array_equal(o["idx"].cpu().numpy(), ei)
        assert np.array_equal(o["w"].cpu().numpy().view(np.uint32), ew.view(np.uint32))
        for got, want in zip(o["map"], (ec, eo, ep, er)):
            assert np.array_equal(got.cpu().numpy(), want)
        assert np.array_equal(o["exp"][0].view(torch.uint8).cpu().numpy(), eq)
        assert np.array_equal(o["exp"][1].cpu().numpy().view(np.uint32), esf.view(np.uint32))
        assert np.array_equal(o["exp"][2].cpu().numpy().view(np.uint32), eow.view(np.uint32))
        sq, ssf = oracle.swiglu_cast_fp8(gu, rw)
        ok, det = swiglu_tolerance_report(o["sw"][0].view(torch.uint8).cpu().numpy(), o["sw"][1].cpu().numpy(),
                                          sq, ssf)
        assert ok, det


def test_single_launch_dispatches_on_two_streams():
    w = W.WORKLOADS["dsv3"]
    E, K, H = w.num_experts, w.num_topk, w.hidden
    T = 4  # 4 tokens x 7 chunks: a few workgroups per grid, both grids resident together
    _log(f"two single-launch dispatches at once T={T}")
    s_all = W.make_scores(w, num_tokens=2 * T)
    x_all = W.make_x(w, num_tokens=2 * T)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = []
    for j, st in enumerate(streams):
        s, x = s_all[j * T:(j + 1) * T], x_all[j * T:(j + 1) * T]
        with torch.cuda.stream(st):
            outs.append(moe.moe_dispatch(_dev(np.ascontiguousarray(s)), _dev(np.ascontiguousarray(x), True), K,
                                         renormalize=True, mode=moe.MOE_DISPATCH_SINGLE_LAUNCH, stream=st))
    for st in streams:
        st.synchronize()
    for j, o in enumerate(outs):
        s, x = s_all[j * T:(j + 1) * T], x_all[j * T:(j + 1) * T]
        ei, ew = oracle.topk_gate(s, K, renormalize=True)
        ec, eo, ep, er = oracle.token_map(ei, E)
        eq, esf, _ = oracle.expand_cast_fp8(x, ep, ew)
        assert np.array_equal(o["topk_idx"].cpu().numpy(), ei)
        assert np.array_equal(o["pos"].cpu().numpy(), ep)
        assert np.array_equal(o["out"].view(torch.uint8).cpu().numpy(), eq)
        assert np.array_equal(o["out_sf"].cpu().numpy().view(np.uint32), esf.view(np.uint32))


def test_explicit_side_stream_allocates_on_it():
    """stream=side while the current stream stays the default one: the binding allocates (and zeroes)
    outputs and workspaces on `side`, so nothing orders them against the default stream's work, and the
    results still equal the oracle's bit for bit."""
    w = W.WORKLOADS["dsv3"]
    T, E, K = 512, w.num_experts, w.num_topk
    scores = W.make_scores(w, T)
    x = W.make_x(w, T)
    s_d, x_d = _dev(scores), _dev(x, True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    assert torch.cuda.current_stream() != side
    _log(f"explicit side stream, T={T}")
    # default-stream work in flight meanwhile: a large fill that the side-stream calls must not wait for
    junk = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    junk.fill_(7)
    d = moe.moe_dispatch(s_d, x_d, K, renormalize=True, mode=moe.MOE_DISPATCH_SINGLE_LAUNCH, stream=side)
    idx, wts = moe.moe_topk_gate(s_d, K, renormalize=True, stream=side)
    counts, offsets, pos, row_token = moe.moe_token_map(idx, E, stream=side)
    q, sf, ow = moe.moe_expand_cast_fp8(x_d, pos, wts, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    o_idx, o_w = oracle.topk_gate(scores, K, renormalize=True)
    o_counts, o_offsets, o_pos, o_rt = oracle.token_map(o_idx, E)
    o_q, o_sf, o_ow = oracle.expand_cast_fp8(x, o_pos, o_w)
    for got in ((d["topk_idx"], d["pos"], d["out"], d["out_sf"], d["out_weights"], d["row_token"]),
                (idx, pos, q, sf, ow, row_token)):
        g_idx, g_pos, g_q, g_sf, g_ow, g_rt = (t.cpu().numpy() for t in
                                               (got[0], got[1], got[2].view(torch.uint8), got[3], got[4], got[5]))
        assert np.array_equal(g_idx, o_idx)
        assert np.array_equal(g_pos, o_pos)
        assert np.array_equal(g_rt, o_rt)
        assert np.array_equal(g_q, o_q)
        assert np.array_equal(g_sf.view(np.uint32), o_sf.view(np.uint32))
        assert np.array_equal(g_ow.view(np.uint32), o_ow.view(np.uint32))
    assert np.array_equal(counts.cpu().numpy(), o_counts) and np.array_equal(offsets.cpu().numpy(), o_offsets)
    del junk
