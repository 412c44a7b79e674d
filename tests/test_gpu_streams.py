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
