"""The dispatch path under HIP graph capture: top-k, token map, expand + cast,
SwiGLU + cast, the single-launch dispatch (its grid barrier included, and its
local-routing form), the top-k-then-copy dispatch, moe_route's local form and
the combine are captured once into one graph and replayed several times, with
new inputs copied into the captured buffers and eager work on other buffers
between the replays.  Every replay must equal the eager result for its
inputs bit for bit (the library records no memset nodes; the barrier
counters carry over from replay to replay)."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import workloads as W

pytestmark = pytest.mark.gpu


def _log(msg):
    sys.__stderr__.write(f"[gpu-graph] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _inputs(seed, T, E, H, R_sw, I):
    rng = np.random.default_rng(seed)
    s = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    x = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)).view(np.int16)).cuda()
    gu = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal((R_sw, 2 * I)).astype(np.float32)).view(np.int16)).cuda()
    y = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal((T * 8, H)).astype(np.float32)).view(np.int16)).cuda()
    return s, x.view(torch.bfloat16), gu.view(torch.bfloat16), y.view(torch.bfloat16)


def _path(s, x, gu, y, K, E, ws_map, ws_disp, out=None):
    """One pass; returns the dict of outputs (written into `out` when given)."""
    o = out if out is not None else {}
    T = s.shape[0]
    o["idx"], o["w"] = moe.moe_topk_gate(s, K, renormalize=True,
                                         out=None if out is None else (out["idx"], out["w"]))
    o["counts"], o["offsets"], o["pos"], o["rt"] = moe.moe_token_map(
        o["idx"], E, workspace=ws_map,
        out=None if out is None else (out["counts"], out["offsets"], out["pos"], out["rt"]))
    o["q"], o["sf"], o["ow"] = moe.moe_expand_cast_fp8(
        x, o["pos"], o["w"], out=None if out is None else (out["q"], out["sf"], out["ow"]))
    o["sq"], o["ssf"] = moe.swiglu_cast_fp8(gu, out=None if out is None else (out["sq"], out["ssf"]))
    o["one"] = moe.moe_dispatch(s, x, K, renormalize=True, mode=moe.MOE_DISPATCH_SINGLE_LAUNCH, workspace=ws_disp,
                                out=None if out is None else out["one"])
    # the forms without a grid barrier: local routing (16 tokens in one launch), the top-k kernel then the map
    # and copies, and moe_route's local form (8 tokens)
    o["local"] = moe.moe_dispatch(s[:16], x[:16], K, renormalize=True, mode=moe.MOE_DISPATCH_SINGLE_LAUNCH,
                                  workspace=ws_disp, out=None if out is None else out["local"])
    o["topk_copy"] = moe.moe_dispatch(s, x, K, renormalize=True, mode=moe.MOE_DISPATCH_TOPK_THEN_COPY,
                                      workspace=ws_disp, out=None if out is None else out["topk_copy"])
    o["route_local"] = moe.moe_route(s[:8], K, renormalize=True, mode=moe.MOE_ROUTE_LOCAL, workspace=ws_disp,
                                     out=None if out is None else out["route_local"])
    o["comb"] = moe.moe_combine(y, o["pos"], o["w"], out=None if out is None else out["comb"])
    return o


def _flat(o):
    res = {}
    for k, v in o.items():
        if isinstance(v, dict):
            for kk, vv in v.items():
                if vv is not None:
                    res[f"{k}.{kk}"] = vv
        elif v is not None:
            res[k] = v
    return {k: (v.view(torch.uint8) if v.dtype == torch.float8_e4m3fn else v).clone() for k, v in res.items()}


def test_graph_replays_match_eager():
    T, E, K, H, R_sw, I = 48, 256, 8, 2048, 256, 512
    ws_map = torch.empty(max(256, moe.moe_token_map_workspace_bytes(T, K, E)), dtype=torch.uint8, device="cuda")
    ws_disp = torch.zeros(moe.moe_dispatch_workspace_bytes(T, K, E), dtype=torch.uint8, device="cuda")
    ws_eager = torch.zeros_like(ws_disp)
    s, x, gu, y = _inputs(0, T, E, H, R_sw, I)
    out = _path(s, x, gu, y, K, E, ws_map, ws_disp)  # allocates the captured outputs
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        _path(s, x, gu, y, K, E, ws_map, ws_disp, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _path(s, x, gu, y, K, E, ws_map, ws_disp, out)
    torch.cuda.synchronize()
    for rep in range(4):
        s2, x2, gu2, y2 = _inputs(100 + rep, T, E, H, R_sw, I)
        s.copy_(s2), x.copy_(x2), gu.copy_(gu2), y.copy_(y2)
        _log(f"replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = _flat(out)
        # eager on separate buffers, interleaved with the replays
        ref = _flat(_path(s2, x2, gu2, y2, K, E, torch.empty_like(ws_map), ws_eager))
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (rep, k)
    words = ws_disp[:12].view(torch.int32).cpu().numpy().view(np.uint32)
    assert words[2] == 0 and words[0] % (1 << 16) == 0, words
