"""Each Python entry point rejects, before any launch, outputs of the wrong
shape, dtype, layout or device and inputs that disagree with each other;
the caller's buffers stay untouched.  No kernel runs on a rejected call."""
import sys

import pytest
import torch

import moe_routing_fp8_amd as moe

pytestmark = pytest.mark.gpu


def _log(msg):
    sys.__stderr__.write(f"[gpu-binding] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _rejects(fn, *guards):
    before = [g.clone() for g in guards]
    with pytest.raises(ValueError):
        fn()
    torch.cuda.synchronize()
    for g, b in zip(guards, before):
        assert torch.equal(g, b)


def test_rejects_bad_outputs_and_inputs():
    T, E, K, H, I = 16, 32, 4, 256, 256
    dev = "cuda"
    _log("binding validation")
    s = torch.randn((T, E), device=dev)
    x = torch.randn((T, H), device=dev).to(torch.bfloat16)
    idx, w = moe.moe_topk_gate(s, K, renormalize=True)
    counts, offsets, pos, rt = moe.moe_token_map(idx, E)
    R = T * K
    q = torch.full((R - 1, H), 7, dtype=torch.uint8, device=dev)  # one row short
    sf = torch.full((R, H // 128), 7.0, device=dev)
    ow = torch.full((R,), 7.0, device=dev)
    _rejects(lambda: moe.moe_expand_cast_fp8(x, pos, w, out=(q, sf, ow)), q, sf, ow)
    q = torch.full((R, H), 7, dtype=torch.uint8, device=dev)
    _rejects(lambda: moe.moe_expand_cast_fp8(x, pos, w, out=(q, sf.to(torch.float16), ow)), q, ow)
    _rejects(lambda: moe.moe_expand_cast_fp8(x, pos, w[:, :2].contiguous(), out=(q, sf, ow)), q, sf, ow)
    _rejects(lambda: moe.moe_expand_cast_fp8(x, pos, w, out=(q, sf, ow.cpu())), q, sf)
    _rejects(lambda: moe.moe_topk_gate(s, K, out=(idx[:, :2].contiguous(), None)), idx)
    short_rt = torch.full((R - 1,), 7, dtype=torch.int32, device=dev)
    _rejects(lambda: moe.moe_token_map(idx, E, out=(counts, offsets, pos, short_rt)), short_rt, counts)
    _rejects(lambda: moe.moe_token_map(idx, E, workspace=torch.empty(64, dtype=torch.int32, device=dev)))
    gu = torch.randn((R, 2 * I), device=dev).to(torch.bfloat16)
    sq = torch.full((R, I), 7, dtype=torch.uint8, device=dev)
    ssf = torch.full((R, I // 128), 7.0, device=dev)
    _rejects(lambda: moe.swiglu_cast_fp8(gu, torch.rand(R - 1, device=dev), out=(sq, ssf)), sq, ssf)
    _rejects(lambda: moe.swiglu_cast_fp8(gu, None, out=(sq[:, :I // 2], ssf)), sq, ssf)
    _rejects(lambda: moe.swiglu_cast(gu, None, dtype="e2m1", group_size=32, out=(sq, ssf)), sq, ssf)
    y = torch.randn((R, H), device=dev).to(torch.bfloat16)
    comb = torch.full((T, H // 2), 7, dtype=torch.bfloat16, device=dev)
    _rejects(lambda: moe.moe_combine(y, pos, w, out=comb), comb)
    _rejects(lambda: moe.moe_combine(y, pos, w[:1].contiguous()))
    bound = moe.moe_token_map_aligned_rows(T, K, E, 16)
    rt_a = torch.full((bound - 1,), 7, dtype=torch.int32, device=dev)
    _rejects(lambda: moe.moe_token_map_aligned(idx, 0, E, 16, num_rows=bound,
                                               out=(counts, offsets, pos, rt_a)), rt_a)
    d = moe.moe_dispatch(s, x, K, renormalize=True)
    d["out_sf"] = d["out_sf"][:-1]
    _rejects(lambda: moe.moe_dispatch(s, x, K, renormalize=True, out=d), d["out"].view(torch.uint8))
    _rejects(lambda: moe.moe_expand_cast_fp8(x, pos, w, out=(q[:-1], sf, ow)), q)


def test_aligned_map_takes_row_count_from_output():
    """With outputs given and no num_rows, the row count is that of row_token."""
    T, E, K = 40, 16, 2
    idx = torch.randint(0, E, (T, K), device="cuda")
    bound = moe.moe_token_map_aligned_rows(T, K, E, 8)
    rt = torch.full((bound + 10,), 7, dtype=torch.int32, device="cuda")
    out = (torch.empty(E, dtype=torch.int32, device="cuda"), torch.empty(E + 1, dtype=torch.int32, device="cuda"),
           torch.empty((T, K), dtype=torch.int32, device="cuda"), rt)
    _log("aligned map, row count from the output")
    moe.moe_token_map_aligned(idx, 0, E, 8, out=out)
    torch.cuda.synchronize()
    offs = out[1].cpu()
    tail = rt[int(offs[-1]):].cpu()
    assert bool((tail == -1).all())  # every row past the segments, up to the output's end, is -1
