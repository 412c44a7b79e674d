"""Guard regions around every output of every entry point: each output is a
view into a larger buffer whose leading and trailing guard elements hold a
fill pattern; after the call (on a side stream) the guards must be
untouched and the view must hold the oracle's result (bit for bit, or the
SwiGLU tolerance).  Sizes are ragged: token counts, expert counts, hidden
sizes and row counts that are not multiples of the workgroup, chunk or tile
sizes, so tail handling writes next to the guards."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W
from oracle.compare import fmt_tolerance_report, swiglu_tolerance_report

pytestmark = pytest.mark.gpu

PAD = 4099  # elements of guard on each side (odd: no alignment luck)


def _log(msg):
    sys.__stderr__.write(f"[gpu-guards] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


class Guarded:
    """A contiguous output of `shape` inside a buffer with PAD guard elements
    on each side (views start 16-byte aligned where the kernels require it)."""

    def __init__(self, shape, dtype, fill):
        n = int(np.prod(shape)) if len(shape) else 1
        esz = torch.empty((), dtype=dtype).element_size()
        lead = (PAD * esz + 15) // 16 * 16 // esz  # >= PAD elements, 16-byte aligned start
        self.lead, self.n, self.fill = lead, n, fill
        self.buf = torch.full((lead + n + PAD,), fill, dtype=dtype, device="cuda")
        self.view = self.buf[lead:lead + n].view(shape)

    def check(self, name):
        b = self.buf.cpu()
        head, tail = b[:self.lead], b[self.lead + self.n:]
        assert bool((head == self.fill).all()), f"{name}: write before the output"
        assert bool((tail == self.fill).all()), f"{name}: write after the output"
        return self.view.cpu().numpy()


def _bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def _run(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = fn(side)
    side.synchronize()
    return out


def _routing(T, E, K, seed, renormalize=False):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((T, E)).astype(np.float32)
    if renormalize:
        s = (1.0 / (1.0 + np.exp(-s.astype(np.float64)))).astype(np.float32)
    return s, rng


@pytest.mark.parametrize("T,E,K,renorm", [(333, 200, 6, True), (333, 100, 3, False), (1001, 256, 8, True),
                                          (77, 1000, 16, False)])
def test_topk_guards(T, E, K, renorm):
    _log(f"topk T={T} E={E} K={K}")
    s, _ = _routing(T, E, K, 1, renorm)
    gi = Guarded((T, K), torch.int64, -77)
    gw = Guarded((T, K), torch.float32, -7.0)
    sd = torch.from_numpy(s).cuda()
    _run(lambda st: moe.moe_topk_gate(sd, K, renormalize=renorm, with_weights=True, out=(gi.view, gw.view),
                                      stream=st))
    ei, ew = oracle.topk_gate(s, K, renormalize=renorm, with_weights=True)
    assert np.array_equal(gi.check("topk_idx"), ei)
    assert np.array_equal(gw.check("topk_weights").view(np.uint32), ew.view(np.uint32))


@pytest.mark.parametrize("T,E,K", [(333, 200, 6), (3001, 256, 8), (9001, 256, 8), (1500, 1000, 5)])
def test_token_map_guards(T, E, K):
    _log(f"token map T={T} E={E} K={K}")
    s, _ = _routing(T, E, K, 2)
    idx, _ = oracle.topk_gate(s, K)
    gc = Guarded((E,), torch.int32, -9)
    go = Guarded((E + 1,), torch.int32, -9)
    gp = Guarded((T, K), torch.int32, -9)
    gr = Guarded((T * K,), torch.int32, -9)
    idd = torch.from_numpy(idx).cuda()
    _run(lambda st: moe.moe_token_map(idd, E, out=(gc.view, go.view, gp.view, gr.view), stream=st))
    ec, eo, ep, er = oracle.token_map(idx, E)
    assert np.array_equal(gc.check("counts"), ec) and np.array_equal(go.check("offsets"), eo)
    assert np.array_equal(gp.check("pos"), ep) and np.array_equal(gr.check("row_token"), er)


def test_swiglu_guards():
    R, I = 333, 384
    _log(f"swiglu R={R} I={I}")
    rng = np.random.default_rng(3)
    gu = W.f32_to_bf16_bits(rng.standard_normal((R, 2 * I)).astype(np.float32))
    rw = rng.random(R, dtype=np.float32)
    gq = Guarded((R, I), torch.uint8, 0x5A)
    gs = Guarded((R, I // 128), torch.float32, -7.0)
    gud, rwd = _bf16(gu), torch.from_numpy(rw).cuda()
    _run(lambda st: moe.swiglu_cast_fp8(gud, rwd, out=(gq.view, gs.view), stream=st))
    eq, esf = oracle.swiglu_cast_fp8(gu, rw)
    ok, det = swiglu_tolerance_report(gq.check("codes"), gs.check("scales"), eq, esf)
    assert ok, det


@pytest.mark.parametrize("H", [136, 7168])
def test_combine_guards(H):
    T, E, K = 333, 200, 6
    _log(f"combine T={T} K={K} H={H}")
    s, rng = _routing(T, E, K, 4, True)
    idx, wt = oracle.topk_gate(s, K, renormalize=True)
    _, _, pos, _ = oracle.token_map(idx, E)
    y = W.f32_to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32))
    go = Guarded((T, H), torch.int16, 0x1234)
    yd, pd, wd = _bf16(y), torch.from_numpy(pos).cuda(), torch.from_numpy(wt).cuda()
    _run(lambda st: moe.moe_combine(yd, pd, wd, out=go.view.view(torch.bfloat16), stream=st))
    assert np.array_equal(go.check("out").view(np.uint16), oracle.combine(y, pos, wt))


def test_aligned_map_and_padded_expand_guards():
    T, E, K, H, begin, end, align = 333, 200, 6, 384, 10, 150, 16
    _log(f"aligned map + padded expand T={T} [{begin},{end}) align={align}")
    s, rng = _routing(T, E, K, 5, True)
    idx, wt = oracle.topk_gate(s, K, renormalize=True)
    EL = end - begin
    rows = oracle.padded_rows_bound(T, K, EL, align) + 5
    gc = Guarded((EL,), torch.int32, -9)
    go = Guarded((EL + 1,), torch.int32, -9)
    gp = Guarded((T, K), torch.int32, -9)
    gr = Guarded((rows,), torch.int32, -9)
    idd = torch.from_numpy(idx).cuda()
    _run(lambda st: moe.moe_token_map_aligned(idd, begin, end, align, out=(gc.view, go.view, gp.view, gr.view),
                                              stream=st))
    ec, eo, ep, er = oracle.token_map_aligned(idx, begin, end, align, num_rows=rows)
    assert np.array_equal(gc.check("counts"), ec) and np.array_equal(go.check("offsets"), eo)
    assert np.array_equal(gp.check("pos"), ep) and np.array_equal(gr.check("row_token"), er)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gq = Guarded((rows, H), torch.uint8, 0x5A)
    gs = Guarded((rows, H // 128), torch.float32, -7.0)
    gw = Guarded((rows,), torch.float32, -7.0)
    xd, wd = _bf16(x), torch.from_numpy(wt).cuda()
    _run(lambda st: moe.moe_expand_cast_fp8_padded(xd, gp.view, gr.view, wd, out=(gq.view, gs.view, gw.view),
                                                   stream=st))
    eq, esf, ew = oracle.expand_cast_fp8_padded(x, ep, er, wt)
    assert np.array_equal(gq.check("codes"), eq)
    assert np.array_equal(gs.check("scales").view(np.uint32), esf.view(np.uint32))
    assert np.array_equal(gw.check("weights").view(np.uint32), ew.view(np.uint32))


@pytest.mark.parametrize("dtype,group,round_sf,ue8m0", [("e2m1", 32, True, True), ("e4m3", 16, False, False),
                                                        ("e2m1", 128, False, False)])
def test_block_scaled_guards(dtype, group, round_sf, ue8m0):
    T, E, K, H = 333, 200, 6, 1024
    _log(f"block-scaled {dtype}/{group} round_sf={round_sf} ue8m0={ue8m0}")
    s, rng = _routing(T, E, K, 6, True)
    idx, wt = oracle.topk_gate(s, K, renormalize=True)
    _, _, pos, _ = oracle.token_map(idx, E)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    fmt = oracle.FMT_E2M1 if dtype == "e2m1" else oracle.FMT_E4M3
    width = H // 2 if dtype == "e2m1" else H
    sdt = torch.uint8 if ue8m0 else torch.float32
    sfill = 0xEE if ue8m0 else -7.0
    R = T * K
    gq = Guarded((R, width), torch.uint8, 0x5A)
    gs = Guarded((R, H // group), sdt, sfill)
    gw = Guarded((R,), torch.float32, -7.0)
    xd, pd, wd = _bf16(x), torch.from_numpy(pos).cuda(), torch.from_numpy(wt).cuda()
    qv = gq.view.view(torch.float8_e4m3fn) if dtype == "e4m3" else gq.view
    _run(lambda st: moe.moe_expand_cast(xd, pd, wd, dtype=dtype, group_size=group, round_sf=round_sf,
                                        sf_ue8m0=ue8m0, out=(qv, gs.view, gw.view), stream=st))
    eq, esf, ew = oracle.expand_cast(x, pos, wt, dtype=fmt, group_size=group, round_sf=round_sf, sf_ue8m0=ue8m0)
    assert np.array_equal(gq.check("codes"), eq)
    assert np.array_equal(gs.check("scales").view(np.uint8), esf.view(np.uint8))
    assert np.array_equal(gw.check("weights").view(np.uint32), ew.view(np.uint32))
    # SwiGLU in the same format
    RS, I = 333, 1024
    gu = W.f32_to_bf16_bits(rng.standard_normal((RS, 2 * I)).astype(np.float32))
    iw = I // 2 if dtype == "e2m1" else I
    gq2 = Guarded((RS, iw), torch.uint8, 0x5A)
    gs2 = Guarded((RS, I // group), sdt, sfill)
    gud = _bf16(gu)
    qv2 = gq2.view.view(torch.float8_e4m3fn) if dtype == "e4m3" else gq2.view
    _run(lambda st: moe.swiglu_cast(gud, None, dtype=dtype, group_size=group, round_sf=round_sf, sf_ue8m0=ue8m0,
                                    out=(qv2, gs2.view), stream=st))
    eq2, esf2 = oracle.swiglu_cast(gu, None, dtype=fmt, group_size=group, round_sf=round_sf, sf_ue8m0=ue8m0)
    ok, det = fmt_tolerance_report(gq2.check("swiglu codes"), gs2.check("swiglu scales"), eq2, esf2, fmt, group,
                                   ue8m0, round_sf)
    assert ok, det


# the single launch: local routing in four-wave workgroups (3 tokens), in sixteen-wave ones (5, and 20 with two
# tokens per wave), the grid barrier (40); the top-k-then-copy form; the routed forms
@pytest.mark.parametrize("T,mode", [(3, moe.MOE_DISPATCH_SINGLE_LAUNCH), (5, moe.MOE_DISPATCH_SINGLE_LAUNCH),
                                    (20, moe.MOE_DISPATCH_SINGLE_LAUNCH), (40, moe.MOE_DISPATCH_SINGLE_LAUNCH),
                                    (40, moe.MOE_DISPATCH_TOPK_THEN_COPY), (77, moe.MOE_DISPATCH_SPLIT),
                                    (77, moe.MOE_DISPATCH_ROUTE_FUSED)])
def test_dispatch_guards(T, mode):
    w = W.WORKLOADS["dsv3"]
    E, K, H = w.num_experts, w.num_topk, w.hidden
    _log(f"dispatch T={T} mode={mode}")
    s = W.make_scores(w, num_tokens=T)
    x = W.make_x(w, num_tokens=T)
    R, G = T * K, H // 128
    g = {"topk_idx": Guarded((T, K), torch.int64, -77), "topk_weights": Guarded((T, K), torch.float32, -7.0),
         "counts": Guarded((E,), torch.int32, -9), "offsets": Guarded((E + 1,), torch.int32, -9),
         "pos": Guarded((T, K), torch.int32, -9), "row_token": Guarded((R,), torch.int32, -9),
         "out": Guarded((R, H), torch.uint8, 0x5A), "out_sf": Guarded((R, G), torch.float32, -7.0),
         "out_weights": Guarded((R,), torch.float32, -7.0)}
    sd, xd = torch.from_numpy(s).cuda(), _bf16(x)
    out = {k: v.view for k, v in g.items()}
    _run(lambda st: moe.moe_dispatch(sd, xd, K, renormalize=True, mode=mode, out=out, stream=st))
    ei, ew = oracle.topk_gate(s, K, renormalize=True)
    ec, eo, ep, er = oracle.token_map(ei, E)
    eq, esf, eow = oracle.expand_cast_fp8(x, ep, ew)
    want = {"topk_idx": ei, "topk_weights": ew.view(np.uint32), "counts": ec, "offsets": eo, "pos": ep,
            "row_token": er, "out": eq, "out_sf": esf.view(np.uint32), "out_weights": eow.view(np.uint32)}
    for k, v in g.items():
        got = v.check(k)
        if got.dtype == np.float32:
            got = got.view(np.uint32)
        assert np.array_equal(got, want[k]), k


@pytest.mark.parametrize("T,mode", [(3, moe.MOE_ROUTE_LOCAL), (20, moe.MOE_ROUTE_LOCAL), (77, moe.MOE_ROUTE_FUSED)])
def test_route_guards(T, mode):
    w = W.WORKLOADS["dsv3"]
    E, K = w.num_experts, w.num_topk
    _log(f"route T={T} mode={mode}")
    s = W.make_scores(w, num_tokens=T)
    R = T * K
    g = {"topk_idx": Guarded((T, K), torch.int64, -77), "topk_weights": Guarded((T, K), torch.float32, -7.0),
         "counts": Guarded((E,), torch.int32, -9), "offsets": Guarded((E + 1,), torch.int32, -9),
         "pos": Guarded((T, K), torch.int32, -9), "row_token": Guarded((R,), torch.int32, -9)}
    sd = torch.from_numpy(s).cuda()
    out = {k: v.view for k, v in g.items()}
    _run(lambda st: moe.moe_route(sd, K, renormalize=True, mode=mode, out=out, stream=st))
    ei, ew = oracle.topk_gate(s, K, renormalize=True)
    ec, eo, ep, er = oracle.token_map(ei, E)
    want = {"topk_idx": ei, "topk_weights": ew.view(np.uint32), "counts": ec, "offsets": eo, "pos": ep,
            "row_token": er}
    for k, v in g.items():
        got = v.check(k)
        if got.dtype == np.float32:
            got = got.view(np.uint32)
        assert np.array_equal(got, want[k]), k
