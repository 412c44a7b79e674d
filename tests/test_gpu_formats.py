"""GPU parity of the block-scaled output formats (moe_expand_cast,
swiglu_cast) against the oracle: e4m3 and FP4 e2m1 codes, groups of 16, 32
and 128 channels, fp32 / power-of-two / UE8M0 scales, default and custom
clamps.  The expand is bit-exact (identity cast on a flat grid and routed
expand on the split-copy kernel, K from 1 to 8, with weights); the SwiGLU
path is within the stated tolerance (scales 1e-6 relative, or a factor 2
at a binade edge with power-of-two scales; dequantised values within one
step of the format).  DeepSeek-V3-shaped inputs (hidden 7168, 1% outliers
x50) and the SwiGLU workload's rows (I = 2048, U(0,1) weights); MXFP8 and
MXFP4 (groups of 32, UE8M0) on the full 4096-token layer and on the large
skewed batch the benchmark times."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W
from oracle.compare import fmt_tolerance_report

pytestmark = pytest.mark.gpu

E4M3, E2M1 = oracle.FMT_E4M3, oracle.FMT_E2M1
FORMATS = [(dt, g, rs, u8) for dt in (E4M3, E2M1) for g in (16, 32, 128)
           for rs, u8 in ((False, False), (True, False), (True, True))]
MXFP8 = (E4M3, 32, True, True)
MXFP4 = (E2M1, 32, True, True)
_CACHE = {}


def _log(msg):
    sys.__stderr__.write(f"[gpu-formats] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def fid(f):
    return f"{'e2m1' if f[0] else 'e4m3'}-g{f[1]}{'-pow2' if f[2] else ''}{'-ue8m0' if f[3] else ''}"


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def d(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype)).cuda()


def dsv3(T):
    if ("dsv3", T) not in _CACHE:
        w = W.WORKLOADS["dsv3"]
        x = W.make_x(w, T)
        idx, wt = oracle.topk_gate(W.make_scores(w, T), w.num_topk, renormalize=True)
        _, _, pos, _ = oracle.token_map(idx, w.num_experts)
        _CACHE[("dsv3", T)] = (x, pos, wt)
    return _CACHE[("dsv3", T)]


def kw(f, clamp_min=0.0):
    return dict(dtype=f[0], group_size=f[1], round_sf=f[2], sf_ue8m0=f[3], clamp_min=clamp_min)


def check_expand(x, pos, wt, f, clamp_min=0.0):
    T, H = x.shape
    _log(f"expand {fid(f)} T={T} H={H} K={1 if pos is None else pos.shape[1]} clamp={clamp_min}")
    q, sf, ow = moe.moe_expand_cast(d_bf16(x), None if pos is None else d(pos, np.int32),
                                    None if wt is None else d(wt, np.float32), **kw(f, clamp_min))
    torch.cuda.synchronize()
    eq, esf, eow = oracle.expand_cast(x, pos, wt, **kw(f, clamp_min))
    gsf = sf.cpu().numpy()
    assert np.array_equal(gsf.view(np.uint8) if f[3] else gsf.view(np.uint32),
                          esf.view(np.uint8) if f[3] else esf.view(np.uint32)), "scales"
    assert np.array_equal(q.cpu().numpy(), eq), "codes"
    if wt is not None:
        assert np.array_equal(ow.cpu().numpy().view(np.uint32), eow.view(np.uint32)), "weights"


@pytest.mark.parametrize("f", FORMATS, ids=fid)
def test_identity_cast(f):
    x, _, _ = dsv3(256)
    check_expand(x, None, None, f)


@pytest.mark.parametrize("f", FORMATS, ids=fid)
def test_routed_expand(f):
    x, pos, wt = dsv3(512)
    check_expand(x, pos, wt, f)


@pytest.mark.parametrize("f", [MXFP8, MXFP4], ids=fid)
def test_mx_formats_full_layer(f):
    x, pos, wt = dsv3(4096)
    check_expand(x, pos, wt, f)


@pytest.mark.parametrize("f", [MXFP8, MXFP4], ids=fid)
def test_mx_formats_large_workload(f):
    """The large skewed batch the benchmark times (32768 tokens, top-8, 262144 rows)."""
    if "large" not in _CACHE:
        w = W.WORKLOADS["large"]
        idx, _ = oracle.topk_gate(W.make_scores(w), w.num_topk)
        _, _, pos, _ = oracle.token_map(idx, w.num_experts)
        _CACHE["large"] = (W.make_x(w), pos)
    x, pos = _CACHE["large"]
    check_expand(x, pos, None, f)


@pytest.mark.parametrize("K", [1, 2, 3, 5])
def test_routed_small_topk_and_hidden(K):
    rng = np.random.default_rng(K)
    T, E = 301, 16
    for H in (128, 1024 + 128, 4096):
        idx, wt = oracle.topk_gate(rng.standard_normal((T, E)).astype(np.float32), K, with_weights=True)
        _, _, pos, _ = oracle.token_map(idx, E)
        x = W.f32_to_bf16_bits((rng.standard_normal((T, H)) * 2.0 ** rng.integers(-20, 20, (T, 1))).astype(np.float32))
        for f in (MXFP4, (E4M3, 16, False, False), (E2M1, 128, True, False)):
            check_expand(x, pos, wt, f)


@pytest.mark.parametrize("group", [16, 32, 128])
def test_e2m1_every_bf16_value(group):
    """Every bf16 value with |x| <= 6 through the e2m1 identity cast with a
    scale of exactly 1 (each group also holds 6.0): the hardware conversion
    against the oracle's round-to-nearest-even."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = bits[np.isfinite(vals) & (np.abs(vals) <= 6)].astype(np.uint16)
    per, H = group - 1, 4096
    n_groups = -(-keep.size // per)
    n_groups = -(-n_groups // (H // group)) * (H // group)  # whole rows
    body = np.resize(keep, n_groups * per).reshape(n_groups, per)  # repeats cyclically to fill
    six = np.full((n_groups, 1), 0x40C0, np.uint16)  # bf16 6.0
    x = np.concatenate([six, body], axis=1).reshape(-1, H)
    for f in ((E2M1, group, False, False), (E2M1, group, True, True)):
        check_expand(x, None, None, f)


def test_custom_clamp_and_zero_rows():
    rng = np.random.default_rng(5)
    x = W.f32_to_bf16_bits((rng.standard_normal((40, 512)) * 1e-3).astype(np.float32))
    x[::3] = 0  # whole rows of zeros: the clamp sets the scale
    x[1::3] = 0x8000  # negative zeros
    for f in (MXFP8, MXFP4, (E2M1, 16, False, False), (E4M3, 128, False, False)):
        check_expand(x, None, None, f)
        check_expand(x, None, None, f, clamp_min=0.5)


def check_swiglu(gu, rw, clamp, f):
    R, two_i = gu.shape
    _log(f"swiglu {fid(f)} R={R} I={two_i // 2} weights={rw is not None} clamp={clamp}")
    q, sf = moe.swiglu_cast(d_bf16(gu), None if rw is None else d(rw, np.float32), clamp, **kw(f))
    torch.cuda.synchronize()
    eq, esf = oracle.swiglu_cast(gu, rw, clamp, **kw(f))
    ok, det = fmt_tolerance_report(q.cpu().numpy(), sf.cpu().numpy(), eq, esf, f[0], f[1], f[3], f[2])
    assert ok, det


@pytest.mark.parametrize("f", FORMATS, ids=fid)
def test_swiglu_formats(f):
    w = W.WORKLOADS["swiglu"]
    if "gu" not in _CACHE:
        _CACHE["gu"] = (W.make_gate_up(w)[:1024], W.make_row_weights(w)[:1024])
    gu, rw = _CACHE["gu"]
    check_swiglu(gu, rw, 0.0, f)


@pytest.mark.parametrize("f", [MXFP8, MXFP4], ids=fid)
def test_swiglu_mx_full_workload_and_clamp(f):
    w = W.WORKLOADS["swiglu"]
    gu, rw = W.make_gate_up(w), W.make_row_weights(w)
    check_swiglu(gu, rw, 0.0, f)
    check_swiglu(gu[:512], None, 1.5, f)


def test_zero_sizes():
    _log("formats: zero rows")
    q, sf, _ = moe.moe_expand_cast(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), dtype="e2m1",
                                   group_size=32, round_sf=True, sf_ue8m0=True)
    q2, sf2 = moe.swiglu_cast(torch.empty((0, 512), dtype=torch.bfloat16, device="cuda"), dtype="e2m1",
                              group_size=32)
    torch.cuda.synchronize()
    assert q.shape == (0, 128) and sf.shape == (0, 8) and q2.shape == (0, 128) and sf2.shape == (0, 8)
