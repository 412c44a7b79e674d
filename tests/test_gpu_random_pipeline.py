"""Randomised end-to-end parity: seeded random shapes through the whole path
and its next rows on the GPU (through the C ABI), each step against the
oracle on the same inputs.

Per configuration (T, E, K, H, I drawn at random, sizes ragged against
every tile: any E from 1 to 1024, K up to min(E, 16), H any multiple of 128,
scores with ties, renormalised or plain weights):
  top-k -> token map -> expand + e4m3 cast          bit-exact
  aligned, expert-local map -> padded expand         bit-exact
  expand in a random block-scaled format             bit-exact
  SwiGLU + cast in a random format                   within the stated tolerance
  combine of random expert rows                      bit-exact
"""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W
from oracle.compare import fmt_tolerance_report

pytestmark = pytest.mark.gpu

SEEDS = list(range(40))


def _log(msg):
    sys.__stderr__.write(f"[gpu-random] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def d(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype)).cuda()


def d_bf16(bits):
    return d(np.asarray(bits, np.uint16).view(np.int16), np.int16).view(torch.bfloat16)


def h(t):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), np.asarray(b, np.float32).view(np.uint32)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a.shape == b.shape and np.array_equal(a, b)


def _config(seed):
    rng = np.random.default_rng([seed, 77])
    E = int(rng.choice([1, 2, 7, 16, 63, 64, 100, 256, 257, 600, 1024]))
    K = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.choice([1, 2, 5, 63, 64, 65, 257, 500]))
    H = 128 * int(rng.integers(1, 17))
    I = 128 * int(rng.integers(1, 9))
    renorm = bool(rng.integers(0, 2))
    return rng, T, E, K, H, I, renorm


@pytest.mark.parametrize("seed", SEEDS)
def test_random_pipeline(seed):
    rng, T, E, K, H, I, renorm = _config(seed)
    _log(f"seed={seed} T={T} E={E} K={K} H={H} I={I} renorm={renorm}")
    scores = rng.standard_normal((T, E)).astype(np.float32)
    scores[rng.random((T, E)) < 0.2] = np.float32(0.5)  # ties
    x = W.f32_to_bf16_bits((rng.standard_normal((T, H)) * 2.0 ** rng.integers(-8, 8, (T, 1))).astype(np.float32))

    # top-k -> map -> expand (weights out whenever they are computed)
    idx_g, w_g = moe.moe_topk_gate(d(scores, np.float32), K, renormalize=renorm, with_weights=True)
    idx_o, w_o = oracle.topk_gate(scores, K, renormalize=renorm, with_weights=True)
    torch.cuda.synchronize()
    assert same(h(idx_g), idx_o) and same(h(w_g), w_o), "top-k"
    counts, offsets, pos_g, rt = moe.moe_token_map(idx_g, E)
    oc, oo, op, ort = oracle.token_map(idx_o, E)
    torch.cuda.synchronize()
    for name, a, b in (("counts", counts, oc), ("offsets", offsets, oo), ("pos", pos_g, op), ("row_token", rt, ort)):
        assert same(h(a), b), name
    q, sf, ow = moe.moe_expand_cast_fp8(d_bf16(x), pos_g, w_g)
    eq, esf, eow = oracle.expand_cast_fp8(x, op, w_o)
    torch.cuda.synchronize()
    assert same(h(q), eq) and same(h(sf), esf) and same(h(ow), eow), "expand"

    # expert-local padded map and expand
    b = int(rng.integers(0, E))
    e = int(rng.integers(b + 1, E + 1))
    align = int(rng.choice([1, 3, 16, 128]))
    ac, ao, ap, art = moe.moe_token_map_aligned(idx_g, b, e, align)
    xc, xo, xp, xrt = oracle.token_map_aligned(idx_o, b, e, align)
    torch.cuda.synchronize()
    for name, a1, b1 in (("counts", ac, xc), ("offsets", ao, xo), ("pos", ap, xp), ("row_token", art, xrt)):
        assert same(h(a1), b1), f"aligned {name}"
    pq, psf, pw = moe.moe_expand_cast_fp8_padded(d_bf16(x), ap, art, w_g)
    eq2, esf2, ew2 = oracle.expand_cast_fp8_padded(x, xp, xrt, w_o)
    torch.cuda.synchronize()
    assert same(h(pq), eq2) and same(h(psf), esf2) and same(h(pw), ew2), "padded expand"

    # a random block-scaled format
    dt = int(rng.integers(0, 2))
    group = int(rng.choice([16, 32, 128]))
    rs = bool(rng.integers(0, 2))
    u8 = rs and bool(rng.integers(0, 2))
    fmt = dict(dtype=dt, group_size=group, round_sf=rs, sf_ue8m0=u8)
    mq, msf, mw = moe.moe_expand_cast(d_bf16(x), pos_g, w_g, **fmt)
    oq3, osf3, ow3 = oracle.expand_cast(x, op, w_o, **fmt)
    torch.cuda.synchronize()
    assert same(h(mq), oq3) and same(h(msf), osf3) and same(h(mw), ow3), f"format expand {fmt}"

    # SwiGLU over the routed rows in that format
    R = T * K
    gu = W.f32_to_bf16_bits((rng.standard_normal((R, 2 * I)) * 3).astype(np.float32))
    rw = rng.random(R, dtype=np.float32)
    sq, ssf = moe.swiglu_cast(d_bf16(gu), d(rw, np.float32), **fmt)
    oq4, osf4 = oracle.swiglu_cast(gu, rw, **fmt)
    torch.cuda.synchronize()
    ok, det = fmt_tolerance_report(h(sq), h(ssf), oq4, osf4, dt, group, u8, rs)
    assert ok, det

    # combine of random expert rows back to token order
    y = W.f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    cg = moe.moe_combine(d_bf16(y), pos_g, w_g)
    co = oracle.combine(y, op, w_o)
    torch.cuda.synchronize()
    assert same(h(cg), co), "combine"
