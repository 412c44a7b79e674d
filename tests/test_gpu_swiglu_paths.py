"""The SwiGLU entry points around their kernel choice ("DeepSeek open-sources
TileKernels", section 3.3): batches of at most 32 rows per compute unit with
I <= 2048 run the latency-oriented row kernel (vector loads first, clamp and
the plain e4m3 format as template flags; past 8 rows per compute unit a row is
split over one-wave workgroups); deeper batches or wider rows run the general
kernel.  Each case runs through the C ABI and is checked against the
oracle within the SwiGLU tolerance (scales 1e-6 relative, values within one
step of the format), with every output prefilled with garbage so an unwritten
element fails."""
import sys

import numpy as np
import pytest
import torch

import moe_routing_fp8_amd as moe
import oracle
import workloads as W
from oracle.compare import fmt_tolerance_report, swiglu_tolerance_report

pytestmark = pytest.mark.gpu


def _log(msg):
    sys.__stderr__.write(f"[gpu-swiglu-paths] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _inputs(rows, inter, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    gu = W.f32_to_bf16_bits((rng.standard_normal((rows, 2 * inter)) * scale).astype(np.float32))
    w = rng.random(rows, dtype=np.float32)
    return gu, w


def _garbage(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xA5)
    return t


def _row_counts():
    b = 32 * _cus()  # the largest batch of the row kernel
    s = 8 * _cus()  # the largest batch that keeps one 256-lane workgroup per row
    return [1, 7, b - 1, b, b + 1, s, s + 1]


# (row-count index into _row_counts(), inter): the row kernel up to the boundary batch at I <= 2048, with one
# 256-lane workgroup per row up to 8 rows per compute unit and one-wave workgroups past it (1, 2 or 4 per row,
# the last one partly or wholly past the row at I = 384, 640 and 1152), the general kernel one row past the
# boundary batch and at I = 2176 (wider than one vector per lane)
CASES = [(0, 128), (1, 2048), (2, 2048), (3, 2048), (4, 2048), (0, 2176), (3, 2176), (1, 128), (3, 1024),
         (5, 2048), (6, 2048), (6, 1024), (6, 640), (6, 1152), (6, 384), (6, 128)]


@pytest.mark.parametrize("rows_i,inter", CASES)
@pytest.mark.parametrize("weighted,clamp", [(True, 0.0), (False, 0.0), (True, 3.5)])
def test_swiglu_cast_fp8_around_the_kernel_choice(rows_i, inter, weighted, clamp):
    rows = _row_counts()[rows_i]
    gu, w = _inputs(rows, inter, 1000 + rows_i + inter, scale=2.0)
    _log(f"e4m3/128 rows={rows} I={inter} weighted={weighted} clamp={clamp}")
    gu_d = torch.from_numpy(gu.view(np.int16)).cuda().view(torch.bfloat16)
    w_d = torch.from_numpy(w).cuda() if weighted else None
    q = _garbage((rows, inter), torch.uint8)
    sf = _garbage((rows, inter // 128), torch.float32)
    moe.swiglu_cast_fp8(gu_d, w_d, clamp_value=clamp, out=(q, sf))
    torch.cuda.synchronize()
    oq, osf = oracle.swiglu_cast_fp8(gu, w if weighted else None, clamp_value=clamp)
    ok, det = swiglu_tolerance_report(q.cpu().numpy(), sf.cpu().numpy(), oq, osf)
    assert ok, det


@pytest.mark.parametrize("fmt", [("e4m3", 32, False, False), ("e4m3", 16, True, True), ("e2m1", 32, True, True),
                                 ("e2m1", 16, False, False)])
@pytest.mark.parametrize("rows_i", [0, 3, 4, 6])
@pytest.mark.parametrize("clamp", [0.0, 2.0])
def test_swiglu_cast_formats_around_the_kernel_choice(fmt, rows_i, clamp):
    dtype, group, round_sf, ue8m0 = fmt
    rows = _row_counts()[rows_i]
    inter = 1024
    gu, w = _inputs(rows, inter, 2000 + rows_i, scale=3.0)
    _log(f"{fmt} rows={rows} clamp={clamp}")
    gu_d = torch.from_numpy(gu.view(np.int16)).cuda().view(torch.bfloat16)
    q, sf = moe.swiglu_cast(gu_d, torch.from_numpy(w).cuda(), clamp_value=clamp, dtype=dtype, group_size=group,
                            round_sf=round_sf, sf_ue8m0=ue8m0)
    torch.cuda.synchronize()
    d = oracle.FMT_E2M1 if dtype == "e2m1" else oracle.FMT_E4M3
    oq, osf = oracle.swiglu_cast(gu, w, clamp_value=clamp, dtype=d, group_size=group, round_sf=round_sf,
                                 sf_ue8m0=ue8m0)
    ok, det = fmt_tolerance_report(q.cpu().numpy(), sf.cpu().numpy(), oq, osf, d, group, ue8m0, round_sf)
    assert ok, det


@pytest.mark.parametrize("split", [False, True])
def test_row_kernel_exact_regions_bit_exact(split):
    """Gates >= 17 (silu(l) == l), 0 and <= -89 give exact values: the row kernel matches the oracle bit for
    bit there, as the general kernel does, with one workgroup per row and with rows split over waves."""
    rows, inter = (_row_counts()[6] if split else 64), 2048
    rng = np.random.default_rng(5)
    gate = rng.choice(np.array([17.0, 40.0, 0.0, -100.0, -89.5, 1e4], np.float32), size=(rows, inter))
    up = rng.standard_normal((rows, inter)).astype(np.float32)
    gu = np.concatenate([W.f32_to_bf16_bits(gate), W.f32_to_bf16_bits(up)], axis=1)
    w = np.float32(2.0) ** rng.integers(-3, 3, rows).astype(np.float32)
    gu_d = torch.from_numpy(gu.view(np.int16)).cuda().view(torch.bfloat16)
    q, sf = moe.swiglu_cast_fp8(gu_d, torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    oq, osf = oracle.swiglu_cast_fp8(gu, w)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), osf.view(np.uint32))
