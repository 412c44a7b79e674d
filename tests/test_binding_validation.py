"""The Python binding's argument checks (CPU: the helpers on host tensors;
no library call).  Caller-supplied outputs must be contiguous, on the
inputs' device, of the right dtype and exactly the shape the call writes:
the C ABI takes raw pointers and cannot see a buffer's size, so a short
output would be written past its end."""
import pytest
import torch

from moe_routing_fp8_amd import _native as N

CPU = torch.device("cpu")


def test_need_out_accepts_exact_outputs_and_none():
    N._need_out(None, torch.int32, (3,), "x", CPU)
    N._need_out(torch.empty((4, 8), dtype=torch.uint8), N._FP8, (4, 8), "out", CPU)
    N._need_out(torch.empty((4, 8), dtype=torch.float8_e4m3fn), N._FP8, (4, 8), "out", CPU)


@pytest.mark.parametrize("t,why", [
    (torch.empty((4, 7), dtype=torch.uint8), "short row"),
    (torch.empty((3, 8), dtype=torch.uint8), "too few rows"),
    (torch.empty((5, 8), dtype=torch.uint8), "too many rows"),
    (torch.empty(32, dtype=torch.uint8), "flat"),
    (torch.empty((4, 8), dtype=torch.int8), "dtype"),
    (torch.empty((8, 4), dtype=torch.uint8).t(), "not contiguous"),
    (torch.empty((4, 16), dtype=torch.uint8)[:, :8], "strided view"),
])
def test_need_out_rejects(t, why):
    with pytest.raises(ValueError):
        N._need_out(t, N._FP8, (4, 8), "out", CPU)


def test_need_out_rejects_other_device():
    t = torch.empty((4, 8), dtype=torch.uint8, device="meta")
    with pytest.raises(ValueError):
        N._need_out(t, N._FP8, (4, 8), "out", CPU)


def test_device_and_shape_helpers():
    a, b = torch.empty(2), torch.empty(3)
    assert N._device(a, None, b) == CPU
    with pytest.raises(ValueError):
        N._device(a, torch.empty(1, device="meta"))
    N._shape(torch.empty((2, 3)), (2, 3), "x")
    with pytest.raises(ValueError):
        N._shape(torch.empty((2, 3)), (3, 2), "x")


def test_workspace_checks():
    assert N._workspace(torch.empty(512, dtype=torch.uint8), CPU) == 512
    for bad in (torch.empty(128, dtype=torch.int32), torch.empty((2, 256), dtype=torch.uint8),
                torch.empty(512, dtype=torch.uint8)[::2]):
        with pytest.raises(ValueError):
            N._workspace(bad, CPU)


def test_call_rejects_host_tensors():
    with pytest.raises(ValueError):
        N._call("moe_topk_gate", CPU, None)
