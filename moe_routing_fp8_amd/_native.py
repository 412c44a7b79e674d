"""ctypes binding of libmoe_fp8.so (the C ABI in include/moe_fp8.h).

Argument marshalling only: every step of the dispatch path runs in the HIP
kernels behind the C ABI.  Tensors are torch device tensors (torch supplies
device memory and streams); outputs are allocated here when not given.
There is no CPU fallback: without the built library every call raises.
"""
import contextlib
import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe_fp8.h")

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

MOE_FMT_E4M3 = 0
MOE_FMT_E2M1 = 1


class moe_cast_format(ctypes.Structure):
    """struct moe_cast_format of include/moe_fp8.h."""
    _fields_ = [("dtype", ctypes.c_int32), ("group_size", ctypes.c_int32), ("round_sf", ctypes.c_int32),
                ("sf_ue8m0", ctypes.c_int32), ("clamp_min", ctypes.c_float)]


_SIGNATURES = {
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_last_hip_error": ([], ctypes.c_int),
    "moe_fp8_version": ([], ctypes.c_int),
    "moe_topk_gate": ([_p, _i64, _i32, _i32, _i32, _p, _p, _p], ctypes.c_int),
    "moe_token_map_workspace_bytes": ([_i64, _i32, _i32], _sz),
    "moe_token_map": ([_p, _i64, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p], ctypes.c_int),
    "moe_token_map_noalloc": ([_p, _i64, _i32, _i32, _p, _p, _p, _p, _p], ctypes.c_int),
    "moe_expand_cast_fp8": ([_p, _i64, _i32, _i32, _p, _p, _i64, _i32, _p, _p, _p, _p], ctypes.c_int),
    "swiglu_cast_fp8": ([_p, _i64, _i32, _p, _f32, _i32, _p, _p, _p], ctypes.c_int),
    "moe_combine": ([_p, _i64, _i32, _p, _p, _i64, _i32, _p, _p], ctypes.c_int),
    "moe_token_map_aligned_rows": ([_i64, _i32, _i32, _i32], _sz),
    "moe_token_map_aligned": ([_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _i64, _p, _sz, _p],
                              ctypes.c_int),
    "moe_expand_cast_fp8_padded": ([_p, _i64, _i32, _i32, _p, _p, _p, _i64, _i32, _p, _p, _p, _p],
                                   ctypes.c_int),
    "moe_expand_cast": ([_p, _i64, _i32, _i32, _p, _p, _i64, ctypes.POINTER(moe_cast_format), _p, _p, _p, _p],
                        ctypes.c_int),
    "swiglu_cast": ([_p, _i64, _i32, _p, _f32, ctypes.POINTER(moe_cast_format), _p, _p, _p], ctypes.c_int),
    "moe_route_workspace_bytes": ([_i64, _i32, _i32], _sz),
    "moe_route": ([_p, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _sz, _i32, _p], ctypes.c_int),
    "moe_dispatch_workspace_bytes": ([_i64, _i32, _i32], _sz),
    "moe_dispatch": ([_p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                      _sz, _i32, _p], ctypes.c_int),
    "moe_check_scores": ([_p, _i64, _i32, _i32, _p, _p], ctypes.c_int),
    "moe_check_topk_idx": ([_p, _i64, _i32, _i32, _p, _p], ctypes.c_int),
    "moe_check_pos_workspace_bytes": ([_i64], _sz),
    "moe_check_pos": ([_p, _i64, _i32, _i64, _p, _sz, _p, _p], ctypes.c_int),
    "moe_check_activations": ([_p, _i64, _p, _p], ctypes.c_int),
    "moe_check_dispatch": ([_p, _sz, _p, _p], ctypes.c_int),
}

# MOE_CHECK_* bits of the input checks (include/moe_fp8.h)
CHECK_FLAGS = {0x01: "MOE_CHECK_NONFINITE_SCORE", 0x02: "MOE_CHECK_NONPOSITIVE_SCORE",
               0x04: "MOE_CHECK_ID_RANGE", 0x08: "MOE_CHECK_ID_DUPLICATE",
               0x10: "MOE_CHECK_POS_RANGE", 0x20: "MOE_CHECK_POS_DUPLICATE",
               0x40: "MOE_CHECK_NONFINITE_ACTIVATION", 0x80: "MOE_CHECK_DISPATCH_TIMEOUT"}

MOE_ROUTE_AUTO = 0
MOE_ROUTE_FUSED = 1
MOE_ROUTE_SPLIT = 2
MOE_ROUTE_LOCAL = 3

MOE_DISPATCH_AUTO = 0
MOE_DISPATCH_SINGLE_LAUNCH = 1
MOE_DISPATCH_SPLIT = 2
MOE_DISPATCH_ROUTE_FUSED = 3
MOE_DISPATCH_TOPK_THEN_COPY = 4

_lib = None


class MoeError(RuntimeError):
    def __init__(self, name, status, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{name} failed: {STATUS_NAMES.get(status, status)}"
        if hip_error:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """Load libmoe_fp8.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; "
                           f"g.build()'` (hipcc, gfx950) first; there is no CPU fallback")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = res
    _lib = handle
    return handle


def header_functions():
    """Names of the functions include/moe_fp8.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "while", "for", "sizeof", "return"})


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _call(name, dev, stream, *args):
    """Calls entry point `name` with `args` and the stream, `dev` current
    (the tensors' device; the stream defaults to its current stream)."""
    if dev.type != "cuda":
        raise ValueError(f"{name}: tensors on {dev}, not a GPU")
    if dev.index is not None and dev.index != torch.cuda.current_device():
        with torch.cuda.device(dev):
            return _call(name, dev, stream, *args)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"{name}: stream on {stream.device}, tensors on {dev}")
    status = getattr(lib(), name)(*args, stream.cuda_stream)
    if status != MOE_OK:
        raise MoeError(name, status, lib().moe_last_hip_error() if status == 4 else 0)


def _alloc_on(stream):
    """Context for the tensors a call allocates (outputs, workspaces, flag
    words): with an explicit `stream` they are allocated, and zeroed, on that
    stream, the one the call's kernels run on, so the caching allocator never
    hands their memory to other work while those kernels may still use it.
    Without one the call runs on the current stream, where they are anyway."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _need(t: torch.Tensor, dtype, ndim, name):
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected a contiguous {ndim}-d {dtype} device tensor, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} on {t.device}")


def _shape(t: torch.Tensor, shape, name):
    if t.shape != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_out(t: Optional[torch.Tensor], dtypes, shape, name, dev):
    """A caller-supplied output: contiguous, on `dev`, of one of `dtypes` and
    exactly `shape` (the kernels write every element the shape implies)."""
    if t is None:
        return
    if isinstance(dtypes, tuple):
        bad_dtype = t.dtype not in dtypes
    else:
        bad_dtype = t.dtype != dtypes
        dtypes = (dtypes,)
    if bad_dtype or t.shape != shape or t.device != dev or not t.is_contiguous():
        if bad_dtype or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {' or '.join(map(str, dtypes))} tensor on {dev}, "
                             f"got {t.dtype} contiguous={t.is_contiguous()} on {t.device}")
        _shape(t, shape, name)


def _device(*ts):
    """The one CUDA device all given tensors are on."""
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError(f"tensors on several devices: {sorted(map(str, devs))}")
    return devs.pop()


def check_flag_names(bits: int):
    """Names of the MOE_CHECK_* bits set in `bits`."""
    return [name for bit, name in CHECK_FLAGS.items() if bits & bit]


def _flags(flags: Optional[torch.Tensor], dev, stream):
    """The caller's flag word, or a new one zeroed on the stream the check runs on."""
    if flags is None:
        with _alloc_on(stream):
            return torch.zeros(1, dtype=torch.int32, device=dev)
    _need_out(flags, torch.int32, (1,), "flags", dev)
    return flags


def moe_check_scores(scores: torch.Tensor, require_positive: bool = False, flags=None, stream=None) -> torch.Tensor:
    """ORs MOE_CHECK_NONFINITE_SCORE / MOE_CHECK_NONPOSITIVE_SCORE into `flags` (int32 [1] on the device,
    zeroed here if None) for the fp32 [T, E] scores; returns `flags` (read it after the stream)."""
    _need(scores, torch.float32, 2, "scores")
    T, E = scores.shape
    dev = scores.device
    flags = _flags(flags, dev, stream)
    _call("moe_check_scores", dev, stream, _ptr(scores), T, E, int(bool(require_positive)), _ptr(flags))
    return flags


def moe_check_topk_idx(topk_idx: torch.Tensor, num_experts: int, flags=None, stream=None) -> torch.Tensor:
    """ORs MOE_CHECK_ID_RANGE / MOE_CHECK_ID_DUPLICATE into `flags` for the int64 [T, K] ids."""
    _need(topk_idx, torch.int64, 2, "topk_idx")
    T, K = topk_idx.shape
    dev = topk_idx.device
    flags = _flags(flags, dev, stream)
    _call("moe_check_topk_idx", dev, stream, _ptr(topk_idx), T, K, num_experts, _ptr(flags))
    return flags


def moe_check_pos(pos: torch.Tensor, num_rows: int, flags=None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """ORs MOE_CHECK_POS_RANGE / MOE_CHECK_POS_DUPLICATE into `flags` for the int32 [T, K] positions
    into num_rows rows."""
    _need(pos, torch.int32, 2, "pos")
    T, K = pos.shape
    dev = pos.device
    flags = _flags(flags, dev, stream)
    need = int(lib().moe_check_pos_workspace_bytes(num_rows))
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _call("moe_check_pos", dev, stream, _ptr(pos), T, K, num_rows, _ptr(workspace), _workspace(workspace, dev),
          _ptr(flags))
    return flags


def moe_check_activations(x: torch.Tensor, flags=None, stream=None) -> torch.Tensor:
    """ORs MOE_CHECK_NONFINITE_ACTIVATION into `flags` if any value of the contiguous bf16 tensor x is NaN
    or infinite (the precondition of the casts and the combine)."""
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError(f"x: expected a contiguous bf16 device tensor, got {x.dtype} on {x.device}")
    dev = x.device
    flags = _flags(flags, dev, stream)
    _call("moe_check_activations", dev, stream, _ptr(x), x.numel(), _ptr(flags))
    return flags


def moe_check_dispatch(workspace: torch.Tensor, flags=None, stream=None) -> torch.Tensor:
    """ORs MOE_CHECK_DISPATCH_TIMEOUT into `flags` if a single-launch moe_dispatch on this workspace gave
    up a grid-barrier wait (its outputs are then invalid; the word stays set until the workspace is zeroed)."""
    dev = workspace.device
    flags = _flags(flags, dev, stream)
    _call("moe_check_dispatch", dev, stream, _ptr(workspace), _workspace(workspace, dev), _ptr(flags))
    return flags


def debug_enabled() -> bool:
    """MOE_FP8_DEBUG set to anything but "" or "0": every call first checks its inputs on the device
    (moe_check_*) and raises ValueError naming what it found.  Each check waits for its stream, so debug
    mode cannot run under graph capture (the calls raise there)."""
    return os.environ.get("MOE_FP8_DEBUG", "0") not in ("", "0")


def _debug_raise(name: str, check, stream, exc=ValueError):
    """Runs `check` (a moe_check_* call returning its flag word), waits for the stream and raises `exc`
    (ValueError for an input that breaks a precondition) naming the bits found."""
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError(f"{name}: MOE_FP8_DEBUG waits for the stream and reads the flags back, which a "
                           "stream under graph capture cannot do; unset it while capturing")
    flags = check()
    (stream if stream is not None else torch.cuda.current_stream(flags.device)).synchronize()
    bits = int(flags.item()) & 0xFFFFFFFF
    if bits:
        raise exc(f"{name}: check failed (MOE_FP8_DEBUG): {', '.join(check_flag_names(bits))}")


def _workspace(ws: torch.Tensor, dev):
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous() or ws.device != dev:
        raise ValueError(f"workspace: expected a contiguous 1-d uint8 tensor on {dev}, got "
                         f"{ws.dtype} {tuple(ws.shape)} on {ws.device}")
    return ws.numel()


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def moe_topk_gate(scores: torch.Tensor, num_topk: int, renormalize: bool = False,
                  with_weights: Optional[bool] = None, out=None, stream=None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """scores fp32 [T, E] -> (topk_idx int64 [T, K], topk_weights fp32 [T, K] or None)."""
    _need(scores, torch.float32, 2, "scores")
    T, E = scores.shape
    dev = scores.device
    want_w = renormalize if with_weights is None else with_weights
    if out is None:
        with _alloc_on(stream):
            idx = torch.empty((T, num_topk), dtype=torch.int64, device=dev)
            w = torch.empty((T, num_topk), dtype=torch.float32, device=dev) if want_w else None
    else:
        idx, w = out
        _need_out(idx, torch.int64, (T, num_topk), "topk_idx", dev)
        _need_out(w, torch.float32, (T, num_topk), "topk_weights", dev)
    if debug_enabled():
        _debug_raise("moe_topk_gate", lambda: moe_check_scores(scores, bool(renormalize), stream=stream), stream)
    _call("moe_topk_gate", dev, stream, _ptr(scores), T, E, num_topk, int(bool(renormalize)), _ptr(idx), _ptr(w))
    return idx, w


def moe_token_map_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int) -> int:
    return int(lib().moe_token_map_workspace_bytes(num_tokens, num_topk, num_experts))


def moe_token_map(topk_idx: torch.Tensor, num_experts: int, with_row_token: bool = True,
                  workspace: Optional[torch.Tensor] = None, out=None, stream=None):
    """topk_idx int64 [T, K] -> (counts int32 [E], offsets int32 [E+1], pos int32 [T, K],
    row_token int32 [T*K] or None)."""
    _need(topk_idx, torch.int64, 2, "topk_idx")
    T, K = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        with _alloc_on(stream):
            counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
            offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
            pos = torch.empty((T, K), dtype=torch.int32, device=dev)
            row_token = torch.empty(T * K, dtype=torch.int32, device=dev) if with_row_token else None
    else:
        counts, offsets, pos, row_token = out
        _need_out(counts, torch.int32, (num_experts,), "expert_counts", dev)
        _need_out(offsets, torch.int32, (num_experts + 1,), "expert_offsets", dev)
        _need_out(pos, torch.int32, (T, K), "pos", dev)
        _need_out(row_token, torch.int32, (T * K,), "row_token", dev)
    need = moe_token_map_workspace_bytes(T, K, num_experts)
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if debug_enabled():
        _debug_raise("moe_token_map", lambda: moe_check_topk_idx(topk_idx, num_experts, stream=stream), stream)
    _call("moe_token_map", dev, stream, _ptr(topk_idx), T, K, num_experts, _ptr(counts), _ptr(offsets), _ptr(pos),
          _ptr(row_token), _ptr(workspace), _workspace(workspace, dev))
    return counts, offsets, pos, row_token


def moe_token_map_noalloc(topk_idx: torch.Tensor, num_experts: int, with_row_token: bool = True, out=None,
                          stream=None):
    """moe_token_map through the entry point that allocates nothing (its count table is the library's
    fixed device array); same outputs.  Pass `out` to keep this call free of allocations too."""
    _need(topk_idx, torch.int64, 2, "topk_idx")
    T, K = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        with _alloc_on(stream):
            counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
            offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
            pos = torch.empty((T, K), dtype=torch.int32, device=dev)
            row_token = torch.empty(T * K, dtype=torch.int32, device=dev) if with_row_token else None
    else:
        counts, offsets, pos, row_token = out
        _need_out(counts, torch.int32, (num_experts,), "expert_counts", dev)
        _need_out(offsets, torch.int32, (num_experts + 1,), "expert_offsets", dev)
        _need_out(pos, torch.int32, (T, K), "pos", dev)
        _need_out(row_token, torch.int32, (T * K,), "row_token", dev)
    if debug_enabled():
        _debug_raise("moe_token_map_noalloc", lambda: moe_check_topk_idx(topk_idx, num_experts, stream=stream),
                     stream)
    _call("moe_token_map_noalloc", dev, stream, _ptr(topk_idx), T, K, num_experts, _ptr(counts), _ptr(offsets),
          _ptr(pos), _ptr(row_token))
    return counts, offsets, pos, row_token


def moe_expand_cast_fp8(x: torch.Tensor, pos: Optional[torch.Tensor] = None,
                        topk_weights: Optional[torch.Tensor] = None, group_size: int = 128,
                        out=None, stream=None):
    """x bf16 [T, H]; pos int32 [T, K] or None (identity) ->
    (out e4m3 [R, H], out_sf fp32 [R, H/group], out_weights fp32 [R] or None)."""
    _need(x, torch.bfloat16, 2, "x")
    T, H = x.shape
    K = 1
    if pos is not None:
        _need(pos, torch.int32, 2, "pos")
        K = pos.shape[1]
        _shape(pos, (T, K), "pos")
    if topk_weights is not None:
        _need(topk_weights, torch.float32, 2, "topk_weights")
        _shape(topk_weights, (T, K), "topk_weights")
    dev = _device(x, pos, topk_weights)
    R = T * K
    G = H // group_size if group_size > 0 else 0
    if out is None:
        with _alloc_on(stream):
            o = torch.empty((R, H), dtype=torch.uint8, device=dev)
            sf = torch.empty((R, G), dtype=torch.float32, device=dev)
            ow = torch.empty(R, dtype=torch.float32, device=dev) if topk_weights is not None else None
    else:
        o, sf, ow = out
        _need_out(o, _FP8, (R, H), "out", dev)
        _need_out(sf, torch.float32, (R, G), "out_sf", dev)
        _need_out(ow, torch.float32, (R,), "out_weights", dev)
        o = o.view(torch.uint8)
    if debug_enabled():
        _debug_raise("moe_expand_cast_fp8", lambda: moe_check_activations(x, stream=stream), stream)
        if pos is not None:
            _debug_raise("moe_expand_cast_fp8", lambda: moe_check_pos(pos, R, stream=stream), stream)
    _call("moe_expand_cast_fp8", dev, stream, _ptr(x), T, H, K, _ptr(pos), _ptr(topk_weights), R, group_size,
          _ptr(o), _ptr(sf), _ptr(ow))
    return o.view(torch.float8_e4m3fn), sf, ow


def swiglu_cast_fp8(gate_up: torch.Tensor, row_weights: Optional[torch.Tensor] = None,
                    clamp_value: float = 0.0, group_size: int = 128, out=None, stream=None):
    """gate_up bf16 [R, 2I] = [gate | up] -> (out e4m3 [R, I], out_sf fp32 [R, I/group])."""
    _need(gate_up, torch.bfloat16, 2, "gate_up")
    R, two_i = gate_up.shape
    if two_i % 2:
        raise ValueError("gate_up: last dimension must be 2 * inter")
    inter = two_i // 2
    if row_weights is not None:
        _need(row_weights, torch.float32, 1, "row_weights")
        _shape(row_weights, (R,), "row_weights")
    dev = _device(gate_up, row_weights)
    G = inter // group_size if group_size > 0 else 0
    if out is None:
        with _alloc_on(stream):
            o = torch.empty((R, inter), dtype=torch.uint8, device=dev)
            sf = torch.empty((R, G), dtype=torch.float32, device=dev)
    else:
        o, sf = out
        _need_out(o, _FP8, (R, inter), "out", dev)
        _need_out(sf, torch.float32, (R, G), "out_sf", dev)
        o = o.view(torch.uint8)
    if debug_enabled():
        _debug_raise("swiglu_cast_fp8", lambda: moe_check_activations(gate_up, stream=stream), stream)
    _call("swiglu_cast_fp8", dev, stream, _ptr(gate_up), R, inter, _ptr(row_weights), float(clamp_value),
          group_size, _ptr(o), _ptr(sf))
    return o.view(torch.float8_e4m3fn), sf


def moe_combine(y_rows: torch.Tensor, pos: torch.Tensor, weights: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y_rows bf16 [R, H] (expert-grouped rows), pos int32 [T, K], weights fp32 [T, K] or None
    -> bf16 [T, H] = sum_k w[t,k] * y_rows[pos[t,k]] (fp32, k order)."""
    _need(y_rows, torch.bfloat16, 2, "y_rows")
    _need(pos, torch.int32, 2, "pos")
    R, H = y_rows.shape
    T, K = pos.shape
    if weights is not None:
        _need(weights, torch.float32, 2, "weights")
        _shape(weights, (T, K), "weights")
    dev = _device(y_rows, pos, weights)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need_out(out, torch.bfloat16, (T, H), "out", dev)
    if debug_enabled():
        _debug_raise("moe_combine", lambda: moe_check_activations(y_rows, stream=stream), stream)
    _call("moe_combine", dev, stream, _ptr(y_rows), R, H, _ptr(pos), _ptr(weights), T, K, _ptr(out))
    return out


def moe_token_map_aligned_rows(num_tokens: int, num_topk: int, num_local_experts: int, align: int) -> int:
    return int(lib().moe_token_map_aligned_rows(num_tokens, num_topk, num_local_experts, align))


def moe_token_map_aligned(topk_idx: torch.Tensor, expert_begin: int, expert_end: int, align: int,
                          num_rows: Optional[int] = None, with_row_token: bool = True,
                          workspace: Optional[torch.Tensor] = None, out=None, stream=None):
    """topk_idx int64 [T, K] -> (counts int32 [EL], offsets int32 [EL+1], pos int32 [T, K],
    row_token int32 [num_rows] or None), segments padded to multiples of align."""
    _need(topk_idx, torch.int64, 2, "topk_idx")
    T, K = topk_idx.shape
    EL = expert_end - expert_begin
    dev = topk_idx.device
    if out is not None and num_rows is None and out[3] is not None:
        num_rows = out[3].numel()
    if num_rows is None:
        num_rows = moe_token_map_aligned_rows(T, K, max(EL, 1), align)
    if out is None:
        with _alloc_on(stream):
            counts = torch.empty(max(EL, 0), dtype=torch.int32, device=dev)
            offsets = torch.empty(max(EL, 0) + 1, dtype=torch.int32, device=dev)
            pos = torch.empty((T, K), dtype=torch.int32, device=dev)
            row_token = torch.empty(num_rows, dtype=torch.int32, device=dev) if with_row_token else None
    else:
        counts, offsets, pos, row_token = out
        _need_out(counts, torch.int32, (max(EL, 0),), "expert_counts", dev)
        _need_out(offsets, torch.int32, (max(EL, 0) + 1,), "expert_offsets", dev)
        _need_out(pos, torch.int32, (T, K), "pos", dev)
        _need_out(row_token, torch.int32, (num_rows,), "row_token", dev)
    need = moe_token_map_workspace_bytes(T, K, max(EL, 1))
    if workspace is None:
        with _alloc_on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _call("moe_token_map_aligned", dev, stream, _ptr(topk_idx), T, K, expert_begin, expert_end, align, _ptr(counts),
          _ptr(offsets), _ptr(pos), _ptr(row_token), num_rows, _ptr(workspace), _workspace(workspace, dev))
    return counts, offsets, pos, row_token


def moe_expand_cast_fp8_padded(x: torch.Tensor, pos: torch.Tensor, row_token: torch.Tensor,
                               topk_weights: Optional[torch.Tensor] = None, group_size: int = 128,
                               out=None, stream=None):
    """x bf16 [T, H]; pos int32 [T, K]; row_token int32 [R] (from moe_token_map_aligned) ->
    (out e4m3 [R, H], out_sf fp32 [R, H/group], out_weights fp32 [R] or None); rows with
    row_token < 0 are zero-filled."""
    _need(x, torch.bfloat16, 2, "x")
    _need(pos, torch.int32, 2, "pos")
    _need(row_token, torch.int32, 1, "row_token")
    T, H = x.shape
    K = pos.shape[1]
    _shape(pos, (T, K), "pos")
    R = row_token.shape[0]
    if topk_weights is not None:
        _need(topk_weights, torch.float32, 2, "topk_weights")
        _shape(topk_weights, (T, K), "topk_weights")
    dev = _device(x, pos, row_token, topk_weights)
    G = H // group_size if group_size > 0 else 0
    if out is None:
        with _alloc_on(stream):
            o = torch.empty((R, H), dtype=torch.uint8, device=dev)
            sf = torch.empty((R, G), dtype=torch.float32, device=dev)
            ow = torch.empty(R, dtype=torch.float32, device=dev) if topk_weights is not None else None
    else:
        o, sf, ow = out
        _need_out(o, _FP8, (R, H), "out", dev)
        _need_out(sf, torch.float32, (R, G), "out_sf", dev)
        _need_out(ow, torch.float32, (R,), "out_weights", dev)
        o = o.view(torch.uint8)
    if debug_enabled():
        _debug_raise("moe_expand_cast_fp8_padded", lambda: moe_check_activations(x, stream=stream), stream)
        _debug_raise("moe_expand_cast_fp8_padded", lambda: moe_check_pos(pos, R, stream=stream), stream)
    _call("moe_expand_cast_fp8_padded", dev, stream, _ptr(x), T, H, K, _ptr(pos), _ptr(topk_weights),
          _ptr(row_token), R, group_size, _ptr(o), _ptr(sf), _ptr(ow))
    return o.view(torch.float8_e4m3fn), sf, ow


def moe_route_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int) -> int:
    return int(lib().moe_route_workspace_bytes(num_tokens, num_topk, num_experts))


def moe_route(scores: torch.Tensor, num_topk: int, renormalize: bool = False, with_weights: Optional[bool] = None,
              with_row_token: bool = True, mode: int = MOE_ROUTE_AUTO, workspace: Optional[torch.Tensor] = None,
              out=None, stream=None):
    """scores fp32 [T, E] -> dict of topk_idx, topk_weights, counts, offsets, pos, row_token (moe_topk_gate then
    moe_token_map, bit for bit).  `mode`: MOE_ROUTE_AUTO (the fastest form measured for the batch),
    MOE_ROUTE_FUSED (the top-k with the counting, then the slots), MOE_ROUTE_SPLIT, or MOE_ROUTE_LOCAL (one
    launch, up to 32 tokens).  `workspace` (uint8, from moe_route_workspace_bytes) must have been zeroed once;
    a fresh zeroed one is made if None."""
    _need(scores, torch.float32, 2, "scores")
    T, E = scores.shape
    K = num_topk
    R = T * K
    dev = _device(scores)
    want_w = renormalize if with_weights is None else with_weights
    if out is None:
        with _alloc_on(stream):
            out = {
                "topk_idx": torch.empty((T, K), dtype=torch.int64, device=dev),
                "topk_weights": torch.empty((T, K), dtype=torch.float32, device=dev) if want_w else None,
                "counts": torch.empty(E, dtype=torch.int32, device=dev),
                "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
                "pos": torch.empty((T, K), dtype=torch.int32, device=dev),
                "row_token": torch.empty(R, dtype=torch.int32, device=dev) if with_row_token else None,
            }
    else:
        for key, dtypes, shape in (("topk_idx", torch.int64, (T, K)), ("topk_weights", torch.float32, (T, K)),
                                   ("counts", torch.int32, (E,)), ("offsets", torch.int32, (E + 1,)),
                                   ("pos", torch.int32, (T, K)), ("row_token", torch.int32, (R,))):
            _need_out(out.get(key), dtypes, shape, key, dev)
    if workspace is None:
        with _alloc_on(stream):  # zeroed on the stream the routing runs on
            workspace = torch.zeros(max(moe_route_workspace_bytes(T, K, E), 256), dtype=torch.uint8, device=dev)
    o = out
    if debug_enabled():
        _debug_raise("moe_route", lambda: moe_check_scores(scores, bool(renormalize), stream=stream), stream)
    _call("moe_route", dev, stream, _ptr(scores), T, E, K, int(bool(renormalize)), _ptr(o["topk_idx"]),
          _ptr(o.get("topk_weights")), _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["pos"]),
          _ptr(o.get("row_token")), _ptr(workspace), _workspace(workspace, dev), mode)
    return o


def moe_dispatch_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int) -> int:
    return int(lib().moe_dispatch_workspace_bytes(num_tokens, num_topk, num_experts))


def moe_dispatch(scores: torch.Tensor, x: torch.Tensor, num_topk: int, renormalize: bool = False,
                 with_weights: Optional[bool] = None, with_row_token: bool = True, group_size: int = 128,
                 mode: int = MOE_DISPATCH_AUTO, workspace: Optional[torch.Tensor] = None, out=None,
                 stream=None):
    """scores fp32 [T, E], x bf16 [T, H] -> dict of topk_idx, topk_weights, counts, offsets, pos,
    row_token, out (e4m3 [T*K, H]), out_sf, out_weights: moe_topk_gate, moe_token_map and
    moe_expand_cast_fp8 in one call, bit for bit.  `mode`: MOE_DISPATCH_AUTO (the fastest form measured for
    the batch), MOE_DISPATCH_SINGLE_LAUNCH, MOE_DISPATCH_TOPK_THEN_COPY, MOE_DISPATCH_ROUTE_FUSED or
    MOE_DISPATCH_SPLIT.  `workspace` (uint8, from moe_dispatch_workspace_bytes) must have been zeroed once; a
    fresh zeroed one is made if None."""
    _need(scores, torch.float32, 2, "scores")
    _need(x, torch.bfloat16, 2, "x")
    T, E = scores.shape
    H = x.shape[1]
    _shape(x, (T, H), "x")
    K = num_topk
    R = T * K
    dev = _device(scores, x)
    G = H // group_size if group_size > 0 else 0
    want_w = renormalize if with_weights is None else with_weights
    if out is None:
        with _alloc_on(stream):
            out = _dispatch_outputs(T, E, K, H, G, R, want_w, with_row_token, dev)
    else:
        for key, dtypes, shape in (("topk_idx", torch.int64, (T, K)), ("topk_weights", torch.float32, (T, K)),
                                   ("counts", torch.int32, (E,)), ("offsets", torch.int32, (E + 1,)),
                                   ("pos", torch.int32, (T, K)), ("row_token", torch.int32, (R,)),
                                   ("out", _FP8, (R, H)), ("out_sf", torch.float32, (R, G)),
                                   ("out_weights", torch.float32, (R,))):
            _need_out(out.get(key), dtypes, shape, key, dev)
    if workspace is None:
        with _alloc_on(stream):  # zeroed on the stream the dispatch runs on
            workspace = torch.zeros(max(moe_dispatch_workspace_bytes(T, K, E), 256), dtype=torch.uint8,
                                    device=dev)
    o = out
    q = o["out"].view(torch.uint8)
    if debug_enabled():
        _debug_raise("moe_dispatch", lambda: moe_check_scores(scores, bool(renormalize), stream=stream), stream)
        _debug_raise("moe_dispatch", lambda: moe_check_activations(x, stream=stream), stream)
    _call("moe_dispatch", dev, stream, _ptr(scores), _ptr(x), T, E, K, H, int(bool(renormalize)), group_size,
          _ptr(o["topk_idx"]), _ptr(o.get("topk_weights")), _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["pos"]),
          _ptr(o.get("row_token")), _ptr(q), _ptr(o["out_sf"]), _ptr(o.get("out_weights")), _ptr(workspace),
          _workspace(workspace, dev), mode)
    o["out"] = q.view(torch.float8_e4m3fn)
    if debug_enabled():
        # a single-launch call whose grid barrier gave up returns MOE_OK with invalid outputs
        _debug_raise("moe_dispatch", lambda: moe_check_dispatch(workspace, stream=stream), stream,
                     exc=RuntimeError)
    return o


def _dispatch_outputs(T, E, K, H, G, R, want_w, with_row_token, dev):
    return {
        "topk_idx": torch.empty((T, K), dtype=torch.int64, device=dev),
        "topk_weights": torch.empty((T, K), dtype=torch.float32, device=dev) if want_w else None,
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "pos": torch.empty((T, K), dtype=torch.int32, device=dev),
        "row_token": torch.empty(R, dtype=torch.int32, device=dev) if with_row_token else None,
        "out": torch.empty((R, H), dtype=torch.uint8, device=dev),
        "out_sf": torch.empty((R, G), dtype=torch.float32, device=dev),
        "out_weights": torch.empty(R, dtype=torch.float32, device=dev) if want_w else None,
    }


def _format(dtype, group_size, round_sf, sf_ue8m0, clamp_min):
    d = {"e4m3": MOE_FMT_E4M3, "e2m1": MOE_FMT_E2M1}.get(dtype, dtype)
    return moe_cast_format(int(d), int(group_size), int(bool(round_sf)), int(bool(sf_ue8m0)), float(clamp_min))


def _format_shapes(rows, width, fmt):
    row_bytes = width // 2 if fmt.dtype == MOE_FMT_E2M1 else width
    G = width // fmt.group_size if fmt.group_size > 0 else 0
    return (rows, row_bytes), (rows, G), torch.uint8 if fmt.sf_ue8m0 else torch.float32


def _format_outputs(rows, width, fmt, dev, out=None):
    oshape, sshape, sdtype = _format_shapes(rows, width, fmt)
    if out is not None:
        o, sf = out
        _need_out(o, _FP8 if fmt.dtype == MOE_FMT_E4M3 else torch.uint8, oshape, "out", dev)
        _need_out(sf, sdtype, sshape, "out_sf", dev)
        return o.view(torch.uint8), sf
    return torch.empty(oshape, dtype=torch.uint8, device=dev), torch.empty(sshape, dtype=sdtype, device=dev)


def _format_outputs_on(stream, rows, width, fmt, dev, out=None):
    with _alloc_on(stream):
        return _format_outputs(rows, width, fmt, dev, out)


def moe_expand_cast(x: torch.Tensor, pos: Optional[torch.Tensor] = None,
                    topk_weights: Optional[torch.Tensor] = None, dtype="e4m3", group_size: int = 128,
                    round_sf: bool = False, sf_ue8m0: bool = False, clamp_min: float = 0.0, out=None,
                    stream=None):
    """x bf16 [T, H]; pos int32 [T, K] or None (identity) -> (codes uint8 [R, H] (e4m3) or [R, H/2]
    (e2m1, element 2i in the low nibble), scales fp32 or uint8 (UE8M0) [R, H/group], weights or None)."""
    _need(x, torch.bfloat16, 2, "x")
    T, H = x.shape
    K = 1
    if pos is not None:
        _need(pos, torch.int32, 2, "pos")
        K = pos.shape[1]
        _shape(pos, (T, K), "pos")
    if topk_weights is not None:
        _need(topk_weights, torch.float32, 2, "topk_weights")
        _shape(topk_weights, (T, K), "topk_weights")
    dev = _device(x, pos, topk_weights)
    fmt = _format(dtype, group_size, round_sf, sf_ue8m0, clamp_min)
    R = T * K
    if out is None:
        o, sf = _format_outputs_on(stream, R, H, fmt, dev)
        with _alloc_on(stream):
            ow = torch.empty(R, dtype=torch.float32, device=dev) if topk_weights is not None else None
    else:
        o, sf = _format_outputs(R, H, fmt, dev, out[:2])
        ow = out[2]
        _need_out(ow, torch.float32, (R,), "out_weights", dev)
    if debug_enabled():
        _debug_raise("moe_expand_cast", lambda: moe_check_activations(x, stream=stream), stream)
        if pos is not None:
            _debug_raise("moe_expand_cast", lambda: moe_check_pos(pos, R, stream=stream), stream)
    _call("moe_expand_cast", dev, stream, _ptr(x), T, H, K, _ptr(pos), _ptr(topk_weights), R, ctypes.byref(fmt),
          _ptr(o), _ptr(sf), _ptr(ow))
    return o, sf, ow


def swiglu_cast(gate_up: torch.Tensor, row_weights: Optional[torch.Tensor] = None, clamp_value: float = 0.0,
                dtype="e4m3", group_size: int = 128, round_sf: bool = False, sf_ue8m0: bool = False,
                clamp_min: float = 0.0, out=None, stream=None):
    """gate_up bf16 [R, 2I] -> (codes uint8 [R, I] or [R, I/2], scales fp32 or uint8 [R, I/group])."""
    _need(gate_up, torch.bfloat16, 2, "gate_up")
    R, two_i = gate_up.shape
    if two_i % 2:
        raise ValueError("gate_up: last dimension must be 2 * inter")
    inter = two_i // 2
    if row_weights is not None:
        _need(row_weights, torch.float32, 1, "row_weights")
        _shape(row_weights, (R,), "row_weights")
    dev = _device(gate_up, row_weights)
    fmt = _format(dtype, group_size, round_sf, sf_ue8m0, clamp_min)
    o, sf = _format_outputs_on(stream, R, inter, fmt, dev, out)
    if debug_enabled():
        _debug_raise("swiglu_cast", lambda: moe_check_activations(gate_up, stream=stream), stream)
    _call("swiglu_cast", dev, stream, _ptr(gate_up), R, inter, _ptr(row_weights), float(clamp_value),
          ctypes.byref(fmt), _ptr(o), _ptr(sf))
    return o, sf
