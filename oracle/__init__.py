"""CPU oracle for the MoE dispatch path (TEST INFRASTRUCTURE ONLY).

The plain, slow, single-threaded C statement of what the GPU library
computes (oracle/oracle.c), wrapped for numpy arrays.  Only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may import this
package; the library never does, and the two share no code.

Pages cited by the C source: "DeepSeek open-sources TileKernels" (itsolotime
article) sections 2, 2.1, 2.2, 3.1-3.3; "CuTeDSL at Perplexity", MoE
dispatch and combine (local kernel).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_e4m3_encode.argtypes = [_f32]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = _f32
    lib.oracle_e4m3_encode_n.argtypes = [_p, _i64, _p]
    lib.oracle_e4m3_encode_n.restype = None
    lib.oracle_cast_group.argtypes = [_p, _i32, _p, _p]
    lib.oracle_cast_group.restype = None
    lib.oracle_topk_gate.argtypes = [_p, _i64, _i32, _i32, _i32, _p, _p]
    lib.oracle_topk_gate.restype = ctypes.c_int
    lib.oracle_token_map.argtypes = [_p, _i64, _i32, _i32, _p, _p, _p, _p]
    lib.oracle_token_map.restype = ctypes.c_int
    lib.oracle_expand_cast_fp8.argtypes = [_p, _i64, _i32, _i32, _p, _p, _i64, _i32, _p, _p, _p]
    lib.oracle_expand_cast_fp8.restype = ctypes.c_int
    lib.oracle_swiglu_cast_fp8.argtypes = [_p, _i64, _i32, _p, _f32, _i32, _p, _p]
    lib.oracle_swiglu_cast_fp8.restype = ctypes.c_int
    lib.oracle_token_map_aligned.argtypes = [_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _i64]
    lib.oracle_token_map_aligned.restype = ctypes.c_int
    lib.oracle_expand_cast_fp8_padded.argtypes = [_p, _i64, _i32, _i32, _p, _p, _p, _i64, _i32, _p, _p, _p]
    lib.oracle_expand_cast_fp8_padded.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [_p, _i64, _i32, _p, _p, _i64, _i32, _p]
    lib.oracle_combine.restype = ctypes.c_int
    lib.oracle_f32_to_bf16.argtypes = [_f32]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_e2m1_encode.argtypes = [_f32]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_decode.restype = _f32
    lib.oracle_default_clamp.argtypes = [_i32]
    lib.oracle_default_clamp.restype = _f32
    lib.oracle_cast_group_fmt.argtypes = [_p, _i32, _i32, _i32, _f32, _p, _p]
    lib.oracle_cast_group_fmt.restype = None
    lib.oracle_ue8m0_encode.argtypes = [_f32]
    lib.oracle_ue8m0_encode.restype = ctypes.c_uint8
    lib.oracle_ue8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_ue8m0_decode.restype = _f32
    lib.oracle_expand_cast.argtypes = [_p, _i64, _i32, _i32, _p, _p, _i64, _i32, _i32, _i32, _f32, _i32,
                                       _p, _p, _p]
    lib.oracle_expand_cast.restype = ctypes.c_int
    lib.oracle_swiglu_cast.argtypes = [_p, _i64, _i32, _p, _f32, _i32, _i32, _i32, _f32, _i32, _p, _p]
    lib.oracle_swiglu_cast.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected the arguments (rc={rc})")


def e4m3_encode(x):
    """OCP e4m3fn codes (uint8) of fp32 values, round to nearest even, saturating."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().oracle_e4m3_encode_n(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_decode(codes):
    """fp32 values of e4m3fn codes (a 256-entry table built from the decoder)."""
    lib = _load()
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], np.float32)
    return table[np.asarray(codes, np.uint8)]


def cast_group(v):
    """One scale group: returns (codes uint8[n], sf float32)."""
    v = _c(v, np.float32)
    q = np.empty(v.size, np.uint8)
    sf = np.zeros(1, np.float32)
    _load().oracle_cast_group(_ptr(v), v.size, _ptr(q), _ptr(sf))
    return q, sf[0]


def topk_gate(scores, num_topk, renormalize=False, with_weights=None):
    """Returns (topk_idx int64[T,K], topk_weights float32[T,K] or None)."""
    scores = _c(scores, np.float32)
    T, E = scores.shape
    idx = np.empty((T, num_topk), np.int64)
    want_w = renormalize if with_weights is None else with_weights
    w = np.empty((T, num_topk), np.float32) if want_w else None
    rc = _load().oracle_topk_gate(_ptr(scores), T, E, num_topk, int(bool(renormalize)),
                                  _ptr(idx), _ptr(w))
    _check(rc, "topk_gate")
    return idx, w


def token_map(topk_idx, num_experts):
    """Returns (counts int32[E], offsets int32[E+1], pos int32[T,K], row_token int32[T*K])."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    counts = np.empty(num_experts, np.int32)
    offsets = np.empty(num_experts + 1, np.int32)
    pos = np.empty((T, K), np.int32)
    row_token = np.empty(T * K, np.int32)
    rc = _load().oracle_token_map(_ptr(topk_idx), T, K, num_experts, _ptr(counts),
                                  _ptr(offsets), _ptr(pos), _ptr(row_token))
    _check(rc, "token_map")
    return counts, offsets, pos, row_token


def expand_cast_fp8(x_bf16, pos=None, topk_weights=None, group_size=128, out=None):
    """x_bf16: uint16[T,H] bf16 bit patterns; pos: int32[T,K] or None (identity).

    Returns (out uint8[R,H], out_sf float32[R,G], out_w float32[R] or None).  Rows
    no copy lands in keep the content of ``out`` if given, else zero.
    """
    x_bf16 = _c(x_bf16, np.uint16)
    T, H = x_bf16.shape
    if pos is None:
        K, R = 1, T
    else:
        pos = _c(pos, np.int32)
        K = pos.shape[1]
        R = T * K
    G = H // group_size
    if out is None:
        out = (np.zeros((R, H), np.uint8), np.zeros((R, G), np.float32),
               np.zeros(R, np.float32) if topk_weights is not None else None)
    o_q, o_sf, o_w = out
    if topk_weights is not None:
        topk_weights = _c(topk_weights, np.float32)
    rc = _load().oracle_expand_cast_fp8(_ptr(x_bf16), T, H, K, _ptr(pos), _ptr(topk_weights),
                                        R, group_size, _ptr(o_q), _ptr(o_sf), _ptr(o_w))
    _check(rc, "expand_cast_fp8")
    return o_q, o_sf, o_w


def swiglu_cast_fp8(gate_up_bf16, row_weights=None, clamp_value=0.0, group_size=128):
    """gate_up_bf16: uint16[R, 2I] = [gate | up].  Returns (codes uint8[R,I], sf float32[R,I/group])."""
    gate_up_bf16 = _c(gate_up_bf16, np.uint16)
    R, two_i = gate_up_bf16.shape
    I = two_i // 2
    out = np.zeros((R, I), np.uint8)
    sf = np.zeros((R, I // group_size), np.float32)
    if row_weights is not None:
        row_weights = _c(row_weights, np.float32)
    rc = _load().oracle_swiglu_cast_fp8(_ptr(gate_up_bf16), R, I, _ptr(row_weights),
                                        float(clamp_value), group_size, _ptr(out), _ptr(sf))
    _check(rc, "swiglu_cast_fp8")
    return out, sf


def combine(y_rows_bf16, pos, weights=None):
    """y_rows_bf16: uint16[R,H] bf16 bits; pos: int32[T,K]; weights fp32[T,K] or None.
    Returns uint16[T,H] bf16 bits of sum_k w[t,k] * y_rows[pos[t,k]] (fp32, k order)."""
    y_rows_bf16 = _c(y_rows_bf16, np.uint16)
    pos = _c(pos, np.int32)
    R, H = y_rows_bf16.shape
    T, K = pos.shape
    out = np.empty((T, H), np.uint16)
    if weights is not None:
        weights = _c(weights, np.float32)
    rc = _load().oracle_combine(_ptr(y_rows_bf16), R, H, _ptr(pos), _ptr(weights), T, K, _ptr(out))
    _check(rc, "combine")
    return out


def f32_to_bf16(x):
    """bf16 bits (round to nearest even) of fp32 values, through the oracle's encoder."""
    lib = _load()
    x = np.asarray(x, np.float32)
    return np.array([lib.oracle_f32_to_bf16(float(v)) for v in x.ravel()], np.uint16).reshape(x.shape)


def padded_rows_bound(num_tokens, num_topk, num_local_experts, align):
    """Rows an aligned map can need: T*K copies plus < align padding per segment."""
    return num_tokens * num_topk + num_local_experts * (align - 1)


def token_map_aligned(topk_idx, expert_begin, expert_end, align, num_rows=None):
    """Returns (counts int32[EL], offsets int32[EL+1], pos int32[T,K], row_token int32[num_rows])."""
    topk_idx = _c(topk_idx, np.int64)
    T, K = topk_idx.shape
    EL = expert_end - expert_begin
    if num_rows is None:
        num_rows = padded_rows_bound(T, K, EL, align)
    counts = np.empty(EL, np.int32)
    offsets = np.empty(EL + 1, np.int32)
    pos = np.empty((T, K), np.int32)
    row_token = np.empty(num_rows, np.int32)
    rc = _load().oracle_token_map_aligned(_ptr(topk_idx), T, K, expert_begin, expert_end, align,
                                          _ptr(counts), _ptr(offsets), _ptr(pos), _ptr(row_token),
                                          num_rows)
    _check(rc, "token_map_aligned")
    return counts, offsets, pos, row_token


def expand_cast_fp8_padded(x_bf16, pos, row_token, topk_weights=None, group_size=128, out=None):
    """Expand into the rows of an aligned map; rows with row_token < 0 are zero-filled."""
    x_bf16 = _c(x_bf16, np.uint16)
    pos = _c(pos, np.int32)
    row_token = _c(row_token, np.int32)
    T, H = x_bf16.shape
    K = pos.shape[1]
    R = row_token.size
    G = H // group_size
    if out is None:
        out = (np.full((R, H), 0xA5, np.uint8), np.full((R, G), 7.0, np.float32),
               np.full(R, 7.0, np.float32) if topk_weights is not None else None)
    o_q, o_sf, o_w = out
    if topk_weights is not None:
        topk_weights = _c(topk_weights, np.float32)
    rc = _load().oracle_expand_cast_fp8_padded(_ptr(x_bf16), T, H, K, _ptr(pos), _ptr(topk_weights),
                                               _ptr(row_token), R, group_size, _ptr(o_q), _ptr(o_sf),
                                               _ptr(o_w))
    _check(rc, "expand_cast_fp8_padded")
    return o_q, o_sf, o_w


FMT_E4M3 = 0
FMT_E2M1 = 1
FMT_MAX = {FMT_E4M3: 448.0, FMT_E2M1: 6.0}


def e2m1_encode(x):
    """OCP FP4 e2m1 codes (uint8, low 4 bits) of fp32 values: nearest, ties to even code, saturating."""
    x = _c(x, np.float32)
    lib = _load()
    return np.array([lib.oracle_e2m1_encode(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def e2m1_decode(codes):
    codes = np.asarray(codes, np.uint8)
    lib = _load()
    return np.array([lib.oracle_e2m1_decode(int(c)) for c in codes.ravel()], np.float32).reshape(codes.shape)


def default_clamp(dtype):
    return float(_load().oracle_default_clamp(dtype))


def cast_group_fmt(v, dtype=FMT_E4M3, round_sf=False, clamp_min=0.0):
    """One group in any format: returns (codes uint8[n] (e2m1 in the low nibble), sf float32)."""
    v = _c(v, np.float32)
    q = np.empty(v.size, np.uint8)
    sf = np.empty(1, np.float32)
    _load().oracle_cast_group_fmt(_ptr(v), v.size, dtype, int(bool(round_sf)), float(clamp_min), _ptr(q), _ptr(sf))
    return q, sf[0]


def ue8m0_encode(pow2):
    return int(_load().oracle_ue8m0_encode(float(pow2)))


def ue8m0_decode(b):
    return float(_load().oracle_ue8m0_decode(int(b)))


def _fmt_out(rows, width, dtype, group_size, sf_ue8m0):
    row_bytes = width // 2 if dtype == FMT_E2M1 else width
    G = width // group_size
    return (np.zeros((rows, row_bytes), np.uint8),
            np.zeros((rows, G), np.uint8 if sf_ue8m0 else np.float32))


def expand_cast(x_bf16, pos=None, topk_weights=None, dtype=FMT_E4M3, group_size=128, round_sf=False,
                clamp_min=0.0, sf_ue8m0=False):
    """Expand + cast in any format.  Returns (out uint8[R, H or H/2], sf float32 or uint8 [R, H/group],
    out_w float32[R] or None)."""
    x_bf16 = _c(x_bf16, np.uint16)
    T, H = x_bf16.shape
    if pos is None:
        K, R = 1, T
    else:
        pos = _c(pos, np.int32)
        K = pos.shape[1]
        R = T * K
    out, sf = _fmt_out(R, H, dtype, group_size, sf_ue8m0)
    ow = None
    if topk_weights is not None:
        topk_weights = _c(topk_weights, np.float32)
        ow = np.zeros(R, np.float32)
    rc = _load().oracle_expand_cast(_ptr(x_bf16), T, H, K, _ptr(pos), _ptr(topk_weights), R, dtype, group_size,
                                    int(bool(round_sf)), float(clamp_min), int(bool(sf_ue8m0)), _ptr(out),
                                    _ptr(sf), _ptr(ow))
    _check(rc, "expand_cast")
    return out, sf, ow


def swiglu_cast(gate_up_bf16, row_weights=None, clamp_value=0.0, dtype=FMT_E4M3, group_size=128,
                round_sf=False, clamp_min=0.0, sf_ue8m0=False):
    """SwiGLU + cast in any format.  Returns (out uint8[R, I or I/2], sf float32 or uint8 [R, I/group])."""
    gate_up_bf16 = _c(gate_up_bf16, np.uint16)
    R, two_i = gate_up_bf16.shape
    inter = two_i // 2
    out, sf = _fmt_out(R, inter, dtype, group_size, sf_ue8m0)
    if row_weights is not None:
        row_weights = _c(row_weights, np.float32)
    rc = _load().oracle_swiglu_cast(_ptr(gate_up_bf16), R, inter, _ptr(row_weights), float(clamp_value), dtype,
                                    group_size, int(bool(round_sf)), float(clamp_min), int(bool(sf_ue8m0)),
                                    _ptr(out), _ptr(sf))
    _check(rc, "swiglu_cast")
    return out, sf


def unpack_e2m1(packed, width):
    """uint8[R, width/2] -> codes uint8[R, width] (element 2i from the low nibble of byte i)."""
    packed = np.asarray(packed, np.uint8)
    out = np.empty(packed.shape[:-1] + (width,), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out
