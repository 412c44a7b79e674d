"""CPU checks of the C ABI (no GPU needed, no kernel launched): the library
loads, exports every function include/moe_fp8.h declares, and rejects
invalid arguments on the host before any HIP call.  Also checks that the
product package never reaches into the oracle."""
import ctypes
import os
import re

import pytest

from moe_routing_fp8_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, WS_SMALL = 1, 2, 3
FAKE = 0x10000  # a non-null, 256-byte aligned address never dereferenced on the host


@pytest.fixture(scope="module")
def lib():
    return _native.lib()


def test_exports_every_declared_symbol(lib):
    names = _native.header_functions()
    assert set(names) >= {"moe_topk_gate", "moe_token_map", "moe_token_map_workspace_bytes",
                          "moe_expand_cast_fp8", "swiglu_cast_fp8", "moe_status_string",
                          "moe_last_hip_error", "moe_fp8_version"}
    raw = ctypes.CDLL(_native.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings_and_version(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.moe_status_string(99) == b"unknown status"
    assert lib.moe_fp8_version() >= 100
    assert lib.moe_last_hip_error() == 0


@pytest.mark.parametrize("args,want", [
    ((None, 4, 16, 2, 0, None, None, None), INVALID),          # null scores
    ((FAKE, 4, 0, 1, 0, FAKE, None, None), INVALID),           # E = 0
    ((FAKE, 4, 1025, 2, 0, FAKE, None, None), INVALID),        # E > 1024
    ((FAKE, 4, 16, 17, 0, FAKE, None, None), INVALID),         # K > E
    ((FAKE, 4, 64, 17, 0, FAKE, None, None), INVALID),         # K > 16
    ((FAKE, 4, 16, 0, 0, FAKE, None, None), INVALID),          # K = 0
    ((FAKE, -1, 16, 2, 0, FAKE, None, None), INVALID),         # T < 0
    ((FAKE, 4, 16, 2, 1, FAKE, None, None), INVALID),          # renormalize without weights
    ((FAKE, 4, 16, 2, 2, FAKE, FAKE, None), INVALID),          # renormalize not 0/1
    ((FAKE + 2, 4, 16, 2, 0, FAKE, None, None), INVALID),      # misaligned scores
    ((None, 0, 16, 2, 0, None, None, None), 0),                # T = 0: no-op
])
def test_topk_validation(lib, args, want):
    assert lib.moe_topk_gate(*args) == want


def test_token_map_validation(lib):
    f = lib.moe_token_map
    ws = lib.moe_token_map_workspace_bytes(1000, 8, 256)
    assert ws > 0 and ws % 256 == 0
    assert lib.moe_token_map_workspace_bytes(0, 8, 256) == 0
    assert lib.moe_token_map_workspace_bytes(10, 0, 256) == 0
    assert lib.moe_token_map_workspace_bytes(10, 8, 2000) == 0
    assert f(FAKE, 1000, 8, 256, None, FAKE, FAKE, None, FAKE, ws, None) == INVALID  # null counts
    assert f(FAKE, 1000, 8, 256, FAKE, FAKE, None, None, FAKE, ws, None) == INVALID  # null pos
    assert f(FAKE, 1000, 8, 256, FAKE, FAKE, FAKE, None, None, ws, None) == INVALID  # null ws
    assert f(FAKE, 1000, 8, 256, FAKE, FAKE, FAKE, None, FAKE + 4, ws, None) == INVALID  # ws align
    assert f(FAKE, 1000, 8, 256, FAKE, FAKE, FAKE, None, FAKE, ws - 256, None) == WS_SMALL
    assert f(FAKE, 1000, 0, 256, FAKE, FAKE, FAKE, None, FAKE, ws, None) == INVALID
    assert f(FAKE, 1000, 8, 1025, FAKE, FAKE, FAKE, None, FAKE, ws, None) == INVALID
    assert f(FAKE, 1 << 29, 8, 256, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == INVALID  # T*K > 2^31-1
    assert f(FAKE + 4, 1000, 8, 256, FAKE, FAKE, FAKE, None, FAKE, ws, None) == INVALID  # idx align


def test_expand_validation(lib):
    f = lib.moe_expand_cast_fp8
    # x, T, H, K, pos, w, R, group, out, sf, out_w, stream
    assert f(None, 8, 256, 2, FAKE, None, 16, 128, FAKE, FAKE, None, None) == INVALID
    assert f(FAKE, 8, 200, 2, FAKE, None, 16, 128, FAKE, FAKE, None, None) == INVALID  # H % group
    assert f(FAKE, 8, 256, 2, FAKE, None, 15, 128, FAKE, FAKE, None, None) == INVALID  # R != T*K
    assert f(FAKE, 8, 256, 2, None, None, 8, 128, FAKE, FAKE, None, None) == INVALID   # identity K != 1
    assert f(FAKE, 8, 256, 1, None, None, 9, 128, FAKE, FAKE, None, None) == INVALID   # identity R != T
    assert f(FAKE, 8, 256, 2, FAKE, FAKE, 16, 128, FAKE, FAKE, None, None) == INVALID  # w without out_w
    assert f(FAKE, 8, 256, 2, FAKE, None, 16, 128, FAKE, FAKE, FAKE, None) == INVALID  # out_w without w
    assert f(FAKE, 8, 256, 2, FAKE, None, 16, 64, FAKE, FAKE, None, None) == UNSUPPORTED  # group 64
    assert f(FAKE + 8, 8, 256, 2, FAKE, None, 16, 128, FAKE, FAKE, None, None) == INVALID  # x align
    assert f(FAKE, 8, 256, 2, FAKE, None, 16, 128, FAKE + 8, FAKE, None, None) == INVALID  # out align
    assert f(FAKE, 8, 256, 17, FAKE, None, 136, 128, FAKE, FAKE, None, None) == INVALID  # K > 16
    assert f(None, 0, 256, 2, None, None, 0, 128, None, None, None, None) == INVALID    # pos NULL, K=2
    assert f(None, 0, 256, 2, FAKE, None, 0, 128, None, None, None, None) == 0          # T = 0 no-op


def test_swiglu_validation(lib):
    f = lib.swiglu_cast_fp8
    # gu, R, I, w, clamp, group, out, sf, stream
    assert f(None, 8, 256, None, 0.0, 128, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 8, 200, None, 0.0, 128, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 8, 256, None, float("nan"), 128, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 8, 256, None, 0.0, 64, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, -1, 256, None, 0.0, 128, FAKE, FAKE, None) == INVALID
    assert f(FAKE + 2, 8, 256, None, 0.0, 128, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 8, 256, FAKE + 1, 0.0, 128, FAKE, FAKE, None) == INVALID
    assert f(None, 0, 256, None, 0.0, 128, None, None, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _native.lib()


def test_product_never_touches_oracle():
    pkg = os.path.join(ROOT, "moe_routing_fp8_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), fn
                assert "liboracle" not in text and "oracle.h" not in text, fn


def test_combine_validation(lib):
    f = lib.moe_combine
    # y, R, H, pos, w, T, K, out, stream
    assert f(FAKE, 16, 256, FAKE, None, 8, 2, None, None) == INVALID          # null out
    assert f(FAKE, 16, 256, None, None, 8, 2, FAKE, None) == INVALID          # null pos
    assert f(None, 16, 256, FAKE, None, 8, 2, FAKE, None) == INVALID          # null rows
    assert f(FAKE, 16, 100, FAKE, None, 8, 2, FAKE, None) == INVALID          # H % 8
    assert f(FAKE, 16, 256, FAKE, None, 8, 0, FAKE, None) == INVALID          # K = 0
    assert f(FAKE, 16, 256, FAKE, None, 8, 17, FAKE, None) == INVALID         # K > 16
    assert f(FAKE + 8, 16, 256, FAKE, None, 8, 2, FAKE, None) == INVALID      # rows align
    assert f(FAKE, 16, 256, FAKE, None, 8, 2, FAKE + 8, None) == INVALID      # out align
    assert f(FAKE, 16, 256, FAKE, FAKE + 2, 8, 2, FAKE, None) == INVALID      # weights align
    assert f(FAKE, -1, 256, FAKE, None, 8, 2, FAKE, None) == INVALID          # R < 0
    assert f(None, 0, 256, None, None, 0, 2, None, None) == 0                  # T = 0 no-op


def test_aligned_rows_bound(lib):
    f = lib.moe_token_map_aligned_rows
    assert f(1000, 8, 32, 128) == 1000 * 8 + 32 * 127
    assert f(1000, 8, 32, 1) == 8000
    assert f(0, 8, 32, 64) == 32 * 63
    assert f(-1, 8, 32, 1) == 0 and f(10, 0, 32, 1) == 0 and f(10, 17, 32, 1) == 0
    assert f(10, 8, 0, 1) == 0 and f(10, 8, 1025, 1) == 0
    assert f(10, 8, 32, 0) == 0 and f(10, 8, 32, 4097) == 0
    assert f(2 ** 28, 16, 4, 1) == 0  # above 2^31 - 1 rows


def test_token_map_aligned_validation(lib):
    f = lib.moe_token_map_aligned
    T, K, b, e, a = 1000, 8, 64, 96, 128
    R = lib.moe_token_map_aligned_rows(T, K, e - b, a)
    ws = lib.moe_token_map_workspace_bytes(T, K, e - b)
    # idx, T, K, begin, end, align, counts, offsets, pos, row_token, R, ws, ws_bytes, stream
    ok = [FAKE, T, K, b, e, a, FAKE, FAKE, FAKE, FAKE, R, FAKE, ws, None]

    def call(**kw):
        args = list(ok)
        names = ["idx", "T", "K", "b", "e", "a", "counts", "offsets", "pos", "rt", "R", "ws",
                 "wsb", "s"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(b=-1) == INVALID
    assert call(e=b) == INVALID                       # empty range
    assert call(b=0, e=1025) == INVALID               # > 1024 local experts
    assert call(a=0) == INVALID and call(a=4097) == INVALID
    assert call(K=0) == INVALID and call(K=17) == INVALID
    assert call(T=-1) == INVALID
    assert call(R=R - 1) == INVALID                   # below the worst case
    assert call(R=2 ** 31) == INVALID
    assert call(counts=None) == INVALID and call(offsets=None) == INVALID
    assert call(idx=None) == INVALID and call(pos=None) == INVALID
    assert call(idx=FAKE + 4) == INVALID and call(pos=FAKE + 2) == INVALID
    assert call(rt=FAKE + 2) == INVALID
    assert call(ws=None) == INVALID and call(ws=FAKE + 64) == INVALID
    assert call(wsb=ws - 1) == WS_SMALL


def test_expand_padded_validation(lib):
    f = lib.moe_expand_cast_fp8_padded
    # x, T, H, K, pos, w, row_token, R, group, out, sf, ow, stream
    ok = [FAKE, 64, 1024, 4, FAKE, None, FAKE, 512, 128, FAKE, FAKE, None, None]

    def call(i, v):
        args = list(ok)
        args[i] = v
        return f(*args)

    assert call(0, None) == INVALID              # null x
    assert call(4, None) == INVALID              # null pos with tokens
    assert call(6, None) == INVALID              # null row_token with rows
    assert call(9, None) == INVALID and call(10, None) == INVALID
    assert call(2, 1000) == INVALID              # H % group
    assert call(8, 64) == UNSUPPORTED            # group 64
    assert call(3, 17) == INVALID and call(3, 0) == INVALID
    assert call(7, -1) == INVALID
    assert call(5, FAKE) == INVALID              # weights without out_weights
    assert call(11, FAKE) == INVALID             # out_weights without weights
    assert call(0, FAKE + 2) == INVALID and call(9, FAKE + 4) == INVALID
    assert call(6, FAKE + 2) == INVALID
    assert f(None, 0, 1024, 4, None, None, None, 0, 128, None, None, None, None) == 0  # no-op


def test_dispatch_validation(lib):
    f = lib.moe_dispatch
    T, E, K, H = 64, 256, 8, 7168
    ws = lib.moe_dispatch_workspace_bytes(T, K, E)
    assert ws == lib.moe_route_workspace_bytes(T, K, E)
    assert lib.moe_dispatch_workspace_bytes(T, 0, E) == 0
    names = ["scores", "x", "T", "E", "K", "H", "renorm", "group", "idx", "w", "counts", "offsets", "pos",
             "rt", "out", "sf", "ow", "ws", "wsb", "mode", "s"]
    ok = [FAKE, FAKE, T, E, K, H, 0, 128, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, ws, 0,
          None]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(mode=5) == INVALID and call(mode=-1) == INVALID
    assert call(E=0) == INVALID and call(E=1025) == INVALID
    assert call(K=0) == INVALID and call(K=17) == INVALID and call(E=4, K=5) == INVALID
    assert call(renorm=1) == INVALID                  # renormalise without weights
    assert call(renorm=2, w=FAKE, ow=FAKE) == INVALID
    assert call(w=FAKE) == INVALID and call(ow=FAKE) == INVALID
    assert call(H=1000) == INVALID and call(group=64) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(counts=None) == INVALID and call(offsets=None) == INVALID
    assert call(scores=None) == INVALID and call(x=None) == INVALID and call(idx=None) == INVALID
    assert call(pos=None) == INVALID and call(out=None) == INVALID and call(sf=None) == INVALID
    assert call(x=FAKE + 8) == INVALID and call(out=FAKE + 8) == INVALID and call(idx=FAKE + 4) == INVALID
    assert call(scores=FAKE + 2) == INVALID
    assert call(ws=None) == INVALID and call(ws=FAKE + 64) == INVALID
    assert call(wsb=ws - 1) == WS_SMALL
    assert call(T=2049, mode=1, wsb=1 << 30) == UNSUPPORTED  # single launch: T*K <= 16384
    # the fused routing: at most 4096 workgroups of 16 tokens
    assert call(T=(1 << 16) + 1, mode=3, wsb=1 << 30) == UNSUPPORTED


def test_route_validation(lib):
    f = lib.moe_route
    T, E, K = 4096, 256, 8
    ws = lib.moe_route_workspace_bytes(T, K, E)
    # header, the fused form's two 64 x 1024 super-chunk tables, then the larger of the map's count table and
    # the fused form's per-workgroup rows (16 tokens per workgroup here)
    rows = -(-(-(-T // 16) * E * 4) // 256) * 256
    assert ws == lib.moe_dispatch_workspace_bytes(T, K, E) == 2048 + 524288 + max(
        lib.moe_token_map_workspace_bytes(T, K, E), rows)
    assert lib.moe_route_workspace_bytes(1 << 17, K, E) == 2048 + 524288 + lib.moe_token_map_workspace_bytes(
        1 << 17, K, E)  # 8192 workgroups: more than the fused form takes, no rows
    assert lib.moe_route_workspace_bytes(T, 0, E) == 0 and lib.moe_route_workspace_bytes(T, K, 1025) == 0
    names = ["scores", "T", "E", "K", "renorm", "idx", "w", "counts", "offsets", "pos", "rt", "ws", "wsb", "mode",
             "s"]
    ok = [FAKE, T, E, K, 0, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, ws, 0, None]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(mode=4) == INVALID and call(mode=-1) == INVALID
    # the local form: at most 32 tokens (refused before any launch)
    assert call(mode=3) == UNSUPPORTED and call(T=33, mode=3) == UNSUPPORTED
    assert call(E=0) == INVALID and call(E=1025) == INVALID
    assert call(K=0) == INVALID and call(K=17) == INVALID and call(E=4, K=5) == INVALID
    assert call(renorm=1) == INVALID and call(renorm=2, w=FAKE) == INVALID
    assert call(T=-1) == INVALID
    assert call(counts=None) == INVALID and call(offsets=None) == INVALID
    assert call(scores=None) == INVALID and call(idx=None) == INVALID and call(pos=None) == INVALID
    assert call(scores=FAKE + 2) == INVALID and call(idx=FAKE + 4) == INVALID and call(pos=FAKE + 2) == INVALID
    assert call(w=FAKE + 2) == INVALID and call(rt=FAKE + 2) == INVALID
    assert call(counts=FAKE + 2) == INVALID and call(offsets=FAKE + 1) == INVALID
    assert call(ws=None) == INVALID and call(ws=FAKE + 64) == INVALID
    assert call(wsb=ws - 1) == WS_SMALL
    # more than 4096 workgroups of 16 tokens: the fused form is unsupported
    assert call(T=(1 << 16) + 1, mode=1, wsb=1 << 30) == UNSUPPORTED


def _fmt(dtype=0, group=32, round_sf=1, ue8m0=1, clamp=0.0):
    return ctypes.byref(_native.moe_cast_format(dtype, group, round_sf, ue8m0, clamp))


def test_expand_cast_format_validation(lib):
    f = lib.moe_expand_cast
    # x, T, H, K, pos, w, R, fmt, out, sf, ow, stream
    def call(fmt, H=1024, out=FAKE, sf=FAKE, T=64, K=4, R=256, pos=FAKE):
        return f(FAKE, T, H, K, pos, None, R, fmt, out, sf, None, None)
    assert call(None) == INVALID                                # no format
    assert call(_fmt(dtype=2)) == INVALID
    assert call(_fmt(group=64)) == INVALID and call(_fmt(group=8)) == INVALID
    assert call(_fmt(round_sf=0, ue8m0=1)) == INVALID            # UE8M0 needs power-of-two scales
    assert call(_fmt(round_sf=2)) == INVALID
    assert call(_fmt(clamp=float("nan"))) == INVALID
    assert call(_fmt(dtype=1, clamp=1e-38)) == INVALID          # below 6 * 2^-126
    assert call(_fmt(clamp=1e38)) == INVALID                    # above 2^126
    assert call(_fmt(), H=1040) == INVALID                      # H % 32
    assert call(_fmt(dtype=0), out=FAKE + 8) == INVALID         # codes 16-byte aligned
    assert call(_fmt(dtype=1), out=FAKE + 8) == INVALID
    assert call(_fmt(dtype=1, group=16), H=1040) == UNSUPPORTED  # e2m1: 32 channels per lane
    assert call(_fmt(dtype=0, ue8m0=0), sf=FAKE + 2) == INVALID  # fp32 scales 4-byte aligned
    assert call(_fmt(), R=255) == INVALID                       # R != T*K
    assert call(_fmt(), pos=None) == INVALID                    # identity needs K = 1
    assert f(None, 0, 1024, 1, None, None, 0, _fmt(), None, None, None, None) == 0  # T = 0 identity


def test_swiglu_cast_format_validation(lib):
    f = lib.swiglu_cast
    def call(fmt, I=2048, out=FAKE, sf=FAKE, R=64, clamp=0.0):
        return f(FAKE, R, I, None, clamp, fmt, out, sf, None)
    assert call(None) == INVALID
    assert call(_fmt(group=48)) == INVALID
    assert call(_fmt(), I=2040) == INVALID
    assert call(_fmt(), clamp=float("nan")) == INVALID
    assert call(_fmt(dtype=1), out=FAKE + 2) == INVALID         # e2m1 codes 4-byte aligned
    assert call(_fmt(dtype=0), out=FAKE + 4) == INVALID         # e4m3 codes 8-byte aligned
    assert call(_fmt(), R=-1) == INVALID
    assert f(None, 0, 2048, None, 0.0, _fmt(), None, None, None) == 0


def test_check_validation(lib):
    """The input checks reject bad arguments on the host and treat T = 0 as a no-op."""
    s, i, p = lib.moe_check_scores, lib.moe_check_topk_idx, lib.moe_check_pos
    assert s(FAKE, 4, 16, 0, None, None) == INVALID             # null flags
    assert s(FAKE, 4, 16, 0, FAKE + 2, None) == INVALID         # misaligned flags
    assert s(None, 4, 16, 0, FAKE, None) == INVALID             # null scores
    assert s(FAKE + 2, 4, 16, 0, FAKE, None) == INVALID         # misaligned scores
    assert s(FAKE, -1, 16, 0, FAKE, None) == INVALID            # T < 0
    assert s(FAKE, 4, 1025, 0, FAKE, None) == INVALID           # E > 1024
    assert s(FAKE, 4, 16, 2, FAKE, None) == INVALID             # require_positive not 0/1
    assert s(None, 0, 16, 0, FAKE, None) == 0                   # T = 0: no-op
    assert i(FAKE, 4, 17, 64, FAKE, None) == INVALID            # K > 16
    assert i(FAKE, 4, 0, 64, FAKE, None) == INVALID             # K = 0
    assert i(FAKE, 4, 8, 0, FAKE, None) == INVALID              # E = 0
    assert i(FAKE + 4, 4, 8, 64, FAKE, None) == INVALID         # misaligned ids
    assert i(FAKE, 4, 8, 64, None, None) == INVALID             # null flags
    assert i(None, 0, 8, 64, FAKE, None) == 0                   # T = 0: no-op
    ws = lib.moe_check_pos_workspace_bytes(100)
    assert ws == 4 * 4 and lib.moe_check_pos_workspace_bytes(0) == 0 and lib.moe_check_pos_workspace_bytes(-5) == 0
    assert lib.moe_check_pos_workspace_bytes(32) == 4 and lib.moe_check_pos_workspace_bytes(33) == 8
    assert p(FAKE, 4, 8, 100, FAKE, ws - 1, FAKE, None) == WS_SMALL
    assert p(FAKE, 4, 8, 100, None, ws, FAKE, None) == INVALID  # null workspace
    assert p(FAKE, 4, 8, -1, FAKE, ws, FAKE, None) == INVALID   # num_rows < 0
    assert p(FAKE, 4, 17, 100, FAKE, ws, FAKE, None) == INVALID  # K > 16
    assert p(FAKE + 2, 4, 8, 100, FAKE, ws, FAKE, None) == INVALID  # misaligned pos
    assert p(FAKE, 4, 8, 100, FAKE, ws, None, None) == INVALID  # null flags
    assert p(None, 0, 8, 100, None, 0, FAKE, None) == 0         # T = 0: no-op


def test_activation_and_dispatch_check_validation(lib):
    """moe_check_activations and moe_check_dispatch reject bad arguments on the host (no kernel runs)."""
    a, d = lib.moe_check_activations, lib.moe_check_dispatch
    assert a(FAKE, 100, None, None) == INVALID                  # null flags
    assert a(FAKE, 100, FAKE + 2, None) == INVALID              # misaligned flags
    assert a(None, 100, FAKE, None) == INVALID                  # null values
    assert a(FAKE + 1, 100, FAKE, None) == INVALID              # misaligned bf16 values
    assert a(FAKE, -1, FAKE, None) == INVALID                   # negative count
    assert a(None, 0, FAKE, None) == 0                          # nothing to check: no-op
    assert d(FAKE, 2048, None, None) == INVALID                 # null flags
    assert d(None, 2048, FAKE, None) == INVALID                 # null workspace
    assert d(FAKE + 8, 2048, FAKE, None) == INVALID             # workspace not 256-byte aligned
    assert d(FAKE, 2047, FAKE, None) == WS_SMALL                # smaller than the barrier header


def test_check_flag_values_match_header():
    with open(_native.HEADER_PATH) as f:
        text = f.read()
    found = {int(v, 16): n for n, v in re.findall(r"#define (MOE_CHECK_[A-Z_]+) (0x[0-9a-fA-F]+)u", text)}
    assert found == _native.CHECK_FLAGS
