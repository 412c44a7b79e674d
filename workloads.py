"""Seeded synthetic inputs for the five workloads (host numpy arrays).

This module holds no arithmetic of the dispatch method: it only draws the
inputs (scores, activations, routing weights) that the GPU library and the
CPU oracle both consume.  Every array comes from
``numpy.random.default_rng([seed, stream])`` so each input has its own
stream and a fixed seed per workload.

Streams: 0 scores/logits, 1 x, 2 expert bias, 3 outlier mask,
4 routing weights, 5 gate/up.

bf16 arrays are returned as uint16 bit patterns, rounded to nearest even
from fp32.

Workloads (shapes from the MoE routing and quantisation sections of the
TileKernels article and the DeepSeek-V3 layer shape: hidden 7168, 256
experts, top-8):
  tiny    T=64,    E=16,  K=2, H=256;   SwiGLU [64, 2x128], weights U(0,1)
  mid     T=1024,  E=256, K=8, H=4096   (scores N(0,1); x N(0,1))
  dsv3    T=4096,  E=256, K=8, H=7168   sigmoid scores, renormalised top-k
                                        weights; x N(0,1) with 1% outliers x50
  swiglu  R=8192,  I=2048               gate/up N(0,1); weights U(0,1)
  large   T=32768, E=256, K=8, H=7168   scores N(0,1) + ln(Zipf(1.2)) per-expert
                                        bias (skewed load, many empty experts)
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_tokens: int = 0
    num_experts: int = 0
    num_topk: int = 0
    hidden: int = 0
    renormalize: bool = False
    scores: str = "normal"  # "normal" | "sigmoid" | "zipf_bias"
    outliers: bool = False
    swiglu_rows: int = 0
    swiglu_inter: int = 0
    swiglu_weights: bool = False
    group_size: int = 128


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 16, 2, 256, swiglu_rows=64, swiglu_inter=128,
                     swiglu_weights=True),
    "mid": Workload("mid", 2, 1024, 256, 8, 4096),
    "dsv3": Workload("dsv3", 3, 4096, 256, 8, 7168, renormalize=True, scores="sigmoid",
                     outliers=True),
    "swiglu": Workload("swiglu", 4, swiglu_rows=8192, swiglu_inter=2048, swiglu_weights=True),
    "large": Workload("large", 5, 32768, 256, 8, 7168, scores="zipf_bias"),
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def f32_to_bf16_bits(a: np.ndarray, chunk: int = 1 << 22) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs: the
    uint32 sum cannot wrap below the NaN patterns)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat_in = a.reshape(-1).view(np.uint32)
    out = np.empty(flat_in.size, np.uint16)
    for s in range(0, flat_in.size, chunk):
        u = flat_in[s:s + chunk]
        r = (u >> 16) & 1
        r += u
        r += 0x7FFF
        r >>= 16
        out[s:s + chunk] = r
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_scores(w: Workload, num_tokens: Optional[int] = None) -> np.ndarray:
    """fp32 [T, E] router scores.  ``num_tokens`` draws only the first rows
    (same values as the full draw for normal/sigmoid/zipf_bias)."""
    T = w.num_tokens if num_tokens is None else num_tokens
    z = _rng(w.seed, 0).standard_normal((T, w.num_experts), dtype=np.float32)
    if w.scores == "normal":
        return z
    if w.scores == "sigmoid":
        return (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)
    if w.scores == "zipf_bias":
        draws = _rng(w.seed, 2).zipf(1.2, w.num_experts)
        bias = np.log(draws.astype(np.float64)).astype(np.float32)
        return (z + bias[None, :]).astype(np.float32)
    raise ValueError(w.scores)


def make_x(w: Workload, num_tokens: Optional[int] = None) -> np.ndarray:
    """bf16 bits [T, H] token activations, N(0,1) (x50 on a 1% outlier mask)."""
    T = w.num_tokens if num_tokens is None else num_tokens
    x = _rng(w.seed, 1).standard_normal((T, w.hidden), dtype=np.float32)
    if w.outliers:
        mask = _rng(w.seed, 3).random((T, w.hidden), dtype=np.float32) < 0.01
        x[mask] *= np.float32(50.0)
    return f32_to_bf16_bits(x)


def make_gate_up(w: Workload, rows: Optional[int] = None, inter: Optional[int] = None,
                 chunk_rows: int = 16384) -> np.ndarray:
    """bf16 bits [R, 2I] = [gate | up], N(0,1).

    ``rows``/``inter`` default to the workload's SwiGLU shape; a dispatch
    workload passes its routed-row count (T*K) to get the SwiGLU input of the
    whole batch.  Drawn in row chunks from one stream (same values as a
    single draw)."""
    R = w.swiglu_rows if rows is None else rows
    I = w.swiglu_inter if inter is None else inter
    rng = _rng(w.seed, 5)
    out = np.empty((R, 2 * I), np.uint16)
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        out[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, 2 * I), dtype=np.float32))
    return out


def make_row_weights(w: Workload, rows: Optional[int] = None) -> Optional[np.ndarray]:
    """fp32 [R] routing weights U[0,1) for the SwiGLU rows, or None."""
    if rows is None:
        if not w.swiglu_weights:
            return None
        rows = w.swiglu_rows
    return _rng(w.seed, 4).random(rows, dtype=np.float32)


def sha256_hex(a: np.ndarray) -> str:
    """SHA-256 of an input array: its dtype, its shape and its bytes (C order)."""
    import hashlib

    a = np.ascontiguousarray(a)
    h = hashlib.sha256()
    h.update(f"{a.dtype.str}{a.shape}".encode())
    h.update(memoryview(a).cast("B"))
    return h.hexdigest()


def input_arrays(name: str):
    """(input name, array) pairs of a workload as the tests and the bench draw
    them: scores, x, gate_up and row weights where the workload has them.  The
    large workload's gate_up is its first 16384 routed rows (one draw chunk)."""
    w = WORKLOADS[name]
    out = []
    if w.num_tokens:
        out.append(("scores", make_scores(w)))
        out.append(("x", make_x(w)))
    if w.swiglu_rows:
        out.append(("gate_up", make_gate_up(w)))
        rw = make_row_weights(w)
        if rw is not None:
            out.append(("row_weights", rw))
    elif name == "large":  # the step's SwiGLU input is drawn from this workload's stream
        out.append(("gate_up", make_gate_up(w, rows=16384, inter=2048)))
    return out
