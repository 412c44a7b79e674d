"""Comparison helpers for checking GPU outputs against the oracle (test
infrastructure only).

For the SwiGLU + e4m3 cast the GPU evaluates exp and the reciprocal with
hardware instructions, so its fp32 values differ from the oracle's IEEE
evaluation by a few ulp.  The agreed tolerance: every scale factor within
1e-6 relative, and every dequantised value (code * scale) within one e4m3
step of the oracle's, the step taken at the larger of the two code
magnitudes.
"""
import numpy as np

from . import e4m3_decode


def e4m3_step(mag):
    """Spacing of e4m3 values at magnitude |mag| (grid units, not scaled)."""
    mag = np.abs(np.asarray(mag, np.float64))
    return np.where(mag < 2.0 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3))


def swiglu_tolerance_report(q_gpu, sf_gpu, q_ref, sf_ref, group=128, sf_rtol=1e-6):
    """Returns (ok, details) for codes uint8 [R, I] and scales fp32 [R, I/group]."""
    q_gpu = np.asarray(q_gpu, np.uint8)
    q_ref = np.asarray(q_ref, np.uint8)
    sf_gpu = np.asarray(sf_gpu, np.float32)
    sf_ref = np.asarray(sf_ref, np.float32)
    sf_err = np.abs(sf_gpu.astype(np.float64) - sf_ref) / np.abs(sf_ref.astype(np.float64))
    cg = e4m3_decode(q_gpu).astype(np.float64)
    cr = e4m3_decode(q_ref).astype(np.float64)
    sg = np.repeat(sf_gpu.astype(np.float64), group, axis=1)
    sr = np.repeat(sf_ref.astype(np.float64), group, axis=1)
    diff = np.abs(cg * sg - cr * sr)
    tol = e4m3_step(np.maximum(np.abs(cg), np.abs(cr))) * np.maximum(sg, sr) * (1 + 2.0 ** -20)
    code_ok = diff <= tol
    details = {
        "max_sf_rel_err": float(sf_err.max()) if sf_err.size else 0.0,
        "codes_differing": int((q_gpu != q_ref).sum()),
        "codes_total": int(q_ref.size),
        "codes_out_of_tol": int((~code_ok).sum()),
    }
    ok = bool(np.all(sf_err <= sf_rtol) and np.all(code_ok))
    return ok, details
