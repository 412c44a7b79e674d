"""Comparison helpers for checking GPU outputs against the oracle (test
infrastructure only).

For the SwiGLU + e4m3 cast the GPU evaluates exp and the reciprocal with
hardware instructions, so its fp32 values differ from the oracle's IEEE
evaluation by a few ulp.  The agreed tolerance: every scale factor within
1e-6 relative, and every dequantised value (code * scale) within one e4m3
step of the oracle's, the step taken at the larger of the two code
magnitudes.  The two allowances compose: where a value sits at a rounding
tie, a scale one fp32 ulp away can send the code one step the other way,
so the dequantised bound is one step at the larger scale plus the code
magnitude times the (already bounded) scale difference.  The extra term is
at most 448e-6 of a scale, far below any step, so a code two steps away
still fails.
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
    mag = np.maximum(np.abs(cg), np.abs(cr))
    tol = (e4m3_step(mag) * np.maximum(sg, sr) + mag * np.abs(sg - sr)) * (1 + 2.0 ** -20)
    code_ok = diff <= tol
    details = {
        "max_sf_rel_err": float(sf_err.max()) if sf_err.size else 0.0,
        "codes_differing": int((q_gpu != q_ref).sum()),
        "codes_total": int(q_ref.size),
        "codes_out_of_tol": int((~code_ok).sum()),
    }
    ok = bool(np.all(sf_err <= sf_rtol) and np.all(code_ok))
    return ok, details


def e2m1_step(mag):
    """Spacing of e2m1 values at magnitude |mag| (grid units): 0.5 up to 2, 1 up to 4, 2 above."""
    mag = np.abs(np.asarray(mag, np.float64))
    return np.where(mag < 2.0, 0.5, np.where(mag < 4.0, 1.0, 2.0))


def _decode_fmt(q, dtype):
    from . import FMT_E2M1, unpack_e2m1
    q = np.asarray(q, np.uint8)
    if dtype == FMT_E2M1:
        codes = unpack_e2m1(q, q.shape[-1] * 2)
        lut = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)
        return lut[codes]
    return e4m3_decode(q).astype(np.float64)


def fmt_tolerance_report(q_gpu, sf_gpu, q_ref, sf_ref, dtype, group, sf_ue8m0=False, round_sf=False,
                         sf_rtol=1e-6):
    """SwiGLU tolerance in any block-scaled format: scales within sf_rtol
    relative, dequantised values within one step of the format at the larger
    of the two code magnitudes (scaled by the larger scale, plus the code
    magnitude times the scale difference where the scales agree).  With
    power-of-two scales a few-ulp difference in the amax can move a group's
    scale by a factor 2 when the amax sits at a binade edge; that is accepted
    only where the oracle's largest code of the group is at the edge (the
    format maximum, or half of it within one step)."""
    from . import FMT_MAX
    sg = np.asarray(sf_gpu)
    sr = np.asarray(sf_ref)
    if sf_ue8m0:
        sg = np.ldexp(1.0, sg.astype(np.int64) - 127)
        sr = np.ldexp(1.0, sr.astype(np.int64) - 127)
    sg = sg.astype(np.float64)
    sr = sr.astype(np.float64)
    cg = _decode_fmt(q_gpu, dtype)
    cr = _decode_fmt(q_ref, dtype)
    rel = np.abs(sg - sr) / np.abs(sr)
    sf_ok = rel <= sf_rtol
    if round_sf:
        maxv = FMT_MAX[dtype]
        step = e2m1_step if dtype == 1 else e4m3_step
        ref_top = np.abs(cr).reshape(cr.shape[0], -1, group).max(axis=2)
        at_edge = (ref_top >= maxv) | (np.abs(ref_top - maxv / 2) <= step(maxv / 2))
        flipped = ((sg == 2 * sr) | (sr == 2 * sg)) & at_edge
        sf_ok = sf_ok | flipped
    sgx = np.repeat(sg, group, axis=1)
    srx = np.repeat(sr, group, axis=1)
    stepf = e2m1_step if dtype == 1 else e4m3_step
    mag = np.maximum(np.abs(cg), np.abs(cr))
    # the scale difference carried by the code, only where the scales agree within sf_rtol (a flipped
    # power-of-two scale is judged on the step alone)
    close = np.repeat(rel <= sf_rtol, group, axis=1)
    tol = (stepf(mag) * np.maximum(sgx, srx) + np.where(close, mag * np.abs(sgx - srx), 0.0)) * (1 + 2.0 ** -20)
    code_ok = np.abs(cg * sgx - cr * srx) <= tol
    details = {"max_sf_rel_err": float(rel.max()) if rel.size else 0.0,
               "scales_differing": int((~(rel <= sf_rtol)).sum()),
               "codes_differing": int((np.asarray(q_gpu) != np.asarray(q_ref)).sum()),
               "codes_out_of_tol": int((~code_ok).sum())}
    return bool(np.all(sf_ok) and np.all(code_ok)), details
