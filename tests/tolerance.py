"""Acceptance checks of device results against the oracle's exact values.

Floating-point bar (bf16 outputs): |dev - exact| <= 2 ulp_bf16(exact) + 2^-20 * S,
where S is the magnitude sum of the terms that formed the element
(|r| + sum |c_p|, or |r| + sum g_j |E_j|) for the residual, and S*|w_h|*inv for
the read. The 2-ulp part is the bar for bf16 outputs; the S part bounds the
fp32 accumulation error of a sum of up to 17 terms ((n-1) 2^-24 S, with margin)
and only matters under cancellation, where a relative bound means nothing.

fp8 bar: codes equal except at most 0.1% of elements off by exactly one step in
the ordered list of e4m3 values (+0 and -0 are the same value), none further.
Per-token scale: relative error <= 1e-6 (about eight fp32 ulps; the scale is
max|y|/448 of fp32-accumulated y).
"""
from __future__ import annotations

import numpy as np
import torch

BF16_ULPS = 2.0
S_FACTOR = 2.0 ** -20
FP8_OFF_BY_ONE_FRACTION = 1e-3
SCALE_REL = 1e-6


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    u = np.exp2(e - 7.0)
    return np.where(a > 0, u, 2.0 ** -133)


def check_bf16(dev_bits: np.ndarray, exact: np.ndarray, s_term: np.ndarray, what: str) -> dict:
    dev = bf16_to_f64(dev_bits)
    err = np.abs(dev - exact)
    ulp = ulp_bf16(exact)
    bound = BF16_ULPS * ulp + S_FACTOR * np.abs(s_term)
    bad = ~(err <= bound)
    stats = {
        "what": what,
        "n": int(err.size),
        "max_err_ulp": float(np.max(err / ulp)) if err.size else 0.0,
        "over_half_ulp": int(np.count_nonzero(err > 0.5 * ulp)),
        "failures": int(np.count_nonzero(bad)),
    }
    if stats["failures"]:
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(
            f"{what}: {stats['failures']} of {err.size} elements outside tolerance; first at flat "
            f"index {i}: dev={dev.ravel()[i]!r} exact={exact.ravel()[i]!r} "
            f"bound={bound.ravel()[i]!r}")
    return stats


def e4m3_rank(codes: np.ndarray) -> np.ndarray:
    """Position of each code in the ordered list of finite e4m3 values (+0 == -0)."""
    c = np.asarray(codes, dtype=np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_fp8(dev_q: np.ndarray, ref_q: np.ndarray, what: str) -> dict:
    d = np.abs(e4m3_rank(dev_q) - e4m3_rank(ref_q))
    n_off1 = int(np.count_nonzero(d == 1))
    n_far = int(np.count_nonzero(d >= 2))
    nan_codes = int(np.count_nonzero((np.asarray(dev_q) & 0x7F) == 0x7F))
    stats = {"what": what, "n": int(d.size), "off_by_one": n_off1, "off_by_more": n_far,
             "nan_codes": nan_codes}
    if n_far or nan_codes or n_off1 > FP8_OFF_BY_ONE_FRACTION * d.size:
        raise AssertionError(f"{what}: fp8 codes outside tolerance: {stats}")
    return stats


def check_scale(dev: np.ndarray, ref: np.ndarray, what: str) -> dict:
    dev = np.asarray(dev, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    zero = ref == 0
    if np.any(dev[zero] != 0):
        raise AssertionError(f"{what}: nonzero scale where the oracle's is 0")
    rel = np.abs(dev[~zero] / ref[~zero] - 1.0)
    worst = float(rel.max()) if rel.size else 0.0
    if worst > SCALE_REL:
        raise AssertionError(f"{what}: scale relative error {worst:.3g} > {SCALE_REL:.3g}")
    return {"what": what, "max_rel": worst}


def read_s_term(x_exact: np.ndarray, mag: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """S*|w_h|*inv for the read's tolerance; x_exact, mag are [rows, H]."""
    inv = 1.0 / np.sqrt(np.mean(x_exact * x_exact, axis=1, keepdims=True) + float(np.float32(eps)))
    return mag * np.abs(np.asarray(w, np.float64))[None, :] * inv
