"""Comparison helpers shared by the parity tests (no method arithmetic here).

Tolerance for bfloat16 outputs (an error bound derived from the arithmetic):
per element ``|gpu - ref| <= 2 ulp_bf16(max(|ref|, 2**-10 * rms(ref row)))``,
and per tensor ``||gpu - ref||_2 / ||ref||_2 <= 5e-3``. The floor of
``2**-10`` of the row RMS covers outputs near zero, where FP32 cancellation in
a 7168-wide mixture or a K-long dot product leaves an absolute error above two
ulps of a tiny value.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def ulp_bf16(a: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at magnitude ``a`` (normal range)."""
    a = np.maximum(np.abs(a), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def compare_bf16(gpu_bits, ref_bits, *, ulps=2.0, rel_l2=5e-3, floor=2.0 ** -10):
    """Returns (ok, report) for two bfloat16 tensors whose last axis is a row."""
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    if g.shape != r.shape:
        return False, f"shape {g.shape} != {r.shape}"
    if not np.isfinite(g).all():
        return False, "non-finite values in the GPU result"
    r2 = r.reshape(-1, r.shape[-1]) if r.ndim else r.reshape(1, 1)
    g2 = g.reshape(r2.shape)
    rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True))
    mag = np.maximum(np.abs(r2), floor * rms)
    tol = ulps * ulp_bf16(mag)
    err = np.abs(g2 - r2)
    bad = err > tol
    l2 = np.linalg.norm(g2 - r2) / max(np.linalg.norm(r2), 1e-300)
    floored = int(np.count_nonzero(np.abs(r2) < floor * rms))
    exact = int(np.count_nonzero(np.asarray(gpu_bits) == np.asarray(ref_bits)))
    report = (f"n={err.size} bitexact={exact} max_err_ulps={np.max(err / ulp_bf16(mag)):.3g} "
              f"bad={int(bad.sum())} rel_l2={l2:.3g} floored={floored}")
    return (not bad.any()) and l2 <= rel_l2, report


def assert_bf16_close(gpu_bits, ref_bits, what="", **kw):
    ok, report = compare_bf16(gpu_bits, ref_bits, **kw)
    assert ok, f"{what}: {report}"
    return report
