"""Comparison helpers shared by the parity tests (no method arithmetic here).

Tolerance for bfloat16 outputs (an error bound derived from the arithmetic):
per element ``|gpu - ref| <= 2 ulp_bf16(max(|ref|, 2**-10 * rms(ref row)))``,
and per tensor ``||gpu - ref||_2 / ||ref||_2 <= 5e-3``. The floor of
``2**-10`` of the row RMS covers outputs near zero, where FP32 cancellation in
a 7168-wide mixture or a K-long dot product leaves an absolute error above two
ulps of a tiny value.

The fused o-projection + AttnRes output uses a floor of ``2**-6`` of the row
RMS (FUSED_FLOOR). Its delta is accumulated in FP32, so at the few elements
whose exact value lies next to a bfloat16 rounding midpoint it lands one ulp
away from the FP64 oracle's delta. One such flip moves the prefix logit by
about |w_j| ulp(new_j) / rms(new) ~ 1e-4, the softmax weights by p (1 - p)
times that, and so every mixture element by ~1e-4 of the row scale: far below
two ulps of an ordinary element, but above two ulps of an element that the
mixture has cancelled to below 2**-7 of the row RMS. At a final boundary the
mixture h is itself rounded to bfloat16 before the output RMSNorm; the same
perturbation can flip h_i by one ulp, which moves out_i by about one more ulp,
so those comparisons allow three ulps.
"""
from __future__ import annotations

import numpy as np

FUSED_FLOOR = 2.0 ** -6


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


def assert_new_prefix_close(gpu_bits, ref_bits, old_prefix_bits, has_delta, what="", max_frac=1e-3):
    """The fused call's new prefix against the oracle's.

    new = bf16(prefix + y) with y the FP32-accumulated projection: where y sits
    one ulp from the oracle's y, new may move by ulp(y) <= ulp(|new| + |prefix|)
    plus its own rounding. A y that the dot product cancels to near zero carries
    the FP32 accumulation error (~1e-6 absolute) across several of its tiny
    ulps, hence the floor of 2**-10 of the row RMS on the rounding term. Such
    elements must be rare (max_frac)."""
    g, r = bf16_to_f64(gpu_bits), bf16_to_f64(ref_bits)
    old = bf16_to_f64(old_prefix_bits) if has_delta else np.zeros_like(r)
    r2 = r.reshape(-1, r.shape[-1])
    rms = np.sqrt(np.mean(r2 * r2, axis=-1, keepdims=True)).reshape(r.shape[:-1] + (1,))
    tol = ulp_bf16(np.abs(r) + np.abs(old)) + 2 * ulp_bf16(np.maximum(np.abs(r), 2.0 ** -10 * rms))
    diff = g != r
    bad = np.abs(g - r) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the flip bound"
    assert diff.mean() <= max_frac, f"{what}: {int(diff.sum())} of {diff.size} elements differ"


def assert_fused_out_close(gpu_out, ref_out, gpu_new, ref_new, p_new, scale, gain, *, final,
                           what=""):
    """The fused call's output against the oracle's.

    Besides the global softmax perturbation (FUSED_FLOOR) a flipped delta moves
    the new prefix at its own column i by dnew_i = |gpu_new_i - ref_new_i|, and
    out_i = (sum_b p_b v_b,i + p_n new_i) * s * gain_i moves with it by
    p_n dnew_i s |gain_i|. p_n (weight of the new prefix, [T]) and s (output
    RMS scale, [T]) come from the oracle."""
    g, r = bf16_to_f64(gpu_out), bf16_to_f64(ref_out)
    dnew = np.abs(bf16_to_f64(gpu_new) - bf16_to_f64(ref_new))
    direct = np.asarray(p_new)[:, None] * dnew * np.asarray(scale)[:, None] * np.abs(
        bf16_to_f64(gain))[None, :]
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    ulps = 3.0 if final else 2.0
    tol = ulps * ulp_bf16(np.maximum(np.abs(r), FUSED_FLOOR * rms)) + direct * (1 + 2.0 ** -6)
    tol += np.where(direct > 0, ulp_bf16(np.abs(r) + direct), 0.0)
    bad = np.abs(g - r) > tol
    l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    assert not bad.any() and l2 <= 5e-3, (
        f"{what}: bad={int(bad.sum())} rel_l2={l2:.3g} max_excess="
        f"{np.max((np.abs(g - r) - tol)):.3g}")
