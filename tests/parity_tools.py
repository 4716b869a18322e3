"""Comparison helpers shared by the parity tests. Every expected value comes
from the FP64 oracle; nothing here runs on the GPU.

Tolerance for bfloat16 outputs (an error bound derived from the arithmetic):
per element ``|gpu - ref| <= 2 ulp_bf16(max(|ref|, 2**-10 * rms(ref row)))``,
and per tensor ``||gpu - ref||_2 / ||ref||_2 <= 5e-3``. The floor of
``2**-10`` of the row RMS covers outputs near zero, where FP32 cancellation in
a 7168-wide mixture or a K-long dot product leaves an absolute error above two
ulps of a tiny value.

The fused o-projection + AttnRes step (``check_fused_step``) is held to that
same bar, in two parts:

* The new prefix ``bf16(prefix + Y)``. The GPU rounds an FP32-accumulated
  projection to the bfloat16 ``Y``; where the exact projection lies next to a
  bfloat16 rounding midpoint, the FP32 sum may land on the other side, so the
  GPU's ``Y`` may be a neighbour of the oracle's. The GPU's new prefix must
  therefore lie between ``bf16(prefix + Y - u)`` and ``bf16(prefix + Y + u)``
  with ``u = ulp_bf16(max(|Y|, 2**-10 rms(Y row)))`` (one ulp of Y; the
  floor covers a projection the dot product cancels to near zero, whose FP32
  accumulation error, about 1e-6 absolute, spans several of its tiny ulps),
  and at most 0.1% of its elements may differ from the oracle's new prefix.
* The output, given the GPU's own new prefix. AttnRes with the delta path off
  takes the delta itself as the new prefix (attn_res.kernel page,
  ClusterAttnRes.post), so the oracle's AttnRes with ``has_delta = 0`` on the
  GPU's new prefix and the launch-time saved blocks is the exact reference of
  everything after the projection: the output is held to the plain 2-ulp bar
  against it, and to the relative-L2 bar against the unconditional oracle.
"""
from __future__ import annotations

import numpy as np

import oracle

FLOOR = 2.0 ** -10


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def ulp_bf16(a: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at magnitude ``a`` (normal range)."""
    a = np.maximum(np.abs(a), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def row_rms(r: np.ndarray) -> np.ndarray:
    """RMS over the last axis, kept as a trailing axis of length 1."""
    return np.sqrt(np.mean(r * r, axis=-1, keepdims=True))


def compare_bf16(gpu_bits, ref_bits, *, ulps=2.0, rel_l2=5e-3, floor=FLOOR):
    """Returns (ok, report) for two bfloat16 tensors whose last axis is a row."""
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    if g.shape != r.shape:
        return False, f"shape {g.shape} != {r.shape}"
    if not np.isfinite(g).all():
        return False, "non-finite values in the GPU result"
    r2 = r.reshape(-1, r.shape[-1]) if r.ndim else r.reshape(1, 1)
    g2 = g.reshape(r2.shape)
    mag = np.maximum(np.abs(r2), floor * row_rms(r2))
    tol = ulps * ulp_bf16(mag)
    err = np.abs(g2 - r2)
    bad = err > tol
    l2 = np.linalg.norm(g2 - r2) / max(np.linalg.norm(r2), 1e-300)
    floored = int(np.count_nonzero(np.abs(r2) < floor * row_rms(r2)))
    exact = int(np.count_nonzero(np.asarray(gpu_bits) == np.asarray(ref_bits)))
    report = (f"n={err.size} bitexact={exact} max_err_ulps={np.max(err / ulp_bf16(mag)):.3g} "
              f"bad={int(bad.sum())} rel_l2={l2:.3g} floored={floored}")
    return (not bad.any()) and l2 <= rel_l2, report


def assert_bf16_close(gpu_bits, ref_bits, what="", **kw):
    ok, report = compare_bf16(gpu_bits, ref_bits, **kw)
    assert ok, f"{what}: {report}"
    return report


def assert_rel_l2(gpu_bits, ref_bits, what="", rel_l2=5e-3):
    g, r = bf16_to_f64(gpu_bits), bf16_to_f64(ref_bits)
    l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    assert np.isfinite(g).all() and l2 <= rel_l2, f"{what}: relative L2 {l2:.3g}"


def new_prefix_bounds(y_ref, old_prefix, has_delta):
    """The interval ``[bf16(prefix + Y - u), bf16(prefix + Y + u)]`` (as float64
    values) that a new prefix formed from a neighbour of the oracle's
    projection ``Y`` falls in (see the module comment). bf16() is the oracle's
    rounding of the exact float64 sum."""
    Y = bf16_to_f64(y_ref)
    u = ulp_bf16(np.maximum(np.abs(Y), FLOOR * row_rms(Y)))
    old = bf16_to_f64(old_prefix) if has_delta else np.zeros_like(Y)
    lo = bf16_to_f64(oracle.round_bf16_array(old + (Y - u)))
    hi = bf16_to_f64(oracle.round_bf16_array(old + (Y + u)))
    return lo, hi


def assert_new_prefix_flip(gpu_new, ref_new, old_prefix, y_ref, has_delta, what="",
                           max_frac=1e-3):
    """The fused call's new prefix: within one projection ulp of the oracle's
    (new_prefix_bounds), and equal to the oracle's on all but ``max_frac`` of
    the elements."""
    g = bf16_to_f64(gpu_new)
    lo, hi = new_prefix_bounds(y_ref, old_prefix, has_delta)
    bad = (g < lo) | (g > hi) | ~np.isfinite(g)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond one projection ulp"
    diff = np.asarray(gpu_new) != np.asarray(ref_new)
    assert diff.mean() <= max_frac, f"{what}: {int(diff.sum())} of {diff.size} elements differ"


def check_fused_step(*, x, W, old_prefix, blocks, norm, query, out_norm, nb, write, has_delta,
                     final, eps, out_eps, gpu_out, gpu_new, what="", nthreads=16):
    """Parity of one fused o-projection + AttnRes step with the oracle (see the
    module comment). ``blocks`` are the saved blocks at launch; returns the
    unconditional oracle result."""
    y = oracle.gemm(x, W, nthreads=nthreads)
    ref = oracle.attnres(y, old_prefix, blocks, norm, query, out_norm, nb=nb, write=write,
                         has_delta=has_delta, final=final, eps=eps, out_eps=out_eps,
                         nthreads=nthreads)
    assert_new_prefix_flip(gpu_new, ref.prefix, old_prefix, y, has_delta, f"{what} new prefix")
    given = oracle.attnres(gpu_new, old_prefix, blocks, norm, query, out_norm, nb=nb,
                           write=write, has_delta=0, final=final, eps=eps, out_eps=out_eps,
                           nthreads=nthreads)
    assert_bf16_close(gpu_out, given.out, f"{what} out (given the GPU's new prefix)")
    assert_rel_l2(gpu_out, ref.out, f"{what} out")
    ref.y = y
    return ref
