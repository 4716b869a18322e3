"""Pins of the oracle's MoE-front epilogue of WsGemm (gemm.ws_gemm page,
WsGemm.epilogue): router rows as FP32 words at bf16 column
router_base + 2 (slot + row), latent rows as bf16 at base + row - split, the
padding rows between dropped, -0.0 stored as +0.0 in both. Checked against
numpy's exact integer products and float32 conversion, torch's bfloat16
conversion, and the layout rules themselves."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from parity_tools import bf16_to_f64

POISON = 0x7FC1
rng = np.random.default_rng(77)


def bits(values) -> np.ndarray:
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def router_words(out, router_base, slot, valid):
    """The FP32 values the router region of `out` holds, [M, valid]."""
    cols = router_base + 2 * (slot + np.arange(valid))
    lo = out[:, cols].astype(np.uint32)
    hi = out[:, cols + 1].astype(np.uint32)
    return (lo | (hi << 16)).view(np.float32), lo | (hi << 16)


def test_integer_data_against_numpy_and_torch():
    M, N, K = 5, 96, 200
    xi, wi = rng.integers(-8, 9, (M, K)), rng.integers(-8, 9, (N, K))
    x, W = bits(xi), bits(wi)
    width, rb, slot, base, valid, split = 512, 256, 4, 8, 24, 40
    out = oracle.moe_front(x, W, np.full((M, width), POISON, np.uint16), router_base=rb,
                           slot=slot, base=base, valid=valid, split=split)
    exact = xi @ wi.T  # int64, exact
    r, _ = router_words(out, rb, slot, valid)
    assert np.array_equal(r, exact[:, :valid].astype(np.float32))  # numpy's float32
    lat = torch.tensor(exact[:, split:], dtype=torch.float64).to(torch.bfloat16)
    lat = lat.view(torch.int16).numpy().view(np.uint16)
    lat = np.where(lat == 0x8000, 0, lat)
    assert np.array_equal(out[:, base:base + N - split], lat)
    # nothing else written: the router region, the latent region, poison elsewhere
    written = np.zeros(width, bool)
    written[rb + 2 * slot: rb + 2 * (slot + valid)] = True
    written[base: base + N - split] = True
    assert np.all(out[:, ~written] == POISON)


def test_normal_data_router_is_the_rounded_exact_sum():
    M, N, K = 3, 64, 1024
    x, W = synth.gemm_inputs(M, N, K, seed=4)
    out = oracle.moe_front(x, W, np.zeros((M, 256), np.uint16), router_base=128, slot=0,
                           base=0, valid=64, split=64)
    r, _ = router_words(out, 128, 0, 64)
    ref = bf16_to_f64(x) @ bf16_to_f64(W).T  # float64, off by far less than a float32 ulp
    f32 = ref.astype(np.float32)
    # away from float32 rounding midpoints the two roundings agree
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    q = np.exp2(e - 23)
    frac = a / q - np.floor(a / q)
    tie = np.abs(frac - 0.5) < 1e-6
    assert np.array_equal(r[~tie], f32[~tie]) and tie.mean() < 0.01


def test_negative_zero_becomes_positive_zero():
    M, N, K = 2, 16, 32
    x = bits(np.full((M, K), -0.0))  # every product is -0.0, every exact sum -0.0
    W = bits(np.ones((N, K)))
    out = oracle.moe_front(x, W, np.full((M, 64), POISON, np.uint16), router_base=32, slot=0,
                           base=0, valid=8, split=8)
    _, words = router_words(out, 32, 0, 8)
    assert np.all(words == 0)  # +0.0, not 0x80000000
    assert np.all(out[:, 0:8] == 0)  # latent -0.0 stored as +0.0


def test_latent_equals_the_plain_gemm_and_padding_is_dropped():
    M, N, K = 4, 48, 96
    x, W = synth.gemm_inputs(M, N, K, seed=9)
    y = oracle.gemm(x, W)
    out = oracle.moe_front(x, W, np.full((M, 128), POISON, np.uint16), router_base=64, slot=2,
                           base=16, valid=8, split=24)
    assert np.array_equal(out[:, 16:16 + 24], y[:, 24:])
    assert np.all(out[:, 0:16] == POISON) and np.all(out[:, 40:64 + 4] == POISON)
