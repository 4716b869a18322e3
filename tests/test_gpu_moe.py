"""Parity of wsgemm_moe_front_run (HIP, gfx950) with the FP64 oracle.

WsGemm's MoE-front epilogue (vLLM gemm.ws_gemm page, module summary and
WsGemm.epilogue): output rows below `valid` (the router shard) are written as
FP32 words at bf16 column router_base + 2 (slot + row), rows from `split` on
(the latent shard) as bf16 at base + row - split, and the padding rows between
nowhere. Integer data make every FP32 sum exact, so there the bits equal the
oracle's; on normal data the router words are held to the FP32 accumulation
bound and the latent values to two bf16 ulps. Both shards come from the same
accumulators as wsgemm_run's y, so rounding a router word to bf16 gives y's
bits exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_tools import DEV, down, lib, up
from parity_tools import assert_bf16_close, bf16_to_f64

pytestmark = pytest.mark.gpu
POISON = 0x7FC1
rng = np.random.default_rng(99)


def bits_of(values):
    t = torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def run_moe(x, W, width, **kw):
    sga = lib()
    M = x.shape[0]
    out = torch.full((M, width), POISON, dtype=torch.int16, device=DEV)
    sga.wsgemm_moe_front_run(up(x), up(W), out, **kw)
    torch.cuda.synchronize()
    return down(out)


def router(out, router_base, slot, valid):
    cols = router_base + 2 * (slot + np.arange(valid))
    w = out[:, cols].astype(np.uint32) | (out[:, cols + 1].astype(np.uint32) << 16)
    return w


LAYOUTS = [
    # M, N, K, width, router_base, slot, base, valid, split
    (8, 4096, 7168, 7168, 3584, 0, 0, 384, 512),
    (3, 96, 200, 512, 256, 4, 8, 24, 40),
    (64, 1000, 1000, 2048, 1024, 12, 2, 0, 0),     # latent only
    (17, 264, 520, 1104, 560, 0, 0, 264, 264),     # router only
    (33, 7168, 256, 8448, 6144, 8, 0, 1024, 1536),
]


@pytest.mark.parametrize("M,N,K,width,rb,slot,base,valid,split", LAYOUTS)
def test_moe_front_exact_integers(M, N, K, width, rb, slot, base, valid, split):
    xi, wi = rng.integers(-8, 9, (M, K)), rng.integers(-8, 9, (N, K))
    x, W = bits_of(xi), bits_of(wi)
    kw = dict(router_base=rb, slot=slot, base=base, valid=valid, split=split)
    got = run_moe(x, W, width, **kw)
    ref = oracle.moe_front(x, W, np.full((M, width), POISON, np.uint16), **kw)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K,width,rb,slot,base,valid,split", LAYOUTS[:2] + LAYOUTS[4:])
def test_moe_front_normal_data(M, N, K, width, rb, slot, base, valid, split):
    x, W = synth.gemm_inputs(M, N, K, seed=M)
    kw = dict(router_base=rb, slot=slot, base=base, valid=valid, split=split)
    got = run_moe(x, W, width, **kw)
    ref = oracle.moe_front(x, W, np.full((M, width), POISON, np.uint16), **kw)
    # router: FP32 accumulation of K products, error <= (log2 K + 2) u sum |x w|
    g = router(got, rb, slot, valid).view(np.float32).astype(np.float64)
    r = router(ref, rb, slot, valid).view(np.float32).astype(np.float64)
    absum = np.abs(bf16_to_f64(x)) @ np.abs(bf16_to_f64(W[:valid])).T
    bound = (math.log2(K) + 2) * 2.0 ** -24 * absum + 2.0 ** -24 * np.abs(r)
    assert np.all(np.abs(g - r) <= bound), "router words beyond the FP32 bound"
    # latent: as wsgemm_run's output
    assert_bf16_close(got[:, base:base + N - split], ref[:, base:base + N - split], "latent")
    # padding rows and everything else untouched
    written = np.zeros(width, bool)
    written[rb + 2 * slot: rb + 2 * (slot + valid)] = True
    written[base: base + N - split] = True
    assert np.all(got[:, ~written] == POISON)


def test_moe_front_shares_wsgemm_accumulators():
    """Router words rounded to bf16, and the latent values, are wsgemm_run's y."""
    M, N, K = 8, 4096, 7168
    x, W = synth.gemm_inputs(M, N, K)
    kw = dict(router_base=3584, slot=0, base=0, valid=384, split=512)
    got = run_moe(x, W, 7168, **kw)
    y = torch.zeros((M, N), dtype=torch.int16, device=DEV)
    lib().wsgemm_run(up(x), up(W), y)
    torch.cuda.synchronize()
    y = down(y)
    w = router(got, 3584, 0, 384).view(np.float32)
    rb = torch.tensor(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rb = np.where(rb == 0x8000, 0, rb)
    assert np.array_equal(rb, y[:, :384])
    assert np.array_equal(got[:, 0:N - 512], y[:, 512:])
