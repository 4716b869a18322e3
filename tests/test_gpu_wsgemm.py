"""Parity of wsgemm_run (HIP, gfx950) with the FP64 oracle.

WsGemm of the vLLM gemm.ws_gemm page: y = bf16(x W^T), FP32 accumulation,
-0.0 stored as +0.0 (positive_zero). Integer-valued operands make every
partial sum exact, so there the GPU must match the oracle bit for bit; on
normal data the bound is two bf16 ulps (floored at 2^-10 of the row RMS) and a
relative L2 error of 5e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_tools import DEV, down, lib, up
from parity_tools import assert_bf16_close

pytestmark = pytest.mark.gpu
rng = np.random.default_rng(2024)


def bits_of(values):
    t = torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def run_gemm(x, W, ldx=None, ldw=None, ldy=None):
    sga = lib()
    M, K = x.shape
    N = W.shape[0]
    ldx, ldw, ldy = ldx or K, ldw or K, ldy or N
    xp = np.zeros((M, ldx), np.uint16); xp[:, :K] = x
    wp = np.zeros((N, ldw), np.uint16); wp[:, :K] = W
    xg, wg = up(xp)[:, :K], up(wp)[:, :K]
    yg = torch.full((M, ldy), 0x7FC1, dtype=torch.int16, device=DEV)  # NaN poison
    sga.wsgemm_run(xg, wg, yg[:, :N])
    torch.cuda.synchronize()
    y = down(yg)
    assert np.all(y[:, N:] == 0x7FC1), "wrote past N"
    return y[:, :N]


@pytest.mark.parametrize("M", [1, 8, 16, 64])
def test_wsgemm_config4(M):
    """K = 7168, N = 4096: the standalone GEMM workload."""
    x, W = synth.gemm_inputs(M, 4096, 7168)
    y = run_gemm(x, W)
    ref = oracle.gemm(x, W, nthreads=16)
    assert_bf16_close(y, ref, f"wsgemm M={M}")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 7168), (8, 7168, 1024), (13, 1000, 1000),
                                   (16, 4096, 7168), (33, 264, 520), (64, 7168, 4096),
                                   (64, 8, 8), (5, 16384, 64), (17, 96, 1016), (49, 520, 24),
                                   (2, 7168, 1032), (31, 40, 8200),
                                   # the 16-row tile (N <= 4096, M <= 16), four-slot ring of
                                   # 512-element chunks: K below one chunk, a ragged third
                                   # chunk, more chunks than slots with a ragged tail
                                   (3, 40, 8), (9, 4096, 1048), (16, 256, 4104), (1, 4096, 2568)])
def test_wsgemm_exact_integers(M, N, K):
    xi = rng.integers(-8, 9, (M, K))
    wi = rng.integers(-8, 9, (N, K))
    x, W = bits_of(xi), bits_of(wi)
    y = run_gemm(x, W)
    assert np.array_equal(y, oracle.gemm(x, W, nthreads=16))


def test_wsgemm_zero_k_and_negative_zero():
    # K = 0: y = +0.0
    xg = torch.zeros((3, 8), dtype=torch.int16, device=DEV)
    wg = torch.zeros((64, 8), dtype=torch.int16, device=DEV)
    yg = torch.full((3, 64), 0x7FC1, dtype=torch.int16, device=DEV)
    lib().wsgemm_run(xg[:, :0], wg[:, :0], yg)
    torch.cuda.synchronize()
    assert np.all(down(yg) == 0)
    # tiny negative products round to -0.0 in bf16 and are stored as +0.0
    x = bits_of(np.full((2, 32), 2.0 ** -70))
    W = bits_of(np.full((16, 32), -(2.0 ** -70)))
    W[8:] = bits_of(np.full((8, 32), -1.0))
    x[1] = 0
    y = run_gemm(x, W)
    assert np.all(y[0, :8] == 0) and np.all(y[1] == 0)
    assert np.array_equal(y, oracle.gemm(x, W))


def test_wsgemm_padded_strides():
    x, W = synth.gemm_inputs(9, 1024, 2048, seed=3)
    y = run_gemm(x, W, ldx=2048 + 64, ldw=2048 + 8, ldy=1024 + 24)
    assert_bf16_close(y, oracle.gemm(x, W, nthreads=16), "padded strides")


def test_wsgemm_deterministic():
    x, W = synth.gemm_inputs(64, 4096, 7168, seed=9)
    a, b = run_gemm(x, W), run_gemm(x, W)
    assert np.array_equal(a, b)


# ---- wsgemm_run_ws: K split across workgroups beyond 32 tokens ------------------

def run_gemm_ws(x, W, ws=None, ldy=None):
    sga = lib()
    M, K = x.shape
    N = W.shape[0]
    ldy = ldy or N
    ws = sga.make_gemm_workspace(M, N, DEV) if ws is None else ws
    yg = torch.full((M, ldy), 0x7FC1, dtype=torch.int16, device=DEV)  # NaN poison
    sga.wsgemm_run_ws(up(x), up(W), yg[:, :N], ws)
    torch.cuda.synchronize()
    words = ws.cpu().numpy().view(np.uint32)
    assert np.all(words[:64] == 0), "workspace header not zero (a wait gave up)"
    assert np.all(words[64:] == 0x80000000), "hand-off not re-armed"
    y = down(yg)
    assert np.all(y[:, N:] == 0x7FC1), "wrote past N"
    return y[:, :N]


@pytest.mark.parametrize("M", [33, 48, 64])
def test_wsgemm_ws_config4(M):
    """K = 7168, N = 4096 (four-way split) beyond 32 tokens."""
    x, W = synth.gemm_inputs(M, 4096, 7168)
    y = run_gemm_ws(x, W)
    ref = oracle.gemm(x, W, nthreads=16)
    assert_bf16_close(y, ref, f"wsgemm_ws M={M}")


@pytest.mark.parametrize("M,N,K", [(64, 7168, 8192), (40, 1000, 1000), (33, 264, 520),
                                   (64, 8, 264), (48, 520, 24), (57, 16384, 256),
                                   (35, 7168, 1032), (64, 4096, 8200)])
def test_wsgemm_ws_exact_integers(M, N, K):
    """Integer operands: every split sums exactly, so the bits equal the oracle's."""
    xi = rng.integers(-8, 9, (M, K))
    wi = rng.integers(-8, 9, (N, K))
    x, W = bits_of(xi), bits_of(wi)
    y = run_gemm_ws(x, W, ldy=N + 8)
    assert np.array_equal(y, oracle.gemm(x, W, nthreads=16))


@pytest.mark.parametrize("M", [1, 8, 32])
def test_wsgemm_ws_up_to_32_tokens_is_wsgemm_run(M):
    x, W = synth.gemm_inputs(M, 4096, 7168)
    assert np.array_equal(run_gemm_ws(x, W), run_gemm(x, W))


def test_wsgemm_ws_reuses_its_workspace_and_is_deterministic():
    x, W = synth.gemm_inputs(64, 4096, 7168)
    ws = lib().make_gemm_workspace(64, 4096, DEV)
    a = run_gemm_ws(x, W, ws)
    b = run_gemm_ws(x, W, ws)
    x2, W2 = synth.gemm_inputs(40, 4096, 7168, seed=3)
    c = run_gemm_ws(x2, W2, ws)  # fewer tokens, same workspace
    assert np.array_equal(a, b)
    assert_bf16_close(c, oracle.gemm(x2, W2, nthreads=16), "reused workspace")


@pytest.mark.parametrize("M", [65, 96, 128])
def test_wsgemm_ws_beyond_64_tokens(M):
    """One pass over W for up to 128 tokens (K split four ways at N = 4096)."""
    x, W = synth.gemm_inputs(M, 4096, 7168, seed=M)
    y = run_gemm_ws(x, W)
    assert_bf16_close(y, oracle.gemm(x, W, nthreads=16), f"wsgemm_ws M={M}")


@pytest.mark.parametrize("M,N,K", [(128, 4096, 7168), (100, 1000, 1000), (128, 8, 264),
                                   (80, 7168, 520), (113, 264, 8200)])
def test_wsgemm_ws_beyond_64_tokens_exact_integers(M, N, K):
    xi = rng.integers(-8, 9, (M, K))
    wi = rng.integers(-8, 9, (N, K))
    x, W = bits_of(xi), bits_of(wi)
    y = run_gemm_ws(x, W, ldy=N + 8)
    assert np.array_equal(y, oracle.gemm(x, W, nthreads=16))
