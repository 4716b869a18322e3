"""Parity of attnres_oproj_run (the fused o-projection + AttnRes, HIP gfx950)
with the FP64 oracle, on the three decode-step workloads and edge cases.

The o-projection output is the AttnRes delta (vLLM oproj.prepared page),
rounded to bf16 with -0.0 made +0.0 (gemm.ws_gemm page, positive_zero), so up
to 32 tokens the fused call must equal wsgemm_run followed by attnres_run bit
for bit. Beyond 32 tokens the fused call splits K over two workgroups, which
sums the projection in another order, so there the two agree up to rounding.
Against the oracle the FP32 accumulation of the GEMM may move a delta by one
bf16 ulp, so out and the new prefix are held to the derived bounds.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_tools import DEV, down, lib, up
from parity_tools import assert_fused_out_close, assert_new_prefix_close, bf16_to_f64

pytestmark = pytest.mark.gpu
POISON = 0x7FC1


def fused(s, *, final, write=None, has_delta=None, aux=True, ws=None):
    sga = lib()
    write = s.write if write is None else write
    has_delta = s.has_delta if has_delta is None else has_delta
    prefix, blocks = up(s.prefix), up(s.blocks)
    out = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    auxg = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV) if aux else None
    ws = sga.make_workspace(s.M, s.H, s.nb, DEV) if ws is None else ws
    sga.attnres_oproj_run(up(s.x), up(s.W), prefix, blocks, up(s.norm), up(s.query),
                          up(s.out_norm), out, auxg, ws, nb=s.nb, write=write,
                          has_delta=has_delta, final_boundary=final, eps=s.eps,
                          out_eps=s.out_eps)
    torch.cuda.synchronize()
    words = ws.cpu().numpy().view(np.uint32)
    assert np.all(words[:64] == 0), "workspace header not zero (a wait gave up)"
    assert np.all(words[64:] == 0x80000000), "mailbox not re-armed"
    return dict(out=down(out), prefix=down(prefix), blocks=down(blocks),
                aux=None if auxg is None else down(auxg))


def split(s, *, final, write=None, has_delta=None):
    """wsgemm_run then attnres_run on the same inputs (the unfused reading)."""
    sga = lib()
    write = s.write if write is None else write
    has_delta = s.has_delta if has_delta is None else has_delta
    y = torch.zeros((s.M, s.H), dtype=torch.int16, device=DEV)
    sga.wsgemm_run(up(s.x), up(s.W), y)
    prefix, blocks = up(s.prefix), up(s.blocks)
    out = torch.zeros((s.M, s.H), dtype=torch.int16, device=DEV)
    aux = torch.zeros((s.M, s.H), dtype=torch.int16, device=DEV)
    sga.attnres_run(y, prefix, blocks, up(s.norm), up(s.query), up(s.out_norm), out, aux,
                    nb=s.nb, write=write, has_delta=has_delta, final_boundary=final, eps=s.eps,
                    out_eps=s.out_eps)
    torch.cuda.synchronize()
    return dict(out=down(out), prefix=down(prefix), blocks=down(blocks), aux=down(aux), y=down(y))


def check(s, r, *, final, write=None, has_delta=None, aux=True, what=""):
    write = s.write if write is None else write
    has_delta = s.has_delta if has_delta is None else has_delta
    y = oracle.gemm(s.x, s.W, nthreads=16)
    ref = oracle.attnres(y, s.prefix, s.blocks, s.norm, s.query, s.out_norm, nb=s.nb,
                         write=write, has_delta=has_delta, final=final, eps=s.eps,
                         out_eps=s.out_eps, nthreads=16)
    h = ref.h_exact if not final or s.nb == 0 else bf16_to_f64(torch_round(ref.h_exact))
    scale = 1.0 / np.sqrt(np.mean(h * h, axis=-1) + np.float32(s.out_eps))
    assert_fused_out_close(r["out"], ref.out, r["prefix"], ref.prefix, ref.probs[:, s.nb], scale,
                           s.out_norm, final=final, what=f"{what} out")
    assert_new_prefix_close(r["prefix"], ref.prefix, s.prefix, has_delta, f"{what} prefix")
    if aux:
        assert np.array_equal(r["aux"], r["prefix"]), f"{what} aux != prefix"
    if write >= 0:
        assert np.array_equal(r["blocks"][:, write], r["prefix"]), f"{what} written slot"
    others = [b for b in range(s.blocks.shape[1]) if b != write]
    assert np.array_equal(r["blocks"][:, others], s.blocks[:, others]), f"{what} untouched slots"
    return ref


def torch_round(h):
    """float64 -> bfloat16 bits through torch (only to size the tolerance)."""
    return torch.tensor(h).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(scope="module")
def configs():
    return {c: synth.config_inputs(c) for c in (0, 1, 2)}


@pytest.mark.parametrize("final", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_fused_configs(configs, cfg, final):
    s = configs[cfg]
    r = fused(s, final=final)
    check(s, r, final=final, what=f"cfg{cfg} final={final}")


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_fused_equals_gemm_then_attnres(configs, cfg):
    s = configs[cfg]
    for final in (0, 1):
        a, b = fused(s, final=final), split(s, final=final)
        if s.M <= 32:
            for k in ("out", "prefix", "blocks", "aux"):
                assert np.array_equal(a[k], b[k]), f"cfg{cfg} final={final}: {k} differs"
        else:  # split K: the same values up to the FP32 summation order
            assert_new_prefix_close(a["prefix"], b["prefix"], s.prefix, s.has_delta,
                                    f"cfg{cfg} final={final} fused vs split prefix")
            assert np.array_equal(a["aux"], a["prefix"]) and np.array_equal(b["aux"], b["prefix"])


@pytest.mark.parametrize("M,K,H,nb,cap,write,has_delta", [
    (13, 1000, 1024, 3, 4, 3, 1),   # ragged tokens, ragged K, narrower rows
    (64, 256, 64, 2, 3, 1, 1),      # more owners than GEMM workgroups; write a scored slot
    (5, 520, 7168, 0, 1, 0, 0),     # nb = 0, delta path off (block-write layer)
    (17, 4096, 7168, 8, 8, 0, 0),   # overwrite a scored slot, no old prefix
    (1, 0, 7168, 1, 1, -1, 1),      # K = 0: delta = +0.0
    (64, 7168, 8192, 8, 9, 8, 1),   # widest rows
    (33, 1000, 1024, 3, 4, 3, 1),   # split K: ragged second half, 33 tokens
    (48, 264, 7168, 2, 3, -1, 1),   # split K: a second half of one k-step
    (40, 2056, 520, 1, 2, 1, 0),    # split K: ragged last row group
])
def test_fused_edges(M, K, H, nb, cap, write, has_delta):
    s = synth.decode_step(M, K, nb, H=H, cap=cap, write=write, has_delta=has_delta, seed=M + K)
    for final in (0, 1):
        r = fused(s, final=final, aux=(M % 2 == 1))
        check(s, r, final=final, aux=(M % 2 == 1), what=f"M={M} K={K} H={H} nb={nb}")


def test_fused_back_to_back_reuses_workspace():
    """Consecutive calls on one workspace: each call leaves the mailbox re-armed."""
    ws = lib().make_workspace(8, 7168, 4, DEV)
    for layer in range(3):
        s = synth.decode_step(8, 2048, 4, layer=layer, seed=5)
        r = fused(s, final=layer % 2, ws=ws)
        check(s, r, final=layer % 2, what=f"layer {layer}")


def test_fused_deterministic(configs):
    s = configs[2]
    a, b = fused(s, final=0), fused(s, final=0)
    for k in ("out", "prefix", "blocks"):
        assert np.array_equal(a[k], b[k]), k


def _fused_buffers(s, *, aux=True):
    sga = lib()
    b = dict(x=up(s.x), W=up(s.W), norm=up(s.norm), query=up(s.query), out_norm=up(s.out_norm),
             prefix=up(s.prefix), blocks=up(s.blocks),
             out=torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV),
             aux=torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV) if aux else None,
             ws=sga.make_workspace(s.M, s.H, s.nb, DEV))
    return b


def _fused_call(s, b, *, final, stream=None):
    lib().attnres_oproj_run(b["x"], b["W"], b["prefix"], b["blocks"], b["norm"], b["query"],
                            b["out_norm"], b["out"], b["aux"], b["ws"], nb=s.nb, write=s.write,
                            has_delta=s.has_delta, final_boundary=final, eps=s.eps,
                            out_eps=s.out_eps, stream=stream)


@pytest.mark.parametrize("cfg", [1, 2])
def test_fused_in_a_hip_graph(configs, cfg):
    """One call captured in a HIP graph and replayed three times, with eager
    restores of the in/out state between replays: every replay equals the
    eager call bit for bit and leaves the workspace re-armed."""
    s = configs[cfg]
    eager = fused(s, final=0)
    b = _fused_buffers(s)
    prefix0, blocks0 = b["prefix"].clone(), b["blocks"].clone()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            _fused_call(s, b, final=0)
    torch.cuda.synchronize()
    for rep in range(3):
        b["prefix"].copy_(prefix0)
        b["blocks"].copy_(blocks0)
        b["out"].fill_(POISON)
        b["aux"].fill_(POISON)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for k in ("out", "prefix", "blocks", "aux"):
            assert np.array_equal(down(b[k]), eager[k]), f"cfg{cfg} replay {rep}: {k}"
        words = b["ws"].cpu().numpy().view(np.uint32)
        assert np.all(words[:64] == 0) and np.all(words[64:] == 0x80000000), f"replay {rep}"


def test_fused_on_two_streams_at_once():
    """Two calls with their own workspaces on two streams, not synchronised
    with each other: each equals its own single-stream result."""
    sa = synth.decode_step(8, 4096, 4, seed=21)
    sb = synth.decode_step(64, 4096, 8, cap=9, write=8, seed=22)
    ea, eb = fused(sa, final=0), fused(sb, final=1)
    ba, bb = _fused_buffers(sa), _fused_buffers(sb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(2):  # the second round reuses the re-armed workspaces
        ba["prefix"].copy_(up(sa.prefix))
        bb["prefix"].copy_(up(sb.prefix))
        bb["blocks"].copy_(up(sb.blocks))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            _fused_call(sa, ba, final=0)
        with torch.cuda.stream(s2):
            _fused_call(sb, bb, final=1)
        torch.cuda.synchronize()
        for k in ("out", "prefix", "blocks", "aux"):
            assert np.array_equal(down(ba[k]), ea[k]), f"stream 1: {k}"
            assert np.array_equal(down(bb[k]), eb[k]), f"stream 2: {k}"
