"""attnres_oproj_run_noalloc (the fused step on the library's own workspace,
for callers that cannot allocate) through the C ABI, HIP gfx950: its outputs
equal attnres_oproj_run's with a caller workspace, bit for bit, over calls in
a row on the shared array, each later call smaller than the one before."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_tools import DEV, down, lib, up

pytestmark = pytest.mark.gpu
POISON = 0x7FC1


def _run(s, *, noalloc, final):
    sga = lib()
    prefix, blocks = up(s.prefix), up(s.blocks)
    out = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    aux = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    args = (up(s.x), up(s.W), prefix, blocks, up(s.norm), up(s.query), up(s.out_norm), out, aux)
    kw = dict(nb=s.nb, write=s.write, has_delta=s.has_delta, final_boundary=final, eps=s.eps,
              out_eps=s.out_eps)
    if noalloc:
        sga.attnres_oproj_run_noalloc(*args, **kw)
        assert sga.attnres_workspace_status(None) == 0, "a wait gave up on the library's array"
    else:
        ws = sga.make_workspace(s.M, s.H, s.nb, DEV)
        sga.attnres_oproj_run(*args, ws, **kw)
        assert sga.attnres_workspace_status(ws) == 0
    torch.cuda.synchronize()
    return {k: down(v) for k, v in (("out", out), ("prefix", prefix), ("blocks", blocks),
                                    ("aux", aux))}


def test_noalloc_equals_caller_workspace_calls_in_a_row():
    """Largest first (64 tokens, split K, block write), then smaller ones:
    every call finds the array armed by the one before."""
    cases = [synth.decode_step(64, 2048, 8, cap=9, write=8, seed=81),
             synth.decode_step(40, 1024, 5, cap=6, write=2, has_delta=0, seed=82),
             synth.decode_step(8, 4096, 4, seed=83),
             synth.decode_step(1, 1024, 1, seed=84)]
    for i, s in enumerate(cases):
        final = i % 2
        a = _run(s, noalloc=True, final=final)
        b = _run(s, noalloc=False, final=final)
        for k in ("out", "prefix", "blocks", "aux"):
            assert np.array_equal(a[k], b[k]), f"call {i} (M={s.M}): {k} differs"
