"""The prepared (tile-major) W layout and the fused step on it, HIP gfx950.

attnres_pack_weights writes W [N, K] as 4 ceil(K / 512) planes of 128
k-values: plane j holds every row's k-values [128 j, 128 j + 128) as one
256-byte segment, rows in order, with the 16-byte piece p of row n at
position p ^ (n & 15) and zeros past K (the weight is prepared once, as
PreparedOproj binds it on the oproj.prepared page). The layout is checked
element by element against that definition written out in numpy; the fused
step on the prepared W must give attnres_oproj_run's bits on the row-major W
(the same operands reach the same matrix-core instructions in the same
order; up to 32 tokens, since beyond that the row-major call rotates the K
order of each workgroup and the prepared one does not) and the oracle's
values at the fused-step bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_tools import DEV, down, lib, up
from parity_tools import check_fused_step

pytestmark = pytest.mark.gpu
POISON = 0x7FC1


def packed_reference(W, K):
    """The documented layout, element by element (numpy)."""
    N = W.shape[0]
    P = 4 * ((K + 511) // 512)
    Wz = np.zeros((N, P * 128), np.uint16)
    Wz[:, :K] = W[:, :K]
    out = np.zeros((P, N, 16, 8), np.uint16)
    for n in range(N):
        for j in range(16):
            p = j ^ (n & 15)
            out[:, n, j, :] = Wz[n].reshape(P, 16, 8)[:, p, :]
    return out.reshape(-1)


@pytest.mark.parametrize("N,K,pad", [(40, 1000, 24), (16, 8, 0), (7168, 4096, 0), (33, 520, 8)])
def test_pack_layout(N, K, pad):
    sga = lib()
    W = synth.normal_bf16(5, 2, N + K, (N, K))
    Wg = torch.full((N, K + pad), POISON, dtype=torch.int16, device=DEV)
    Wg[:, :K] = up(W)
    nbytes = sga.attnres_packed_weights_size(N, K)
    Wp = torch.full((nbytes // 2 + 64,), POISON, dtype=torch.int16, device=DEV)
    sga.attnres_pack_weights(Wg[:, :K], Wp)
    torch.cuda.synchronize()
    got = down(Wp)
    assert np.array_equal(got[:nbytes // 2], packed_reference(W, K)), "packed layout"
    assert np.all(got[nbytes // 2:] == POISON), "wrote past the packed size"


def _run(s, *, packed, final, write=None, has_delta=None):
    sga = lib()
    write = s.write if write is None else write
    has_delta = s.has_delta if has_delta is None else has_delta
    prefix, blocks = up(s.prefix), up(s.blocks)
    out = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    aux = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    ws = sga.make_workspace(s.M, s.H, s.nb, DEV)
    kw = dict(nb=s.nb, write=write, has_delta=has_delta, final_boundary=final, eps=s.eps,
              out_eps=s.out_eps)
    Wg = up(s.W)
    if packed:
        Wp = sga.attnres_pack_weights(Wg)
        sga.attnres_oproj_packed_run(up(s.x), Wp, s.H, prefix, blocks, up(s.norm), up(s.query),
                                     up(s.out_norm), out, aux, ws, **kw)
    else:
        sga.attnres_oproj_run(up(s.x), Wg, prefix, blocks, up(s.norm), up(s.query),
                              up(s.out_norm), out, aux, ws, **kw)
    assert sga.attnres_workspace_status(ws) == 0
    torch.cuda.synchronize()
    return {k: down(v) for k, v in (("out", out), ("prefix", prefix), ("blocks", blocks),
                                    ("aux", aux))}


@pytest.fixture(scope="module")
def configs():
    return {c: synth.config_inputs(c) for c in (0, 1, 2)}


@pytest.mark.parametrize("final", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_packed_equals_row_major_and_oracle(configs, cfg, final):
    s = configs[cfg]
    a = _run(s, packed=True, final=final)
    if s.M <= 32:
        b = _run(s, packed=False, final=final)
        for k in ("out", "prefix", "blocks", "aux"):
            assert np.array_equal(a[k], b[k]), f"cfg{cfg} final={final}: {k} differs"
    assert np.array_equal(a["aux"], a["prefix"])
    if s.write >= 0:
        assert np.array_equal(a["blocks"][:, s.write], a["prefix"])
    check_fused_step(x=s.x, W=s.W, old_prefix=s.prefix, blocks=s.blocks, norm=s.norm,
                     query=s.query, out_norm=s.out_norm, nb=s.nb, write=s.write,
                     has_delta=s.has_delta, final=final, eps=s.eps, out_eps=s.out_eps,
                     gpu_out=a["out"], gpu_new=a["prefix"], what=f"packed cfg{cfg}")


@pytest.mark.parametrize("M,K,H,nb,cap,write,has_delta", [
    (13, 1000, 1024, 3, 4, 3, 1),   # ragged K (zero-padded planes), narrower rows
    (8, 1000, 5008, 2, 3, -1, 1),   # 22-row groups: second row tile partly filled, ragged last group
    (8, 1000, 7000, 2, 3, 1, 1),    # prepared W: 32-row groups, last one 24 rows; row-major: 30 rows, last 10
    (40, 1000, 1024, 3, 4, 1, 1),   # split K, ragged second half
    (48, 264, 7168, 2, 3, -1, 0),   # split K, a second half of one k-step
    (1, 8, 7168, 1, 1, -1, 1),      # K of one piece
    (24, 2056, 520, 2, 3, 2, 1),    # two token tiles, ragged last row group
    (8, 32760, 512, 2, 3, -1, 1),   # long K: 256 planes, the last zero-padded
    (40, 32760, 512, 2, 3, 2, 1),   # split K over long rows
])
def test_packed_edges(M, K, H, nb, cap, write, has_delta):
    s = synth.decode_step(M, K, nb, H=H, cap=cap, write=write, has_delta=has_delta,
                          seed=500 + M + K)
    a = _run(s, packed=True, final=0)
    if M <= 32:
        b = _run(s, packed=False, final=0)
        for k in ("out", "prefix", "blocks", "aux"):
            assert np.array_equal(a[k], b[k]), f"M={M} K={K} H={H}: {k} differs"
    check_fused_step(x=s.x, W=s.W, old_prefix=s.prefix, blocks=s.blocks, norm=s.norm,
                     query=s.query, out_norm=s.out_norm, nb=nb, write=write, has_delta=has_delta,
                     final=0, eps=s.eps, out_eps=s.out_eps, gpu_out=a["out"], gpu_new=a["prefix"],
                     what=f"packed M={M} K={K} H={H}")


def _run_ahead(s, nn, nq, *, packed, final, pad=8):
    """attnres_oproj_packed_ahead_run (packed) or attnres_oproj_ahead_run."""
    sga = lib()
    prefix, blocks = up(s.prefix), up(s.blocks)
    out = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    aux = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    ws = sga.make_workspace(s.M, s.H, s.nb, DEV)
    mix = torch.full((s.M, s.H + pad), float("nan"), dtype=torch.float32, device=DEV)
    scal = torch.full((s.M, 2), float("nan"), dtype=torch.float32, device=DEV)
    kw = dict(nb=s.nb, write=s.write, has_delta=s.has_delta, final_boundary=final, eps=s.eps,
              out_eps=s.out_eps, next_eps=1e-5)
    args = (prefix, blocks, up(s.norm), up(s.query), up(s.out_norm), out, aux, ws, up(nn), up(nq),
            mix[:, :s.H], scal)
    if packed:
        Wp = sga.attnres_pack_weights(up(s.W))
        sga.attnres_oproj_packed_ahead_run(up(s.x), Wp, s.H, *args, **kw)
    else:
        sga.attnres_oproj_ahead_run(up(s.x), up(s.W), *args, **kw)
    assert sga.attnres_workspace_status(ws) == 0
    torch.cuda.synchronize()
    res = {k: down(v) for k, v in (("out", out), ("prefix", prefix), ("blocks", blocks),
                                   ("aux", aux))}
    m = mix.cpu().numpy()
    assert np.all(np.isnan(m[:, s.H:])), "wrote into the mixture rows' padding"
    res["mixture"] = m[:, :s.H].view(np.uint32)
    res["scal"] = scal.cpu().numpy().view(np.uint32)
    return res


@pytest.mark.parametrize("M,K,H,nb,cap,write,final", [
    (1, 1024, 7168, 1, 1, -1, 0),    # one token, config 0 shape
    (8, 4096, 7168, 4, 4, -1, 1),    # config 1 shape, final boundary
    (13, 1000, 1024, 3, 4, 2, 0),    # ragged K, a scored slot written
    (40, 1000, 1024, 3, 4, 3, 0),    # split K, a block written after the scored ones
])
def test_packed_ahead_equals_row_major_ahead(M, K, H, nb, cap, write, final):
    """The look-ahead statistics do not involve W: bit-equal to the row-major
    call's. The step's own outputs equal the plain prepared call's bit for bit
    and, up to 32 tokens, the row-major look-ahead call's too."""
    s = synth.decode_step(M, K, nb, H=H, cap=cap, write=write, has_delta=1, seed=700 + M + K)
    n = synth.decode_step(1, None, 0, H=H, seed=78, layer=1)
    a = _run_ahead(s, n.norm, n.query, packed=True, final=final)
    b = _run_ahead(s, n.norm, n.query, packed=False, final=final)
    for k in ("mixture", "scal"):
        assert np.array_equal(a[k], b[k]), f"M={M}: look-ahead {k} differs"
    plain = _run(s, packed=True, final=final)
    for k in ("out", "prefix", "blocks", "aux"):
        assert np.array_equal(a[k], plain[k]), f"M={M}: {k} differs from the plain prepared call"
        if M <= 32:
            assert np.array_equal(a[k], b[k]), f"M={M}: {k} differs from the row-major call"
