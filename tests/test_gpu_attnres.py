"""Parity of attnres_run (HIP, gfx950) with the FP64 oracle.

AttnRes of ClusterAttnRes (vLLM attn_res.kernel page) with the delta given as
a tensor. The new prefix is a single correctly rounded bf16 sum, so prefix,
aux and the written block slot must equal the oracle's bits exactly; the
output is held to two bf16 ulps (floored at 2^-10 of the row RMS) and a
relative L2 error of 5e-3. Every untouched element is poisoned with a NaN
pattern and must come back unchanged.
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
POISON = 0x7FC1


def run(s, *, nb, write, has_delta, final, aux=True, pad=0, slot_major=False, T=None):
    """Runs attnres_run on padded, poisoned buffers; returns host copies."""
    sga = lib()
    T = s.M if T is None else T
    H, cap = s.H, s.blocks.shape[1]
    ld = H + pad

    def padded(a):
        p = np.full((a.shape[0], ld), POISON, np.uint16)
        p[:, :H] = a
        return up(p)

    delta, prefix = padded(s.delta[:T]), padded(s.prefix[:T])
    out = torch.full((T, ld), POISON, dtype=torch.int16, device=DEV)
    auxg = torch.full((T, ld), POISON, dtype=torch.int16, device=DEV) if aux else None
    if slot_major:
        store = up(np.ascontiguousarray(s.blocks[:T].transpose(1, 0, 2)))  # [cap, T, H]
        blocks = store.permute(1, 0, 2)  # [T, cap, H]: token stride H, slot stride T*H
    else:
        bl = np.full((T, cap, ld), POISON, np.uint16)
        bl[:, :, :H] = s.blocks[:T]
        store = up(bl)
        blocks = store[:, :, :H]
    sga.attnres_run(delta[:, :H], prefix[:, :H], blocks, up(s.norm), up(s.query), up(s.out_norm),
                    out[:, :H], None if auxg is None else auxg[:, :H], nb=nb, write=write,
                    has_delta=has_delta, final_boundary=final, eps=s.eps, out_eps=s.out_eps)
    torch.cuda.synchronize()
    res = dict(out=down(out), prefix=down(prefix), delta=down(delta),
               aux=None if auxg is None else down(auxg))
    for k in ("out", "prefix", "delta", "aux"):
        if res[k] is not None:
            assert np.all(res[k][:, H:] == POISON), f"{k}: wrote past H"
            res[k] = res[k][:, :H]
    full = down(store)
    if slot_major:
        res["blocks"] = np.ascontiguousarray(full.transpose(1, 0, 2))
    else:
        assert np.all(full[:, :, H:] == POISON), "blocks: wrote past H"
        res["blocks"] = full[:, :, :H]
    return res


def check(s, r, *, nb, write, has_delta, final, aux=True, T=None, what=""):
    T = s.M if T is None else T
    ref = oracle.attnres(s.delta[:T], s.prefix[:T], s.blocks[:T], s.norm, s.query, s.out_norm,
                         nb=nb, write=write, has_delta=has_delta, final=final, eps=s.eps,
                         out_eps=s.out_eps, aux=aux, nthreads=16)
    assert_bf16_close(r["out"], ref.out, f"{what} out")
    assert np.array_equal(r["prefix"], ref.prefix), f"{what} prefix not bit-exact"
    if aux:
        assert np.array_equal(r["aux"], ref.prefix), f"{what} aux"
    assert np.array_equal(r["blocks"], ref.blocks), f"{what} blocks (written slot / untouched slots)"
    assert np.array_equal(r["delta"], s.delta[:T]), f"{what} delta modified"
    return ref


@pytest.mark.parametrize("nb", list(range(9)))
def test_attnres_sweep_final(nb):
    """T = 256 tokens, final boundary, per-block scales in [0.5, 4]."""
    s = synth.config_inputs(3, nb=nb)
    r = run(s, nb=nb, write=-1, has_delta=1, final=1)
    check(s, r, nb=nb, write=-1, has_delta=1, final=1, what=f"sweep nb={nb}")


@pytest.mark.parametrize("final", [0, 1])
@pytest.mark.parametrize("nb,cap,write,has_delta,aux", [
    (0, 1, -1, 1, True), (0, 1, 0, 0, False), (1, 1, -1, 1, True), (3, 4, 3, 1, True),
    (3, 3, 1, 1, True), (4, 4, -1, 0, False), (8, 9, 8, 1, True), (8, 8, 0, 0, True),
])
def test_attnres_flags(final, nb, cap, write, has_delta, aux):
    s = synth.decode_step(5, None, nb, cap=cap, seed=100 + nb + 10 * final)
    r = run(s, nb=nb, write=write, has_delta=has_delta, final=final, aux=aux, pad=16)
    check(s, r, nb=nb, write=write, has_delta=has_delta, final=final, aux=aux,
          what=f"flags nb={nb} w={write} d={has_delta} f={final}")


@pytest.mark.parametrize("H", [8, 64, 1000, 4104, 7168, 8192])
def test_attnres_widths(H):
    s = synth.decode_step(3, None, 3, H=H, cap=4, seed=7)
    for final in (0, 1):
        r = run(s, nb=3, write=3, has_delta=1, final=final, pad=8)
        check(s, r, nb=3, write=3, has_delta=1, final=final, what=f"H={H}")


def test_attnres_slot_major_blocks():
    s = synth.decode_step(6, None, 4, cap=5, seed=3)
    r = run(s, nb=4, write=4, has_delta=1, final=0, slot_major=True)
    ref = oracle.attnres(s.delta, s.prefix, s.blocks, s.norm, s.query, s.out_norm, nb=4, write=4,
                         nthreads=16)
    assert_bf16_close(r["out"], ref.out, "slot-major out")
    assert np.array_equal(r["blocks"], ref.blocks)


def test_attnres_deterministic():
    s = synth.config_inputs(3, nb=8)
    a = run(s, nb=8, write=-1, has_delta=1, final=1)
    b = run(s, nb=8, write=-1, has_delta=1, final=1)
    for k in ("out", "prefix", "aux"):
        assert np.array_equal(a[k], b[k]), k


def test_attnres_empty():
    s = synth.decode_step(2, None, 1, seed=1)
    sga = lib()
    z = torch.zeros((0, s.H), dtype=torch.int16, device=DEV)
    bl = torch.zeros((0, 1, s.H), dtype=torch.int16, device=DEV)
    sga.attnres_run(z, z, bl, up(s.norm), up(s.query), up(s.out_norm), z, None, nb=1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,H,nb,cap,write,has_delta,final,aux,pad,slot_major", [
    (257, 7168, 4, 5, 2, 0, 0, True, 0, False),    # odd T, overwrite a scored slot, no old prefix
    (300, 1000, 3, 4, 3, 1, 1, False, 8, False),   # rows not a multiple of 512 columns, padded rows
    (258, 4104, 8, 9, 8, 1, 0, True, 0, True),     # slot-major blocks, block write after the scored slots
    (260, 8192, 8, 8, 0, 1, 1, True, 0, False),    # widest rows, all slots scored
    (512, 2048, 0, 1, 0, 0, 1, True, 0, False),    # nb = 0, delta path off
])
def test_attnres_many_tokens(T, H, nb, cap, write, has_delta, final, aux, pad,
                                          slot_major):
    """Many tokens (more than half the compute units), odd counts, widths that
    are not a multiple of 512 columns, padded and slot-major layouts."""
    s = synth.decode_step(T, None, nb, H=H, cap=cap, seed=T + H + nb)
    r = run(s, nb=nb, write=write, has_delta=has_delta, final=final, aux=aux, pad=pad,
            slot_major=slot_major)
    if slot_major:
        ref = oracle.attnres(s.delta, s.prefix, s.blocks, s.norm, s.query, s.out_norm, nb=nb,
                             write=write, has_delta=has_delta, final=final, eps=s.eps,
                             out_eps=s.out_eps, aux=aux, nthreads=16)
        assert_bf16_close(r["out"], ref.out, "slot-major out")
        assert np.array_equal(r["prefix"], ref.prefix)
        assert np.array_equal(r["blocks"], ref.blocks)
    else:
        check(s, r, nb=nb, write=write, has_delta=has_delta, final=final, aux=aux,
              what=f"T={T} H={H} nb={nb}")


def _special_pairs(T, H, *, negative_zero_delta, seed):
    """prefix / delta bit patterns mixing ordinary values with signed zeros,
    bfloat16 subnormals, the smallest normals and exact cancellations."""
    rng = np.random.default_rng(seed)
    tiny = [0x0000, 0x8000, 0x0001, 0x8001, 0x0003, 0x8003, 0x0040, 0x807F, 0x0080, 0x8080,
            0x3FC0, 0xBFC0]  # +-0, subnormals, smallest normals, +-1.5
    s = synth.decode_step(T, None, 1, H=H, cap=2, seed=seed)
    prefix, delta = s.prefix.copy(), s.delta.copy()
    special = rng.random((T, H)) < 0.6
    prefix[special] = rng.choice(tiny, size=int(special.sum()))
    delta[special] = rng.choice(tiny, size=int(special.sum()))
    cancel = special & (rng.random((T, H)) < 0.4)
    delta[cancel] = prefix[cancel] ^ 0x8000  # x + (-x): an exact zero
    if not negative_zero_delta:  # the fused call's delta: -0.0 is stored as +0.0
        delta[delta == 0x8000] = 0x0000
    s.prefix, s.delta = prefix, delta
    return s


@pytest.mark.parametrize("has_delta", [1, 0])
def test_residual_add_keeps_signed_zeros_and_subnormals(has_delta):
    """The new prefix bf16(prefix + delta) with signed zeros, subnormals and
    exact cancellations is the oracle's bit for bit, and with a delta that
    never holds -0.0 (the projection's, -0.0 made +0.0 as on the gemm.ws_gemm
    page, positive_zero) it never holds -0.0 either: an exact zero sum is
    +0.0 and subnormals are neither flushed nor sign-flipped. The fused call's
    mailbox relies on this, since its sentinel is the pair (+0.0, -0.0)."""
    s = _special_pairs(4, 1024, negative_zero_delta=False, seed=11)
    r = run(s, nb=1, write=1, has_delta=has_delta, final=0)
    ref = check(s, r, nb=1, write=1, has_delta=has_delta, final=0, what="signed zeros")
    assert not np.any(r["prefix"] == 0x8000), "a new prefix element is -0.0"
    assert np.count_nonzero((r["prefix"] & 0x7F80) == 0) > 1000  # zeros and subnormals present
    if has_delta:
        assert np.any((r["prefix"] & 0x7FFF) != 0) and np.array_equal(r["prefix"], ref.prefix)


def test_residual_add_negative_zero_delta_matches_oracle():
    """With -0.0 in the delta (which the fused call never passes), -0.0 + -0.0
    is -0.0 on both sides: the sum is the IEEE one, bit for bit."""
    s = _special_pairs(4, 1024, negative_zero_delta=True, seed=12)
    r = run(s, nb=1, write=-1, has_delta=1, final=1)
    ref = check(s, r, nb=1, write=-1, has_delta=1, final=1, what="negative-zero delta")
    both = (s.prefix == 0x8000) & (s.delta == 0x8000)
    assert both.any() and np.all(ref.prefix[both] == 0x8000)
