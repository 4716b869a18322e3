"""A multi-layer decode chain through the C ABI, HIP gfx950, against the oracle.

Per decoder layer (oproj.prepared page, PreparedOproj.__init__: the o-projection
AttnRes scores prev_valid_blocks + is_block_write_layer blocks and takes the
delta path only off block-write layers; attn_res.kernel page: the final
boundary rounds the mixture before its RMSNorm):

  1. pre-attention AttnRes on the previous MLP output (attnres_run): at a
     block-write layer it saves the completed block prefix into the next
     free slot (write = valid), which then counts as valid;
  2. the o-projection with its AttnRes (attnres_oproj_run) scoring every
     valid block; at a block-write layer has_delta = 0, so the prefix
     restarts from the projection output;
  3. after the last layer, one final-boundary AttnRes.

The attention and MLP outputs are synthetic. Every call is checked against
the oracle on the state the GPU carries into it (so a legitimate one-ulp
difference does not compound), the block slots and the valid count evolve
exactly, untouched slots keep their poison, and the same chain with the
look-ahead statistics (attnres_oproj_ahead_run, then attnres_post_run for the
next pre-attention AttnRes) gives the same bits throughout.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_tools import DEV, down, lib, up
from parity_tools import assert_bf16_close, check_fused_step

pytestmark = pytest.mark.gpu
POISON = 0x7FC1
H = 7168


def chain_inputs(L, M, K, writes, seed=5):
    """Weights and synthetic activations of an L-layer chain; block-write
    layers are those in `writes`."""
    cap = len(writes)
    base = synth.decode_step(M, K, 0, cap=cap, seed=seed)
    layers = []
    for l in range(L):
        sa = synth.decode_step(M, K, 0, cap=cap, seed=seed, layer=2 * l + 1, with_delta=True)
        mlp = synth.decode_step(M, K, 0, cap=cap, seed=seed, layer=2 * l + 2)
        layers.append(dict(
            delta=sa.delta,                         # previous MLP output
            sa=(sa.norm, sa.query, sa.out_norm),    # pre-attention AttnRes weights
            x=mlp.x, W=mlp.W,                       # attention output, o-projection
            mlp=(mlp.norm, mlp.query, mlp.out_norm),  # post-attention AttnRes weights
            write=l in writes))
    final = synth.decode_step(M, K, 0, cap=cap, seed=seed, layer=2 * L + 1, with_delta=True)
    return base.prefix, cap, layers, final


def run_chain(prefix0, cap, layers, final, *, ahead, check):
    """Runs the chain on the GPU; with `check`, compares every call with the
    oracle on the GPU's own state. Returns every output and the final state."""
    sga = lib()
    M = prefix0.shape[0]
    prefix = up(prefix0)
    blocks = up(np.full((M, cap, H), POISON, np.uint16))
    ws = sga.make_workspace(M, H, cap, DEV)
    mix = torch.full((M, H), float("nan"), dtype=torch.float32, device=DEV)
    scal = torch.full((M, 2), float("nan"), dtype=torch.float32, device=DEV)
    valid, outs, have_stats = 0, [], False
    for l, ly in enumerate(layers):
        # 1. pre-attention AttnRes
        nb, write = valid, (valid if ly["write"] else -1)
        st_prefix, st_blocks = down(prefix), down(blocks)
        out = torch.zeros((M, H), dtype=torch.int16, device=DEV)
        g = [up(a) for a in ly["sa"]]
        if ahead and have_stats:
            sga.attnres_post_run(up(ly["delta"]), prefix, blocks, *g, out, None, mix, scal,
                                 nb=nb, write=write)
        else:
            sga.attnres_run(up(ly["delta"]), prefix, blocks, *g, out, None, nb=nb, write=write)
        torch.cuda.synchronize()
        outs.append(down(out))
        if check:
            ref = oracle.attnres(ly["delta"], st_prefix, st_blocks, *ly["sa"], nb=nb,
                                 write=write, aux=False, nthreads=16)
            assert_bf16_close(outs[-1], ref.out, f"layer {l} pre-attention out")
            assert np.array_equal(down(prefix), ref.prefix), f"layer {l} pre-attention prefix"
            assert np.array_equal(down(blocks), ref.blocks), f"layer {l} pre-attention blocks"
        if ly["write"]:
            valid += 1
        # 2. o-projection + AttnRes, scoring every valid block
        nb, has_delta = valid, 0 if ly["write"] else 1
        st_prefix, st_blocks = down(prefix), down(blocks)
        out = torch.zeros((M, H), dtype=torch.int16, device=DEV)
        g = [up(a) for a in ly["mlp"]]
        if ahead:
            nxt = layers[l + 1]["sa"] if l + 1 < len(layers) else final_weights(final)
            sga.attnres_oproj_ahead_run(up(ly["x"]), up(ly["W"]), prefix, blocks, *g, out, None,
                                        ws, up(nxt[0]), up(nxt[1]), mix, scal, nb=nb,
                                        has_delta=has_delta)
            have_stats = True
        else:
            sga.attnres_oproj_run(up(ly["x"]), up(ly["W"]), prefix, blocks, *g, out, None, ws,
                                  nb=nb, has_delta=has_delta)
        torch.cuda.synchronize()
        outs.append(down(out))
        if check:
            # the new prefix within one projection ulp of the oracle's, the
            # output at the 2-ulp bar given the GPU's own new prefix
            nn, nq, no = ly["mlp"]
            check_fused_step(x=ly["x"], W=ly["W"], old_prefix=st_prefix, blocks=st_blocks,
                             norm=nn, query=nq, out_norm=no, nb=nb, write=-1,
                             has_delta=has_delta, final=0, eps=1e-6, out_eps=1e-6,
                             gpu_out=outs[-1], gpu_new=down(prefix), what=f"layer {l} o-proj")
            assert np.array_equal(down(blocks), st_blocks), f"layer {l}: o-proj wrote a block"
    # 3. final boundary
    st_prefix, st_blocks = down(prefix), down(blocks)
    out = torch.zeros((M, H), dtype=torch.int16, device=DEV)
    fw = [up(a) for a in final_weights(final)]
    if ahead:
        sga.attnres_post_run(up(final.delta), prefix, blocks, *fw, out, None, mix, scal,
                             nb=valid, final_boundary=1)
    else:
        sga.attnres_run(up(final.delta), prefix, blocks, *fw, out, None, nb=valid,
                        final_boundary=1)
    torch.cuda.synchronize()
    outs.append(down(out))
    if check:
        ref = oracle.attnres(final.delta, st_prefix, st_blocks, *final_weights(final), nb=valid,
                             final=1, aux=False, nthreads=16)
        assert_bf16_close(outs[-1], ref.out, "final boundary out")
        assert np.array_equal(down(prefix), ref.prefix), "final prefix"
    assert sga.attnres_workspace_status(ws) == 0, "a wait gave up"
    words = ws.cpu().numpy().view(np.uint32)
    assert np.all(words[:64] == 0) and np.all(words[64:] == 0x80000000), "workspace"
    return outs, down(prefix), down(blocks), valid


def final_weights(final):
    return final.norm, final.query, final.out_norm


@pytest.mark.parametrize("M,K,L,writes", [(8, 512, 5, (0, 2, 4)), (3, 256, 4, (1, 2)),
                                          (40, 256, 3, (0, 1))])
def test_chain_matches_oracle_and_state_evolves(M, K, L, writes):
    prefix0, cap, layers, final = chain_inputs(L, M, K, writes)
    outs, prefix, blocks, valid = run_chain(prefix0, cap, layers, final, ahead=False, check=True)
    assert valid == len(writes)
    assert not np.any(blocks == POISON)  # every slot written exactly when its layer came


@pytest.mark.parametrize("M,K,L,writes", [(8, 512, 5, (0, 2, 4)), (40, 256, 3, (0, 1))])
def test_chain_with_lookahead_statistics_is_the_same_computation(M, K, L, writes):
    prefix0, cap, layers, final = chain_inputs(L, M, K, writes, seed=9)
    a = run_chain(prefix0, cap, layers, final, ahead=False, check=False)
    b = run_chain(prefix0, cap, layers, final, ahead=True, check=False)
    for i, (x, y) in enumerate(zip(a[0], b[0])):
        assert np.array_equal(x, y), f"call {i}: {int((x != y).sum())} outputs differ"
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and a[3] == b[3]
