"""Parity of the look-ahead statistics (attnres_oproj_ahead_run) and of AttnRes
on carried statistics (attnres_post_run), HIP gfx950, with the FP64 oracle.

The fused o-projection can also store the pre() state of the next layer's
AttnRes over the same saved blocks (vLLM oproj.prepared page,
PreparedOproj.bind_ahead; the state is ClusterAttnRes's mixture row and
maximum / exp_sum on the attn_res.kernel page). Checks:
  * the call's own outputs are those of attnres_oproj_run, bit for bit;
  * the statistics match the oracle's (attnres_pre) within a bound derived
    from FP32 sums of H products;
  * attnres_post_run on the oracle's statistics (rounded to float32) matches
    the oracle's post() on the same float32 statistics (2 bf16 ulps, exact
    state writes);
  * the chain: post on the GPU's statistics equals attnres_run with the next
    layer's weights over the same blocks, bit for bit (same reduction tree).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_tools import DEV, down, lib, up
from parity_tools import assert_bf16_close, bf16_to_f64

pytestmark = pytest.mark.gpu
POISON = 0x7FC1
U32 = 2.0 ** -24
NEXT_EPS = 1e-5


def next_weights(s, seed=77):
    """The next layer's norm and query: same distributions, another layer."""
    n = synth.decode_step(1, None, 0, H=s.H, seed=seed, layer=1)
    return n.norm, n.query


def run_fused(s, *, final, ahead, nn=None, nq=None, write=None, pad=8):
    sga = lib()
    write = s.write if write is None else write
    prefix, blocks = up(s.prefix), up(s.blocks)
    out = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    aux = torch.full((s.M, s.H), POISON, dtype=torch.int16, device=DEV)
    ws = sga.make_workspace(s.M, s.H, s.nb, DEV)
    res = {}
    if ahead:
        mix_store = torch.full((s.M, s.H + pad), float("nan"), dtype=torch.float32, device=DEV)
        scal = torch.full((s.M, 2), float("nan"), dtype=torch.float32, device=DEV)
        sga.attnres_oproj_ahead_run(up(s.x), up(s.W), prefix, blocks, up(s.norm), up(s.query),
                                    up(s.out_norm), out, aux, ws, up(nn), up(nq),
                                    mix_store[:, :s.H], scal, nb=s.nb, write=write,
                                    has_delta=s.has_delta, final_boundary=final, eps=s.eps,
                                    out_eps=s.out_eps, next_eps=NEXT_EPS)
    else:
        sga.attnres_oproj_run(up(s.x), up(s.W), prefix, blocks, up(s.norm), up(s.query),
                              up(s.out_norm), out, aux, ws, nb=s.nb, write=write,
                              has_delta=s.has_delta, final_boundary=final, eps=s.eps,
                              out_eps=s.out_eps)
    torch.cuda.synchronize()
    words = ws.cpu().numpy().view(np.uint32)
    assert np.all(words[:64] == 0), "workspace header not zero (a wait gave up)"
    assert np.all(words[64:] == 0x80000000), "mailbox not re-armed"
    res.update(out=down(out), prefix=down(prefix), blocks=down(blocks), aux=down(aux))
    if ahead:
        m = mix_store.cpu().numpy()
        assert np.all(np.isnan(m[:, s.H:])), "mixture: wrote past H"
        res.update(mixture=m[:, :s.H], scal=scal.cpu().numpy(), gpu_mix=mix_store[:, :s.H],
                   gpu_scal=scal)
    return res


def check_statistics(s, mix, scal, nn, nq, exact_sums=False):
    """GPU statistics against the oracle's, within a bound derived from the
    FP32 arithmetic: each logit is a product of an H-term FP32 dot product and
    a reciprocal root (error <= ~(log2 H + 4) u of the absolute sums; with
    ``exact_sums`` the inputs make every FP32 sum exact and only the root and
    the products round), e_b = exp(l_b - m) adds a few ulps of its argument,
    and the mixture / exp_sum are at most 8-term FP32 sums."""
    ref_mix, ref_scal = oracle.attnres_pre(s.blocks, nn, nq, nb=s.nb, eps=NEXT_EPS, nthreads=16)
    if s.nb == 0:
        assert not mix.any() and not scal.any(), "nb == 0: statistics must be zero"
        return
    w = bf16_to_f64(nn) * bf16_to_f64(nq)
    v = bf16_to_f64(s.blocks[:, :s.nb])  # [M, nb, H]
    ss = np.sum(v * v, axis=-1)
    r = 1.0 / np.sqrt(ss / s.H + np.float32(NEXT_EPS))
    lg = np.sum(v * w, axis=-1) * r
    absd = np.sum(np.abs(v * w), axis=-1) * r
    k = np.log2(s.H) + 4
    tol_l = 8 * U32 * np.abs(lg) if exact_sums else k * U32 * (absd + np.abs(lg))  # [M, nb]
    m = ref_scal[:, 0]
    assert np.allclose(m, lg.max(axis=1), rtol=1e-12, atol=1e-12)  # oracle self-consistency
    tol_m = tol_l.max(axis=1)
    assert np.all(np.abs(scal[:, 0] - m) <= tol_m + U32 * np.abs(m)), "maximum"
    e = np.exp(lg - m[:, None])
    tol_e = e * (tol_l + tol_m[:, None] + 8 * U32 * (1 + np.abs(lg - m[:, None])))
    S = ref_scal[:, 1]
    assert np.all(np.abs(scal[:, 1] - S) <= tol_e.sum(axis=1) + 8 * U32 * S), "exp_sum"
    tol_mix = np.einsum("mb,mbh->mh", tol_e, np.abs(v)) + 8 * U32 * np.einsum(
        "mb,mbh->mh", e, np.abs(v))
    bad = np.abs(mix.astype(np.float64) - ref_mix) > tol_mix
    assert not bad.any(), f"mixture: {int(bad.sum())} elements beyond the bound"


@pytest.fixture(scope="module")
def configs():
    return {c: synth.config_inputs(c) for c in (0, 1, 2)}


@pytest.mark.parametrize("final", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_ahead_outputs_are_those_of_the_plain_call(configs, cfg, final):
    s = configs[cfg]
    nn, nq = next_weights(s)
    a = run_fused(s, final=final, ahead=True, nn=nn, nq=nq)
    b = run_fused(s, final=final, ahead=False)
    for k in ("out", "prefix", "blocks", "aux"):
        assert np.array_equal(a[k], b[k]), f"cfg{cfg} {k} differs from attnres_oproj_run"


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_ahead_statistics_match_oracle(configs, cfg):
    s = configs[cfg]
    nn, nq = next_weights(s)
    a = run_fused(s, final=0, ahead=True, nn=nn, nq=nq)
    check_statistics(s, a["mixture"], a["scal"], nn, nq)


@pytest.mark.parametrize("M,K,nb,cap,write", [
    (1, 64, 0, 1, -1),      # no saved blocks: zero statistics
    (3, 256, 1, 2, 1),      # one block
    (17, 520, 3, 4, 2),     # two token tiles, a scored slot overwritten after pre
    (40, 1000, 5, 6, 5),    # split K, two tokens per owner, odd token count per owner
])
def test_ahead_edges(M, K, nb, cap, write):
    s = synth.decode_step(M, K, nb, cap=cap, write=write, seed=100 + M)
    nn, nq = next_weights(s, seed=5 + M)
    a = run_fused(s, final=0, ahead=True, nn=nn, nq=nq)
    b = run_fused(s, final=0, ahead=False)
    for k in ("out", "prefix", "blocks", "aux"):
        assert np.array_equal(a[k], b[k]), f"{k} differs from attnres_oproj_run"
    # statistics use the blocks as they were at launch (the written slot's old value)
    check_statistics(s, a["mixture"], a["scal"], nn, nq)


def test_ahead_statistics_with_exact_sums():
    """Dyadic saved blocks (mostly zero, so eps weighs on every logit) and
    dyadic weights: every FP32 sum is exact, so the statistics must match the
    oracle to a few ulps; a wrong eps, weight row or block shows at once."""
    rng = np.random.default_rng(2024)
    s = synth.decode_step(8, 256, 4, cap=4, seed=61)
    vals = np.array([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], np.float32)
    v = rng.choice(vals, size=s.blocks.shape) * (rng.random(s.blocks.shape) < 0.1)
    to_bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731
    s.blocks = to_bits(v)
    nn = to_bits(rng.choice(np.array([0.5, 1.0, 2.0], np.float32), size=s.H))
    nq = to_bits(rng.choice(np.array([-0.25, -0.125, 0.125, 0.25], np.float32), size=s.H))
    a = run_fused(s, final=0, ahead=True, nn=nn, nq=nq)
    check_statistics(s, a["mixture"], a["scal"], nn, nq, exact_sums=True)


def run_post(s, mix, scal, *, nb, write, has_delta, final, T=None, blocks=True):
    sga = lib()
    T = s.M if T is None else T
    H = s.H
    prefix = up(s.prefix[:T])
    out = torch.full((T, H), POISON, dtype=torch.int16, device=DEV)
    aux = torch.full((T, H), POISON, dtype=torch.int16, device=DEV)
    cap = s.blocks.shape[1]
    bl = up(np.full((T, cap, H), POISON, np.uint16)) if blocks else None
    mix_g = None if mix is None else torch.from_numpy(np.ascontiguousarray(mix[:T], np.float32)).to(DEV)
    scal_g = None if scal is None else torch.from_numpy(np.ascontiguousarray(scal[:T], np.float32)).to(DEV)
    sga.attnres_post_run(up(s.delta[:T]), prefix, bl, up(s.norm), up(s.query), up(s.out_norm),
                         out, aux, mix_g, scal_g, nb=nb, write=write, has_delta=has_delta,
                         final_boundary=final, eps=s.eps, out_eps=s.out_eps)
    torch.cuda.synchronize()
    return dict(out=down(out), prefix=down(prefix), aux=down(aux),
                blocks=None if bl is None else down(bl))


@pytest.mark.parametrize("final", [0, 1])
@pytest.mark.parametrize("nb,cap,write,has_delta", [(0, 1, -1, 1), (1, 1, 0, 1), (4, 4, -1, 1),
                                                    (8, 9, 8, 1), (3, 4, 1, 0), (8, 8, 2, 1)])
def test_post_run_matches_oracle(nb, cap, write, has_delta, final):
    s = synth.decode_step(6, None, nb, cap=cap, write=write, has_delta=has_delta, seed=40 + nb,
                          block_scales=True)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=nb, eps=s.eps, nthreads=16)
    mix32, scal32 = mix.astype(np.float32), scal.astype(np.float32)
    r = run_post(s, mix32, scal32, nb=nb, write=write, has_delta=has_delta, final=final)
    ref = oracle.attnres_post(s.delta, s.prefix, s.blocks, s.norm, s.query, s.out_norm, mix32,
                              scal32, nb=nb, write=write, has_delta=has_delta, final=final,
                              eps=s.eps, out_eps=s.out_eps, nthreads=16)
    assert_bf16_close(r["out"], ref.out, "post out")
    assert np.array_equal(r["prefix"], ref.prefix), "prefix not bit-exact"
    assert np.array_equal(r["aux"], ref.prefix), "aux"
    for b in range(cap):  # the saved blocks are written only (slot write), never read
        want = ref.prefix if b == write else np.full_like(ref.prefix, POISON)
        assert np.array_equal(r["blocks"][:, b], want), f"slot {b}"


def test_post_run_many_tokens_and_no_blocks():
    s = synth.decode_step(300, None, 8, cap=8, seed=3, block_scales=True)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=8, eps=s.eps, nthreads=16)
    mix32, scal32 = mix.astype(np.float32), scal.astype(np.float32)
    r = run_post(s, mix32, scal32, nb=8, write=-1, has_delta=1, final=1, blocks=False)
    ref = oracle.attnres_post(s.delta, s.prefix, s.blocks, s.norm, s.query, s.out_norm, mix32,
                              scal32, nb=8, final=1, eps=s.eps, out_eps=s.out_eps, nthreads=16)
    assert_bf16_close(r["out"], ref.out, "post out")
    assert np.array_equal(r["prefix"], ref.prefix)


@pytest.mark.parametrize("cfg", [1, 2])
@pytest.mark.parametrize("final", [0, 1])
def test_chain_equals_attnres_run_with_the_next_weights(configs, cfg, final):
    """The next layer's AttnRes on carried statistics is the same computation,
    bit for bit, as attnres_run re-reading the saved blocks."""
    s = configs[cfg]
    assert s.write < 0 or s.write >= s.nb  # the scored blocks are unchanged by the fused call
    nn, nq = next_weights(s)
    a = run_fused(s, final=0, ahead=True, nn=nn, nq=nq)
    sga = lib()
    nxt = synth.decode_step(s.M, None, s.nb, cap=s.blocks.shape[1], seed=900 + cfg, layer=2)
    H = s.H

    def post_call():
        prefix = up(a["prefix"])
        out = torch.zeros((s.M, H), dtype=torch.int16, device=DEV)
        sga.attnres_post_run(up(nxt.delta), prefix, None, up(nn), up(nq), up(s.out_norm), out,
                             None, a["gpu_mix"], a["gpu_scal"], nb=s.nb, final_boundary=final,
                             eps=NEXT_EPS, out_eps=s.out_eps)
        torch.cuda.synchronize()
        return down(out), down(prefix)

    def run_call():
        prefix = up(a["prefix"])
        out = torch.zeros((s.M, H), dtype=torch.int16, device=DEV)
        sga.attnres_run(up(nxt.delta), prefix, up(a["blocks"]), up(nn), up(nq), up(s.out_norm),
                        out, None, nb=s.nb, final_boundary=final, eps=NEXT_EPS,
                        out_eps=s.out_eps)
        torch.cuda.synchronize()
        return down(out), down(prefix)

    o1, p1 = post_call()
    o2, p2 = run_call()
    assert np.array_equal(p1, p2)
    assert np.array_equal(o1, o2), f"{int((o1 != o2).sum())} outputs differ"
