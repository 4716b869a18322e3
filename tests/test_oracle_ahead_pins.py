"""Pins of the oracle's saved-block statistics and of post() on given statistics.

The statistics are the state ClusterAttnRes carries from pre() to post()
(attn_res.kernel page: the mixture row and the scalars maximum and exp_sum),
which the fused o-projection also stores for the next layer's AttnRes over the
same saved blocks (oproj.prepared page, PreparedOproj.bind_ahead). The pins use
what the pages and the mathematics fix: the one-block and equal-block closed
forms, the composition pre + post = the plain softmax form (a separate code
path of the oracle), and the invariance of post under a shift of the carried
maximum.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity_tools import bf16_to_f64

EPS = float(np.float32(1e-6))


def _inputs(T=3, H=7168, nb=3, cap=None, seed=21):
    return synth.decode_step(T, None, nb, H=H, cap=cap, seed=seed)


def _plain(s, **kw):
    kw.setdefault("nb", s.nb)
    return oracle.attnres(s.delta, s.prefix, s.blocks, s.norm, s.query, s.out_norm, **kw)


def _post(s, mix, scal, **kw):
    kw.setdefault("nb", s.nb)
    return oracle.attnres_post(s.delta, s.prefix, s.blocks, s.norm, s.query, s.out_norm, mix,
                               scal, **kw)


def test_pre_one_block_is_that_block():
    s = _inputs(nb=1)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=1)
    r = _plain(s)
    assert np.array_equal(scal[:, 1], np.ones(s.M))  # S = exp(0)
    assert np.array_equal(mix, bf16_to_f64(s.blocks[:, 0]))  # 1 * v_0, exact
    lg = r.logits[:, 0]  # the plain form's block logit
    assert np.all(np.abs(scal[:, 0] - lg) <= 1e-13 * np.maximum(1.0, np.abs(lg)))


def test_pre_equal_blocks_sum_to_nb_copies():
    nb = 5
    s = _inputs(nb=nb)
    s.blocks[:, 1:nb] = s.blocks[:, :1]
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=nb)
    assert np.array_equal(scal[:, 1], np.full(s.M, float(nb)))  # every e_b = exp(0)
    assert np.array_equal(mix, nb * bf16_to_f64(s.blocks[:, 0]))  # exact: small multiples


def test_pre_without_blocks_is_zero():
    s = _inputs(nb=0)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=0)
    assert not mix.any() and not scal.any()


def test_pre_maximum_is_the_largest_logit():
    s = _inputs(nb=8, T=4, seed=5)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=8)
    r = _plain(s)
    lg = r.logits[:, :8]
    assert np.all(np.abs(scal[:, 0] - lg.max(axis=1)) <= 1e-13 * np.maximum(1.0, np.abs(scal[:, 0])))
    # exp_sum >= 1 (the largest term is exp(0)) and <= nb
    assert np.all(scal[:, 1] >= 1.0) and np.all(scal[:, 1] <= 8.0)


@pytest.mark.parametrize("final", [0, 1])
@pytest.mark.parametrize("nb,cap,write,has_delta", [(0, 1, -1, 1), (1, 1, -1, 1), (4, 4, -1, 1),
                                                    (8, 9, 8, 1), (3, 4, 1, 0), (2, 3, 2, 0)])
def test_pre_then_post_is_the_plain_form(final, nb, cap, write, has_delta):
    s = _inputs(T=4, nb=nb, cap=cap, seed=31 + nb)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=nb)
    a = _plain(s, write=write, has_delta=has_delta, final=final)
    b = _post(s, mix, scal, write=write, has_delta=has_delta, final=final)
    scale = np.max(np.abs(a.out_exact))
    assert np.max(np.abs(a.out_exact - b.out_exact)) <= 1e-12 * scale
    # state writes: the same bits in the same places
    assert np.array_equal(a.prefix, b.prefix) and np.array_equal(a.aux, b.aux)
    assert np.array_equal(a.blocks, b.blocks)


def test_post_is_invariant_under_a_shift_of_the_carried_maximum():
    """(m, S, mix) and (m + d, S e^-d, mix e^-d) describe the same softmax state."""
    s = _inputs(T=3, nb=4, seed=8)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=4)
    for d in (-3.0, 0.7, 5.0):
        sh = scal.copy()
        sh[:, 0] += d
        sh[:, 1] *= np.exp(-d)
        for final in (0, 1):
            a = _post(s, mix, scal, final=final)
            b = _post(s, mix * np.exp(-d), sh, final=final)
            assert np.max(np.abs(a.out_exact - b.out_exact)) <= 1e-12 * np.max(np.abs(a.out_exact))


def test_post_with_float32_statistics_stays_close():
    """Statistics stored as float32 (the GPU's width) move the output by about
    float32 precision, far inside one bf16 ulp."""
    s = _inputs(T=4, nb=8, cap=9, seed=9)
    mix, scal = oracle.attnres_pre(s.blocks, s.norm, s.query, nb=8)
    a = _post(s, mix, scal)
    b = _post(s, mix.astype(np.float32), scal.astype(np.float32))
    assert np.max(np.abs(a.out_exact - b.out_exact)) <= 1e-6 * np.max(np.abs(a.out_exact))


def test_pre_uses_its_own_weights_and_eps():
    """Statistics for another layer's norm, query and eps: the same as that
    layer's own plain AttnRes over the same blocks."""
    s = _inputs(T=2, nb=3, seed=12)
    nxt = _inputs(T=2, nb=3, seed=13)
    mix, scal = oracle.attnres_pre(s.blocks, nxt.norm, nxt.query, nb=3, eps=1e-5)
    r = oracle.attnres(s.delta, s.prefix, s.blocks, nxt.norm, nxt.query, s.out_norm, nb=3,
                       eps=1e-5)
    lg = r.logits[:, :3]
    assert np.all(np.abs(scal[:, 0] - lg.max(axis=1)) <= 1e-13 * np.maximum(1.0, np.abs(lg.max(axis=1))))
    b = oracle.attnres_post(s.delta, s.prefix, s.blocks, nxt.norm, nxt.query, s.out_norm, mix,
                            scal, nb=3, eps=1e-5)
    assert np.max(np.abs(r.out_exact - b.out_exact)) <= 1e-12 * np.max(np.abs(r.out_exact))
