"""Pins of the FP64 CPU oracle against facts it does not compute itself.

Every check here is something other than the oracle: library routines
(numpy matmul, torch rms_norm, torch's bfloat16 conversion), closed forms,
invariants of softmax and RMSNorm, hand-derived rounding cases and an
independent 60-digit brute force on 8-wide rows. The AttnRes definition they
pin is the one of ClusterAttnRes (pre / weights / post and the rstd helper) on
the vLLM attn_res.kernel page; the GEMM is WsGemm's y = x W^T with the -0.0
rule of positive_zero (gemm.ws_gemm page).
"""
from __future__ import annotations

import decimal
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_tools import bf16_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def bits(values) -> np.ndarray:
    """Exact float values (representable in bf16) -> bf16 bits, via torch."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    back = t.to(torch.float32).numpy()
    assert np.array_equal(back, np.asarray(values, dtype=np.float32)), "not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def torch_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """torch's float64 -> bfloat16 conversion (an independent rounding routine)."""
    return torch.tensor(x64, dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def near_bf16_tie(x64: np.ndarray, rel=1e-12) -> np.ndarray:
    """True where x lies within rel of a rounding midpoint of bfloat16."""
    a = np.abs(x64)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    q = np.exp2(e - 7)
    frac = a / q - np.floor(a / q)
    return np.abs(frac - 0.5) * q <= rel * np.maximum(a, 1e-300)


# --------------------------------------------------------------------------
# bfloat16 rounding
# --------------------------------------------------------------------------

def test_round_golden_cases():
    path = os.path.join(GOLDEN, "bf16_rounding.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        expr, want = line.rsplit(None, 1)
        value = eval(expr, {"__builtins__": {}})  # arithmetic on literals only
        assert oracle.round_bf16(value) == int(want, 16), (expr, hex(oracle.round_bf16(value)))
        n += 1
    assert n >= 15


def test_round_matches_torch_conversion():
    x = rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 30, 200_000))
    ours = np.array([oracle.round_bf16(v) for v in x[:20000]], dtype=np.uint16)
    theirs = torch_bf16_bits(x[:20000])
    # torch rounds double -> float -> bfloat16; the two agree except where the
    # first rounding lands exactly on a bfloat16 midpoint.
    f32 = x[:20000].astype(np.float32).astype(np.float64)
    double_round = near_bf16_tie(f32, rel=0.0) & (f32 != x[:20000])
    assert np.array_equal(ours[~double_round], theirs[~double_round])


def test_round_array_equals_scalar_rounding():
    """The array form is the scalar rule applied per element (golden cases,
    zeros of both signs, subnormals and random magnitudes)."""
    vals = [0.0, -0.0, 2.0 ** -133, -(2.0 ** -134), 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
            -(1.0 + 2.0 ** -8), 3.0e38, 2.0 ** -126 * 1.5]
    x = np.concatenate([np.array(vals), rng.standard_normal(4991) * np.exp2(
        rng.integers(-140, 120, 4991))]).reshape(50, -1)
    got = oracle.round_bf16_array(x)
    want = np.array([oracle.round_bf16(v) for v in x.ravel()], np.uint16).reshape(x.shape)
    assert got.shape == x.shape and np.array_equal(got, want)


# --------------------------------------------------------------------------
# GEMM pins (O-1 .. O-4)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 40, 96), (8, 33, 200), (16, 16, 1024), (64, 24, 520)])
def test_gemm_exact_integers(M, N, K):
    """Integers in [-8, 8]: every partial sum is an exact integer, so the FP64
    sum is exact in any order and a single rounding of the integer follows."""
    xi = rng.integers(-8, 9, (M, K))
    wi = rng.integers(-8, 9, (N, K))
    y = oracle.gemm(bits(xi), bits(wi))
    exact = xi.astype(np.int64) @ wi.T.astype(np.int64)
    assert np.abs(exact).max() < 2 ** 24
    want = torch_bf16_bits(exact.astype(np.float64))  # exact in float32 first
    want[want == 0x8000] = 0
    assert np.array_equal(y, want)


def test_gemm_identity_and_permutation():
    K = 64
    x = synth.normal_bf16(3, 1, 0, (5, K))
    eye = np.zeros((K, K), np.float32)
    perm = rng.permutation(K)
    eye[np.arange(K), perm] = 1.0
    y = oracle.gemm(x, bits(eye))
    want = x[:, perm].copy()
    want[want == 0x8000] = 0  # -0 * 1 summed from +0 is +0
    assert np.array_equal(y, want)


def test_gemm_zero_and_negative_zero():
    K = 32
    x = np.zeros((2, K), np.uint16)
    w = bits(-np.ones((3, K), np.float32))
    assert np.all(oracle.gemm(x, w) == 0)  # -0 products sum to +0
    # a tiny negative product rounds to -0 in bfloat16 and is stored as +0
    x1 = bits(np.full((1, 1), 2.0 ** -70, np.float32))
    w1 = bits(np.full((1, 1), -(2.0 ** -70), np.float32))
    y, ye = oracle.gemm(x1, w1, exact=True)
    assert ye[0, 0] == -(2.0 ** -140)
    assert oracle.round_bf16(ye[0, 0]) == 0x8000
    assert y[0, 0] == 0


def test_gemm_matches_numpy_matmul():
    x, W = synth.gemm_inputs(7, 300, 776, seed=5)
    y, ye = oracle.gemm(x, W, exact=True)
    ref = bf16_to_f64(x) @ bf16_to_f64(W).T
    assert np.max(np.abs(ye - ref) / np.maximum(np.abs(ref), 1e-3)) <= 1e-12
    want = torch_bf16_bits(ye)
    want[want == 0x8000] = 0
    tie = near_bf16_tie(ye, rel=0.0) | (ye.astype(np.float32) != ye) & near_bf16_tie(
        ye.astype(np.float32).astype(np.float64), rel=0.0)
    assert np.array_equal(y[~tie], want[~tie])


def test_gemm_threads_bit_identical():
    x, W = synth.gemm_inputs(9, 64, 256, seed=2)
    assert np.array_equal(oracle.gemm(x, W, nthreads=1), oracle.gemm(x, W, nthreads=4))
    # one token: the element split still spreads it over every thread, with the
    # same bits and the same exact sums
    x1 = x[:1]
    a, ea = oracle.gemm(x1, W, nthreads=1, exact=True)
    b, eb = oracle.gemm(x1, W, nthreads=7, exact=True)
    assert np.array_equal(a, b) and np.array_equal(ea, eb)


# --------------------------------------------------------------------------
# AttnRes pins (O-5 .. O-11, O-13)
# --------------------------------------------------------------------------

def _inputs(T=3, H=7168, nb=3, cap=None, seed=7, layer=0):
    s = synth.decode_step(T, None, nb, H=H, cap=cap, seed=seed, layer=layer)
    return s


def _run(s, **kw):
    kw.setdefault("nb", s.nb)
    return oracle.attnres(s.delta, s.prefix, s.blocks, s.norm, s.query, s.out_norm, **kw)


def _torch_rmsnorm(h, gain, eps):
    ht = torch.tensor(h, dtype=torch.float64)
    g = torch.tensor(gain, dtype=torch.float64)
    return torch.nn.functional.rms_norm(ht, (ht.shape[-1],), weight=g, eps=eps).numpy()


def test_nb0_is_residual_add_then_rmsnorm():
    s = _inputs(nb=0)
    r = _run(s, nb=0)
    eps = float(np.float32(1e-6))
    new64 = bf16_to_f64(s.prefix) + bf16_to_f64(s.delta)  # exact in float64
    new = torch_bf16_bits(new64)
    single = new64.astype(np.float32) == new64  # float32 step exact: single rounding
    assert np.array_equal(r.prefix[single], new[single])
    assert single.mean() > 0.99
    want = _torch_rmsnorm(bf16_to_f64(r.prefix), bf16_to_f64(s.out_norm), eps)
    assert np.max(np.abs(r.out_exact - want) / np.maximum(np.abs(want), 1e-3)) <= 1e-12


def test_softmax_weights_sum_to_one():
    s = _inputs(nb=8)
    for final in (0, 1):
        r = _run(s, final=final)
        p = r.probs[:, :9]
        assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-14)
        assert np.all(p >= 0)
        # and the weights follow the logits: softmax of the logits (numpy)
        lg = r.logits[:, :9]
        ref = np.exp(lg - lg.max(axis=1, keepdims=True))
        ref /= ref.sum(axis=1, keepdims=True)
        assert np.allclose(p, ref, rtol=1e-13, atol=1e-16)


def test_logits_closed_form():
    """l_b = (v_b . (norm*query)) / sqrt(mean(v_b^2) + eps), numpy in float64."""
    s = _inputs(nb=4)
    r = _run(s)
    eps = float(np.float32(1e-6))
    w = bf16_to_f64(s.norm) * bf16_to_f64(s.query)
    for t in range(s.M):
        for b in range(4):
            v = bf16_to_f64(s.blocks[t, b])
            want = np.dot(v, w) / math.sqrt(np.mean(v * v) + eps)
            assert abs(r.logits[t, b] - want) <= 1e-12 * max(1.0, abs(want))
        new = bf16_to_f64(r.prefix[t])
        want = np.dot(new, w) / math.sqrt(np.mean(new * new) + eps)
        assert abs(r.logits[t, 4] - want) <= 1e-12 * max(1.0, abs(want))


def test_equal_logits_give_the_mean():
    s = _inputs(nb=5)
    s.query[:] = 0  # every logit is exactly 0
    for final in (0, 1):
        r = _run(s, final=final)
        assert np.all(r.logits[:, :6] == 0.0)
        vs = bf16_to_f64(s.blocks[:, :5])
        mean = (vs.sum(axis=1) + bf16_to_f64(r.prefix)) / 6.0
        assert np.max(np.abs(r.h_exact - mean)) <= 1e-14 * np.max(np.abs(mean))
        if final == 0:
            want = _torch_rmsnorm(mean, bf16_to_f64(s.out_norm), float(np.float32(1e-6)))
            assert np.max(np.abs(r.out_exact - want) / np.maximum(np.abs(want), 1e-3)) <= 1e-12


@pytest.mark.parametrize("c", [0.75, -3.0, 1.0 / 1024])
def test_constant_rows_give_the_gain(c):
    s = _inputs(nb=3, T=2)
    cb = bits(np.array([c], np.float32))[0]
    s.blocks[:] = cb
    s.prefix[:] = cb
    s.delta[:] = 0
    oe = float(np.float32(1e-6))
    for final in (0, 1):
        r = _run(s, final=final)
        assert np.all(r.prefix == cb)
        want = bf16_to_f64(s.out_norm) * c / math.sqrt(c * c + oe)
        assert np.max(np.abs(r.out_exact - want[None])) <= 1e-13


def test_block_permutation_invariance():
    s = _inputs(nb=6)
    r0 = _run(s)
    perm = [3, 0, 5, 1, 4, 2]
    s2 = _inputs(nb=6)
    s2.blocks[:, :6] = s.blocks[:, perm]
    r1 = _run(s2)
    assert np.max(np.abs(r0.out_exact - r1.out_exact)) <= 1e-14 * np.max(np.abs(r0.out_exact))
    tie = near_bf16_tie(r0.out_exact, rel=1e-12)
    assert np.array_equal(r0.out[~tie], r1.out[~tie])


def test_scale_invariance_of_logits_without_eps():
    s = _inputs(nb=3, T=2)
    r0 = _run(s, eps=0.0, out_eps=0.0)
    s2 = _inputs(nb=3, T=2)
    scaled = bf16_to_f64(s.blocks[:, 1]) * 4.0  # exact in bf16
    s2.blocks[:, 1] = torch_bf16_bits(scaled)
    r1 = _run(s2, eps=0.0, out_eps=0.0)
    assert np.allclose(r0.logits[:, :4], r1.logits[:, :4], rtol=1e-13, atol=0)
    # the mixture moves linearly in the scaled block: h1 - h0 = p_1 (4 - 1) v_1
    dv = (r0.probs[:, 1:2] * 3.0) * bf16_to_f64(s.blocks[:, 1])
    assert np.max(np.abs((r1.h_exact - r0.h_exact) - dv)) <= 1e-13


def test_one_hot_limit():
    s = _inputs(nb=4)
    star = 2
    s.norm[:] = bits(np.array([1.0], np.float32))[0]
    s.query[:] = torch_bf16_bits(bf16_to_f64(s.blocks[0, star]) / 64.0)  # exact scaling
    r = _run(s, nb=4)
    assert np.delete(r.probs[0, :5], star).max() < 1e-30
    want = _torch_rmsnorm(bf16_to_f64(s.blocks[0, star]), bf16_to_f64(s.out_norm),
                          float(np.float32(1e-6)))
    assert np.max(np.abs(r.out_exact[0] - want) / np.maximum(np.abs(want), 1e-3)) <= 1e-10


def test_state_writes_and_index_placement():
    s = _inputs(nb=3, cap=5, T=3)
    r = _run(s, write=4)
    assert np.array_equal(r.aux, r.prefix)
    assert np.array_equal(r.blocks[:, 4], r.prefix)
    assert np.array_equal(r.blocks[:, :4], s.blocks[:, :4])  # untouched slots
    # overwriting a scored slot: the score uses its launch-time value
    r_over = _run(s, write=1)
    r_none = _run(s, write=-1)
    assert np.array_equal(r_over.out, r_none.out)
    assert np.array_equal(r_over.blocks[:, 1], r_none.prefix)
    # has_delta = 0: the delta is the new prefix and the old prefix is not read
    s.prefix[:] = 0x7FC0  # NaN would poison any read
    r0 = _run(s, has_delta=0)
    assert np.array_equal(r0.prefix, s.delta)
    assert np.isfinite(r0.out_exact).all()


@pytest.mark.parametrize("final", [0, 1])
@pytest.mark.parametrize("nb,cap,write,has_delta", [(0, 1, -1, 1), (1, 1, -1, 1), (4, 4, -1, 1),
                                                    (8, 9, 8, 1), (8, 9, 3, 0), (2, 3, 2, 0)])
def test_streaming_form_equals_plain_form(final, nb, cap, write, has_delta):
    s = _inputs(T=4, nb=nb, cap=cap, seed=11 + nb)
    a = _run(s, write=write, has_delta=has_delta, final=final)
    b = _run(s, write=write, has_delta=has_delta, final=final, streaming=True)
    scale = np.max(np.abs(a.out_exact))
    assert np.max(np.abs(a.out_exact - b.out_exact)) <= 1e-12 * scale
    tie = near_bf16_tie(a.out_exact, rel=1e-11)
    assert np.array_equal(a.out[~tie], b.out[~tie])
    assert np.array_equal(a.prefix, b.prefix) and np.array_equal(a.blocks, b.blocks)


def test_streaming_form_on_the_attnres_sweep():
    for nb in (0, 3, 8):
        s = synth.config_inputs(3, nb=nb)
        s.delta, s.prefix, s.blocks = s.delta[:16], s.prefix[:16], s.blocks[:16]
        a = _run(s, final=1)
        b = _run(s, final=1, streaming=True)
        assert np.max(np.abs(a.out_exact - b.out_exact)) <= 1e-12 * np.max(np.abs(a.out_exact))


def test_attnres_threads_bit_identical():
    s = _inputs(T=6, nb=2)
    a, b = _run(s, nthreads=1), _run(s, nthreads=3)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.prefix, b.prefix)


def test_fused_is_gemm_then_attnres():
    s = synth.decode_step(3, 256, 2, H=64, cap=3, write=2)
    f = oracle.attnres_oproj(s.x, s.W, s.prefix, s.blocks, s.norm, s.query, s.out_norm,
                             nb=2, write=2)
    y = oracle.gemm(s.x, s.W)
    assert np.array_equal(f.y, y)
    a = oracle.attnres(y, s.prefix, s.blocks, s.norm, s.query, s.out_norm, nb=2, write=2)
    assert np.array_equal(f.out, a.out) and np.array_equal(f.blocks, a.blocks)


# --------------------------------------------------------------------------
# O-12: 60-digit brute force on 8-wide rows, every flag combination
# --------------------------------------------------------------------------

D = decimal.Decimal
DYADIC = [-2.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0]


def _rne_bf16_fraction(x: Fraction) -> Fraction:
    """Nearest bfloat16 value to an exact rational (ties to even), normal range."""
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = 0
    while a >= Fraction(2) ** e:
        e += 1
    while a < Fraction(2) ** (e - 1):
        e -= 1
    q = Fraction(2) ** max(e - 8, -133)
    n, rem = divmod(a, q)
    if rem * 2 > q or (rem * 2 == q and n % 2 == 1):
        n += 1
    return (n * q) if x > 0 else -(n * q)


def _brute(delta, prefix, blocks, norm, query, gain, nb, has_delta, final, eps, oeps):
    H = len(norm)
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        F = lambda v: Fraction(float(v))  # noqa: E731  (inputs are dyadic: exact)
        w = [F(norm[i]) * F(query[i]) for i in range(H)]
        Deps, Doe = D(eps), D(oeps)

        def rr(ss, e):  # 1 / sqrt(ss / H + e)
            return 1 / (D(ss.numerator) / D(ss.denominator) / H + e).sqrt()

        def todec(f):
            return D(f.numerator) / D(f.denominator)

        new = []
        for i in range(H):
            v = F(prefix[i]) + F(delta[i]) if has_delta else F(delta[i])
            new.append(_rne_bf16_fraction(v))
        rows = [[F(blocks[b][i]) for i in range(H)] for b in range(nb)] + [new]
        lg = []
        for row in rows:
            ss = sum(v * v for v in row)
            d = sum(row[i] * w[i] for i in range(H))
            lg.append(todec(d) * rr(ss, Deps))
        if nb == 0:
            h = [todec(v) for v in new]
        else:
            L = max(lg)
            e = [(x - L).exp() for x in lg]
            Z = sum(e)
            p = [x / Z for x in e]
            h = [sum(p[j] * todec(rows[j][i]) for j in range(nb + 1)) for i in range(H)]
            if final:
                h = [todec(_rne_bf16_fraction(Fraction(x))) for x in h]
        hs = sum(x * x for x in h)
        s = 1 / (hs / H + Doe).sqrt()
        out = [h[i] * s * todec(F(gain[i])) for i in range(H)]
        return [float(v) for v in new], [float(o) for o in out]


def test_brute_force_h8_all_flags():
    H, T = 8, 2
    eps = float(np.float32(1e-6))
    count = 0
    for nb in range(4):
        cap = nb + 1
        for has_delta, final, aux in itertools.product((0, 1), (0, 1), (False, True)):
            for write in range(-1, cap):
                pick = lambda *shape: rng.choice(DYADIC, size=shape).astype(np.float32)  # noqa
                delta, prefix = pick(T, H), pick(T, H)
                blocks = pick(T, cap, H)
                norm = rng.choice([0.5, 1.0, 2.0, -1.0], size=H).astype(np.float32)
                query, gain = pick(H), rng.choice([0.5, 1.0, 2.0], size=H).astype(np.float32)
                r = oracle.attnres(bits(delta), bits(prefix), bits(blocks), bits(norm),
                                   bits(query), bits(gain), nb=nb, write=write,
                                   has_delta=has_delta, final=final, aux=aux)
                for t in range(T):
                    new, out = _brute(delta[t], prefix[t], blocks[t], norm, query, gain, nb,
                                      has_delta, final, eps, eps)
                    assert np.array_equal(bf16_to_f64(r.prefix[t]), np.array(new))
                    got = r.out_exact[t]
                    assert np.max(np.abs(got - np.array(out))) <= 1e-12 * max(1.0, np.max(np.abs(out)))
                    tie = near_bf16_tie(np.array(out), rel=1e-12)
                    want = torch_bf16_bits(np.array(out))
                    assert np.array_equal(r.out[t][~tie], want[~tie])
                    if aux:
                        assert np.array_equal(r.aux[t], r.prefix[t])
                    if write >= 0:
                        assert np.array_equal(r.blocks[t, write], r.prefix[t])
                    for b in range(cap):
                        if b != write:
                            assert np.array_equal(r.blocks[t, b], bits(blocks[t, b]))
                count += 1
    assert count == 8 * (2 + 3 + 4 + 5)  # every (nb, flags, write) combination ran


# --------------------------------------------------------------------------
# the input generator
# --------------------------------------------------------------------------

def test_splitmix64_published_vector():
    want = [int(l) for l in open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt"))
            if l.strip() and not l.startswith("#")]
    assert synth.splitmix64(1234567, 5) == want


def test_generator_vectorised_equals_scalar_definition():
    base = synth.stream_base(0, 2, 3)
    scalar = [synth.mix_int(base + (j + 1) * synth.GAMMA) for j in range(10, 20)]
    assert [int(v) for v in synth.words(0, 2, 3, 10, 10)] == scalar
    u = synth.uniforms(0, 2, 3, 10, 4)
    assert np.array_equal(u, np.array([(v >> 11) * 2.0 ** -53 for v in scalar[:4]]))
    # a slice regenerated on its own equals the same slice of the whole stream
    a = synth.normals(0, 1, 0, 1000)
    b = synth.normals(0, 1, 0, 100, start=450)
    assert np.array_equal(a[450:550], b)


def test_generator_distributions_and_bf16_encoding():
    z = synth.normals(0, 4, 0, 400_000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    b = synth.to_bf16_bits(z)
    want = torch.tensor(z.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, want)
    s = synth.decode_step(2, 512, 1, H=7168)
    wstd = bf16_to_f64(s.W).std() * math.sqrt(512)
    assert abs(wstd - 1) < 0.01
    assert abs(bf16_to_f64(s.norm).mean() - 1) < 0.01
    assert abs(bf16_to_f64(s.query).std() * math.sqrt(7168) - 1) < 0.05
