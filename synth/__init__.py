"""Seeded synthetic inputs for the o-projection + AttnRes decode step.

This module only draws numbers: it holds none of the method's arithmetic and is
shared by the tests, the benchmark and the callers of the CPU oracle. Every
value is a pure function of ``(seed, stream, layer, index)``, so any slice of
any tensor can be regenerated on its own.

Generator (counter based, SplitMix64 of Steele, Lea and Flood, 2014, with
Vigna's published mixing constants):

* ``mix(z)``: ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31`` (all mod 2**64).
* SplitMix64 seeded with ``s`` returns ``mix(s + n * GAMMA)`` as its n-th
  output (n = 1, 2, ...), ``GAMMA = 0x9E3779B97F4A7C15``.
* A stream's key packs ``seed`` (32 bits), ``stream`` (8 bits) and ``layer``
  (24 bits): ``key = seed | stream << 32 | layer << 40``; its base is the first
  SplitMix64 output of ``key``: ``base = mix(key + GAMMA)``.
* Raw word ``j`` of the stream is output ``j + 1`` of SplitMix64 seeded with
  ``base``; the uniform ``u_j = (word >> 11) * 2**-53`` lies in [0, 1).
* Normal ``i`` uses ``u_{2i}`` and ``u_{2i+1}`` (Box-Muller, cosine branch):
  ``z = sqrt(-2 ln(1 - u_{2i})) * cos(2 pi u_{2i+1})``.
* Values are scaled and shifted in float64, rounded to float32 (nearest even),
  then to bfloat16 (nearest even) and handed out as raw ``uint16`` bit
  patterns.

Distributions of the decode workload (hidden width 7168):

* x, prefix, saved blocks, delta: N(0, 1); W: N(0, 1) / sqrt(K);
* norm and out_norm gains: 1 + 0.1 N(0, 1); query: N(0, 1) / sqrt(7168);
* AttnRes-only sweep: block b of every token is additionally scaled by
  ``s_b = 0.5 + 3.5 u_b`` from stream ``block_scale``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

STREAMS = {
    "x": 1,
    "W": 2,
    "prefix": 3,
    "blocks": 4,
    "delta": 5,
    "norm": 6,
    "query": 7,
    "out_norm": 8,
    "block_scale": 9,
}

_CHUNK = 1 << 22  # values per vectorised chunk (bounded temporaries)


def mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function applied elementwise to uint64 words."""
    z = np.asarray(z, dtype=np.uint64).copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def mix_int(z: int) -> int:
    """Scalar SplitMix64 output function on a Python int."""
    z &= _MASK64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _MASK64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _MASK64
    z ^= z >> 31
    return z


def splitmix64(seed: int, count: int) -> list[int]:
    """The first ``count`` outputs of SplitMix64 seeded with ``seed``."""
    return [mix_int(seed + n * GAMMA) for n in range(1, count + 1)]


def stream_base(seed: int, stream: int, layer: int) -> int:
    if not (0 <= seed < 1 << 32 and 0 <= stream < 1 << 8 and 0 <= layer < 1 << 24):
        raise ValueError("seed, stream or layer out of range")
    key = seed | (stream << 32) | (layer << 40)
    return mix_int(key + GAMMA)


def words(seed: int, stream: int, layer: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit words ``start .. start+count-1`` of one stream."""
    base = np.uint64(stream_base(seed, stream, layer))
    j = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    return mix(base + j * np.uint64(GAMMA))


def uniforms(seed: int, stream: int, layer: int, start: int, count: int) -> np.ndarray:
    w = words(seed, stream, layer, start, count)
    return (w >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))


def normals(seed: int, stream: int, layer: int, count: int, start: int = 0) -> np.ndarray:
    """Standard normals ``start .. start+count-1`` of one stream, float64."""
    out = np.empty(count, dtype=np.float64)
    for lo in range(0, count, _CHUNK):
        n = min(_CHUNK, count - lo)
        u = uniforms(seed, stream, layer, 2 * (start + lo), 2 * n)
        u1, u2 = u[0::2], u[1::2]
        out[lo : lo + n] = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * math.pi * u2)
    return out


def to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest even) -> bfloat16 bits (nearest even)."""
    f = np.ascontiguousarray(values, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def normal_bf16(seed, stream, layer, shape, scale=1.0, shift=0.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _CHUNK):
        k = min(_CHUNK, n - lo)
        z = normals(seed, stream, layer, k, start=lo)
        out[lo : lo + k] = to_bf16_bits(shift + scale * z)
    return out.reshape(shape)


# --------------------------------------------------------------------------
# The decode-step workloads.
# --------------------------------------------------------------------------

HIDDEN = 7168


@dataclass
class StepInputs:
    """Host copies (bfloat16 bit patterns as uint16) of one layer-step's inputs."""

    M: int
    K: int
    H: int
    nb: int
    cap: int
    write: int
    has_delta: int
    final: int
    eps: float
    out_eps: float
    x: np.ndarray | None  # [M, K]
    W: np.ndarray | None  # [H, K]
    delta: np.ndarray | None  # [M, H]
    prefix: np.ndarray  # [M, H]
    blocks: np.ndarray  # [M, cap, H]
    norm: np.ndarray  # [H]
    query: np.ndarray  # [H]
    out_norm: np.ndarray  # [H]
    with_aux: bool = True
    meta: dict = field(default_factory=dict)


def decode_step(
    M: int,
    K: int | None,
    nb: int,
    *,
    H: int = HIDDEN,
    cap: int | None = None,
    write: int = -1,
    has_delta: int = 1,
    final: int = 0,
    seed: int = 0,
    layer: int = 0,
    block_scales: bool = False,
    with_delta: bool = False,
    eps: float = 1e-6,
    out_eps: float = 1e-6,
) -> StepInputs:
    """Inputs for one fused step (``K`` given) or one AttnRes-only step (``K`` None).

    ``block_scales`` multiplies saved block ``b`` of every token by
    ``0.5 + 3.5 u_b`` (the AttnRes-only sweep)."""
    if cap is None:
        cap = max(nb, write + 1, 1)
    g = lambda name, shape, scale=1.0, shift=0.0: normal_bf16(  # noqa: E731
        seed, STREAMS[name], layer, shape, scale, shift
    )
    x = W = delta = None
    if K is not None:
        x = g("x", (M, K))
        W = g("W", (H, K), 1.0 / math.sqrt(max(K, 1)))
    if with_delta or K is None:
        delta = g("delta", (M, H))
    prefix = g("prefix", (M, H))
    if block_scales:
        s = 0.5 + 3.5 * uniforms(seed, STREAMS["block_scale"], layer, 0, cap)
        z = normals(seed, STREAMS["blocks"], layer, M * cap * H).reshape(M, cap, H)
        blocks = to_bf16_bits(z * s[None, :, None]).reshape(M, cap, H)
    else:
        blocks = g("blocks", (M, cap, H))
    norm = g("norm", (H,), 0.1, 1.0)
    query = g("query", (H,), 1.0 / math.sqrt(HIDDEN))
    out_norm = g("out_norm", (H,), 0.1, 1.0)
    return StepInputs(
        M=M, K=K or 0, H=H, nb=nb, cap=cap, write=write, has_delta=has_delta,
        final=final, eps=eps, out_eps=out_eps, x=x, W=W, delta=delta,
        prefix=prefix, blocks=blocks, norm=norm, query=query, out_norm=out_norm,
    )


def gemm_inputs(M: int, N: int, K: int, *, seed: int = 0, layer: int = 0):
    """x [M, K] ~ N(0, 1) and W [N, K] ~ N(0, 1)/sqrt(K), bfloat16 bits."""
    x = normal_bf16(seed, STREAMS["x"], layer, (M, K))
    W = normal_bf16(seed, STREAMS["W"], layer, (N, K), 1.0 / math.sqrt(K))
    return x, W


# The five workloads of the decode step, by number.
CONFIGS = {
    0: dict(kind="fused", M=1, K=1024, nb=1, write=-1, has_delta=1),
    1: dict(kind="fused", M=8, K=4096, nb=4, write=-1, has_delta=1),
    2: dict(kind="fused", M=64, K=8192, nb=8, write=8, cap=9, has_delta=1),
    3: dict(kind="attnres", T=256, nb=tuple(range(9)), write=-1, has_delta=1, final=1),
    4: dict(kind="gemm", K=7168, N=4096, M=(1, 8, 16, 64)),
}


def config_inputs(cfg: int, *, final: int = 0, nb: int | None = None, M: int | None = None,
                  layer: int = 0, seed: int = 0):
    """Inputs of workload ``cfg`` (0-2 fused, 3 AttnRes-only, 4 GEMM)."""
    c = CONFIGS[cfg]
    if c["kind"] == "fused":
        return decode_step(c["M"], c["K"], c["nb"], cap=c.get("cap"), write=c["write"],
                           has_delta=c["has_delta"], final=final, seed=seed, layer=layer)
    if c["kind"] == "attnres":
        nb = 8 if nb is None else nb
        return decode_step(c["T"], None, nb, write=-1, has_delta=1, final=1,
                           block_scales=True, seed=seed, layer=layer)
    M = 1 if M is None else M
    return gemm_inputs(M, c["N"], c["K"], seed=seed, layer=layer)
