"""ctypes front end of the FP64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are its only callers. The product path never
imports this package, and this package never imports the product.

All arrays are numpy ``uint16`` arrays holding bfloat16 bit patterns. Functions
copy their inputs, so the caller's arrays are left untouched; in/out tensors
(prefix, blocks) come back as new arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

# Strict IEEE double: no contraction into fused multiply-adds, no reassociation.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm", "-lpthread"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.oracle_gemm.argtypes = [P, I64, P, I64, P, I64, P, I, I, I, I]
        lib.oracle_attnres.argtypes = [P, I64, P, I64, P, I64, I64, I, P, P, P, P, I64, P, I64,
                                       F, F, I, I, I, I, I, I, P, P, P, P, I]
        lib.oracle_attnres_streaming.argtypes = [P, I64, P, I64, P, I64, I64, I, P, P, P, P, I64,
                                                 P, I64, F, F, I, I, I, I, I, I, P, I]
        lib.oracle_attnres_oproj.argtypes = [P, I64, P, I64, I, P, I64, P, I64, I64, I, P, P, P,
                                             P, I64, P, I64, F, F, I, I, I, I, I, I, P, P, I]
        lib.oracle_attnres_pre.argtypes = [P, I64, I64, I, P, P, F, I, I, I, P, I64, P, I]
        lib.oracle_attnres_post.argtypes = [P, I64, P, I64, P, I64, I64, I, P, P, P, P, I64, P,
                                            I64, P, I64, P, F, F, I, I, I, I, I, I, P, I]
        lib.oracle_moe_front.argtypes = [P, I64, P, I64, I, I, I, P, I64, I, I, I, I, I]
        lib.oracle_moe_front.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_bf16_n.argtypes = [P, P, I64]
        lib.oracle_round_bf16_n.restype = None
        for f in ("oracle_gemm", "oracle_attnres", "oracle_attnres_streaming",
                  "oracle_attnres_oproj", "oracle_attnres_pre", "oracle_attnres_post"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def round_bf16(z: float) -> int:
    return int(_load().oracle_round_bf16(float(z)))


def round_bf16_array(z) -> np.ndarray:
    """``round_bf16`` of every element of the float64 array ``z`` (same shape)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    out = np.zeros(z.shape, np.uint16)
    _load().oracle_round_bf16_n(_p(z), _p(out), z.size)
    return out


def gemm(x, W, nthreads: int = 1, exact: bool = False):
    """``y = bf16(x . W^T)`` (-0.0 stored as +0.0); with ``exact`` also the FP64 sums."""
    x, W = _u16(x), _u16(W)
    M, K = x.shape
    N = W.shape[0]
    y = np.zeros((M, N), np.uint16)
    ye = np.zeros((M, N), np.float64) if exact else None
    rc = _load().oracle_gemm(_p(x), K, _p(W), K, _p(y), N, _p(ye), M, N, K, nthreads)
    if rc:
        raise ValueError("oracle_gemm: invalid arguments")
    return (y, ye) if exact else y


@dataclass
class AttnResResult:
    out: np.ndarray
    prefix: np.ndarray
    blocks: np.ndarray | None
    aux: np.ndarray | None
    out_exact: np.ndarray
    h_exact: np.ndarray | None = None
    probs: np.ndarray | None = None
    logits: np.ndarray | None = None
    y: np.ndarray | None = None


def attnres(delta, prefix, blocks, norm, query, out_norm, *, nb, write=-1, has_delta=1,
            final=0, eps=1e-6, out_eps=1e-6, aux=True, nthreads=1, streaming=False):
    """AttnRes for every token of ``delta`` [T, H]; blocks [T, cap, H]."""
    delta, prefix = _u16(delta), _u16(prefix).copy()
    T, H = delta.shape
    if blocks is None:
        blocks = np.zeros((T, 1, H), np.uint16)
    blocks = _u16(blocks).copy()
    cap = blocks.shape[1]
    norm, query, out_norm = _u16(norm), _u16(query), _u16(out_norm)
    out = np.zeros((T, H), np.uint16)
    auxa = np.zeros((T, H), np.uint16) if aux else None
    oe = np.zeros((T, H), np.float64)
    lib = _load()
    if streaming:
        rc = lib.oracle_attnres_streaming(
            _p(delta), H, _p(prefix), H, _p(blocks), cap * H, H, cap, _p(norm), _p(query),
            _p(out_norm), _p(out), H, _p(auxa), H, eps, out_eps, T, H, nb, write, has_delta,
            final, _p(oe), nthreads)
        he = probs = logits = None
    else:
        he = np.zeros((T, H), np.float64)
        probs = np.zeros((T, 9), np.float64)
        logits = np.zeros((T, 9), np.float64)
        rc = lib.oracle_attnres(
            _p(delta), H, _p(prefix), H, _p(blocks), cap * H, H, cap, _p(norm), _p(query),
            _p(out_norm), _p(out), H, _p(auxa), H, eps, out_eps, T, H, nb, write, has_delta,
            final, _p(he), _p(oe), _p(probs), _p(logits), nthreads)
    if rc:
        raise ValueError("oracle_attnres: invalid arguments")
    return AttnResResult(out=out, prefix=prefix, blocks=blocks, aux=auxa, out_exact=oe,
                         h_exact=he, probs=probs, logits=logits)


def attnres_oproj(x, W, prefix, blocks, norm, query, out_norm, *, nb, write=-1, has_delta=1,
                  final=0, eps=1e-6, out_eps=1e-6, aux=True, nthreads=1):
    """Fused step: delta = bf16(x . W^T) (-0.0 -> +0.0), then AttnRes."""
    x, W = _u16(x), _u16(W)
    M, K = x.shape
    H = W.shape[0]
    prefix = _u16(prefix).copy()
    blocks = _u16(blocks).copy()
    cap = blocks.shape[1]
    norm, query, out_norm = _u16(norm), _u16(query), _u16(out_norm)
    out = np.zeros((M, H), np.uint16)
    auxa = np.zeros((M, H), np.uint16) if aux else None
    y = np.zeros((M, H), np.uint16)
    oe = np.zeros((M, H), np.float64)
    rc = _load().oracle_attnres_oproj(
        _p(x), K, _p(W), K, K, _p(prefix), H, _p(blocks), cap * H, H, cap, _p(norm), _p(query),
        _p(out_norm), _p(out), H, _p(auxa), H, eps, out_eps, M, H, nb, write, has_delta, final,
        _p(y), _p(oe), nthreads)
    if rc:
        raise ValueError("oracle_attnres_oproj: invalid arguments")
    return AttnResResult(out=out, prefix=prefix, blocks=blocks, aux=auxa, out_exact=oe, y=y)


def attnres_pre(blocks, norm, query, *, nb, eps=1e-6, nthreads=1):
    """Saved-block statistics of every token of ``blocks`` [T, cap, H]: the
    unnormalised mixture [T, H] and (maximum, exp_sum) [T, 2], in FP64."""
    blocks = _u16(blocks)
    T, cap, H = blocks.shape
    norm, query = _u16(norm), _u16(query)
    mixture = np.zeros((T, H), np.float64)
    scal = np.zeros((T, 2), np.float64)
    rc = _load().oracle_attnres_pre(_p(blocks), cap * H, H, cap, _p(norm), _p(query), eps, T, H,
                                    nb, _p(mixture), H, _p(scal), nthreads)
    if rc:
        raise ValueError("oracle_attnres_pre: invalid arguments")
    return mixture, scal


def attnres_post(delta, prefix, blocks, norm, query, out_norm, mixture, scal, *, nb, write=-1,
                 has_delta=1, final=0, eps=1e-6, out_eps=1e-6, aux=True, nthreads=1):
    """AttnRes post() on given saved-block statistics ``mixture`` [T, H] and
    ``scal`` [T, 2] (any float dtype; widened exactly to FP64)."""
    delta, prefix = _u16(delta), _u16(prefix).copy()
    T, H = delta.shape
    if blocks is None:
        blocks = np.zeros((T, 1, H), np.uint16)
    blocks = _u16(blocks).copy()
    cap = blocks.shape[1]
    norm, query, out_norm = _u16(norm), _u16(query), _u16(out_norm)
    mix64 = np.ascontiguousarray(mixture, dtype=np.float64)
    scal64 = np.ascontiguousarray(scal, dtype=np.float64)
    out = np.zeros((T, H), np.uint16)
    auxa = np.zeros((T, H), np.uint16) if aux else None
    oe = np.zeros((T, H), np.float64)
    rc = _load().oracle_attnres_post(
        _p(delta), H, _p(prefix), H, _p(blocks), cap * H, H, cap, _p(norm), _p(query),
        _p(out_norm), _p(out), H, _p(auxa), H, _p(mix64), H, _p(scal64), eps, out_eps, T, H, nb,
        write, has_delta, final, _p(oe), nthreads)
    if rc:
        raise ValueError("oracle_attnres_post: invalid arguments")
    return AttnResResult(out=out, prefix=prefix, blocks=blocks, aux=auxa, out_exact=oe)


def moe_front(x, W, out, *, router_base, slot, base, valid, split):
    """The MoE-front epilogue of y = x W^T into a copy of ``out`` [M, width]
    (bf16 patterns): router rows c < valid as FP32 words at bf16 column
    router_base + 2 (slot + c), latent rows c >= split as bf16 at column
    base + c - split, the rows between dropped."""
    x, W = _u16(x), _u16(W)
    M, K = x.shape
    N = W.shape[0]
    out = _u16(out).copy()
    rc = _load().oracle_moe_front(_p(x), K, _p(W), K, M, N, K, _p(out), out.shape[1], router_base,
                                  slot, base, valid, split)
    if rc:
        raise ValueError("oracle_moe_front: invalid arguments")
    return out
