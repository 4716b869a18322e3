"""Python binding of libattnres.so (argument marshalling only).

The entry points carry the names of the C ABI in ``include/attnres.h`` and
take torch tensors that live on the GPU: bfloat16 (or 16-bit integer views of
bfloat16 bits) with contiguous rows; carried saved-block statistics are
float32. Every step of the computation
runs in the library's HIP kernels; this module only reads pointers, strides
and the current stream, calls the C function and raises ``AttnResError`` on a
non-zero return code. There is no fallback: without the built library the
import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import _build

LIB_PATH = _build.LIB

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(hipcc --offload-arch=gfx950)"
    )

_lib = ctypes.CDLL(LIB_PATH)
_P, _I64, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib.attnres_run.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _I, _P, _P, _P, _P, _I64, _P,
                             _I64, _F, _F, _I, _I, _I, _I, _I, _I, _P]
_lib.wsgemm_run.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I, _I, _I, _P]
_lib.wsgemm_moe_front_run.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I, _I, _I, _I, _I, _I, _I,
                                      _I, _P]
_lib.wsgemm_workspace_size.argtypes = [_I, _I]
_lib.wsgemm_workspace_size.restype = _SZ
_lib.wsgemm_run_ws.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I, _I, _I, _P, _SZ, _P]
_lib.attnres_oproj_workspace_size.argtypes = [_I, _I, _I]
_lib.attnres_oproj_workspace_size.restype = _SZ
_lib.attnres_oproj_workspace_init.argtypes = [_P, _SZ, _P]
_lib.attnres_oproj_workspace_init.restype = _I
_lib.attnres_oproj_run.argtypes = [_P, _I64, _P, _I64, _I, _P, _I64, _P, _I64, _I64, _I, _P, _P,
                                   _P, _P, _I64, _P, _I64, _F, _F, _I, _I, _I, _I, _I, _I, _P,
                                   _SZ, _P]
_lib.attnres_packed_weights_size.argtypes = [_I, _I]
_lib.attnres_packed_weights_size.restype = _SZ
_lib.attnres_pack_weights.argtypes = [_P, _I64, _I, _I, _P, _SZ, _P]
_lib.attnres_pack_weights.restype = _I
_lib.attnres_oproj_packed_run.argtypes = [_P, _I64, _P, _SZ, _I, _P, _I64, _P, _I64, _I64, _I,
                                          _P, _P, _P, _P, _I64, _P, _I64, _F, _F, _I, _I, _I, _I,
                                          _I, _I, _P, _SZ, _P]
_lib.attnres_oproj_packed_run.restype = _I
_lib.attnres_oproj_run_noalloc.argtypes = [_P, _I64, _P, _I64, _I, _P, _I64, _P, _I64, _I64, _I,
                                           _P, _P, _P, _P, _I64, _P, _I64, _F, _F, _I, _I, _I, _I,
                                           _I, _I, _P]
_lib.attnres_oproj_ahead_run.argtypes = [_P, _I64, _P, _I64, _I, _P, _I64, _P, _I64, _I64, _I,
                                         _P, _P, _P, _P, _I64, _P, _I64, _F, _F, _I, _I, _I, _I,
                                         _I, _I, _P, _P, _F, _P, _I64, _P, _P, _SZ, _P]
_lib.attnres_oproj_packed_ahead_run.argtypes = [_P, _I64, _P, _SZ, _I, _P, _I64, _P, _I64, _I64,
                                                _I, _P, _P, _P, _P, _I64, _P, _I64, _F, _F, _I,
                                                _I, _I, _I, _I, _I, _P, _P, _F, _P, _I64, _P, _P,
                                                _SZ, _P]
_lib.attnres_post_run.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _I, _P, _P, _P, _P, _I64,
                                  _P, _I64, _P, _I64, _P, _F, _F, _I, _I, _I, _I, _I, _I, _P]
_lib.attnres_workspace_status.argtypes = [_P, _SZ, _P]
_lib.attnres_workspace_status.restype = _I
_lib.attnres_stream_read.argtypes = [_P, _SZ, _P, _P]
_lib.attnres_stream_read.restype = _I
_lib.attnres_strerror.argtypes = [_I]
_lib.attnres_strerror.restype = ctypes.c_char_p
for _f in (_lib.attnres_run, _lib.wsgemm_run, _lib.wsgemm_run_ws, _lib.wsgemm_moe_front_run,
           _lib.attnres_oproj_run, _lib.attnres_oproj_run_noalloc,
           _lib.attnres_oproj_ahead_run, _lib.attnres_oproj_packed_ahead_run,
           _lib.attnres_post_run):
    _f.restype = _I

EXPORTS = ("attnres_run", "wsgemm_run", "wsgemm_moe_front_run", "wsgemm_workspace_size",
           "wsgemm_run_ws",
           "attnres_oproj_run", "attnres_oproj_workspace_size",
           "attnres_oproj_workspace_init", "attnres_oproj_ahead_run", "attnres_post_run",
           "attnres_strerror", "attnres_stream_read", "attnres_workspace_status",
           "attnres_oproj_run_noalloc", "attnres_packed_weights_size", "attnres_pack_weights",
           "attnres_oproj_packed_run", "attnres_oproj_packed_ahead_run")

STREAM_READ_SINK_WORDS = 65536  # ATTNRES_STREAM_READ_SINK_WORDS
EWAIT = -7  # ATTNRES_EWAIT: a wait of an earlier call on the workspace gave up


class AttnResError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def attnres_strerror(code: int) -> str:
    return _lib.attnres_strerror(int(code)).decode()


strerror = attnres_strerror


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise AttnResError(-1, "tensors must be on the GPU")
    if t.element_size() != 2:
        raise AttnResError(-1, "tensors must hold 16-bit (bfloat16) elements")
    return ctypes.c_void_p(t.data_ptr())


def _fptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise AttnResError(-1, "tensors must be on the GPU")
    if t.dtype != torch.float32:
        raise AttnResError(-1, "saved-block statistics must be float32")
    return ctypes.c_void_p(t.data_ptr())


def _row_stride(t):
    if t is None:
        return 0
    if t.stride(-1) != 1:
        raise AttnResError(-1, "rows must be contiguous")
    return t.stride(-2) if t.dim() >= 2 else t.shape[-1]


def _rows(t, rows, cols, name):
    """t is a 2-D tensor with at least rows x cols elements (the kernels index
    it by those counts: a smaller tensor would be read or written out of
    bounds)."""
    if t is None:
        return
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols:
        raise AttnResError(-1, f"{name} must be [>= {rows}, >= {cols}], got {tuple(t.shape)}")


def _vec(t, n, name):
    if t is None:
        return
    if t.dim() != 1 or t.shape[0] < n:
        raise AttnResError(-1, f"{name} must hold >= {n} elements, got {tuple(t.shape)}")


def _blocks(t, T, H):
    """blocks [>= T, cap, >= H] (the library checks nb and write against cap)."""
    if t is None:
        return
    if t.dim() != 3 or t.shape[0] < T or t.shape[2] < H:
        raise AttnResError(-1, f"blocks must be [>= {T}, cap, >= {H}], got {tuple(t.shape)}")


def _attn_shapes(T, H, prefix, blocks, norm, query, out_norm, out, aux):
    _rows(prefix, T, H, "prefix")
    _rows(out, T, H, "out")
    _rows(aux, T, H, "aux")
    _blocks(blocks, T, H)
    for t, name in ((norm, "norm"), (query, "query"), (out_norm, "out_norm")):
        _vec(t, H, name)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, where: str):
    if rc != 0:
        raise AttnResError(rc, where)


def attnres_stream_read(src, sink, stream=None):
    """Measurement helper: reads every byte of the contiguous device tensor src
    once (16-byte non-temporal loads); sink (STREAM_READ_SINK_WORDS 32-bit
    words) receives one XOR of the words each workgroup read."""
    if not src.is_contiguous():
        raise AttnResError(-1, "attnres_stream_read: src must be contiguous")
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 4 * STREAM_READ_SINK_WORDS:
        raise AttnResError(-1, "attnres_stream_read: sink too small")
    rc = _lib.attnres_stream_read(ctypes.c_void_p(src.data_ptr() if nbytes else 0), nbytes,
                                  ctypes.c_void_p(sink.data_ptr()), _stream(stream))
    _check(rc, "attnres_stream_read")
    return sink


def wsgemm_run(x, W, y, stream=None):
    """y[M, N] = bf16(x[M, K] W[N, K]^T) (-0.0 stored as +0.0)."""
    M, K = x.shape
    N = W.shape[0]
    _rows(W, N, K, "W")
    _rows(y, M, N, "y")
    rc = _lib.wsgemm_run(_ptr(x), _row_stride(x), _ptr(W), _row_stride(W), _ptr(y),
                         _row_stride(y), M, N, K, _stream(stream))
    _check(rc, "wsgemm_run")
    return y


def wsgemm_moe_front_run(x, W, out, *, router_base, slot, base, valid, split, stream=None):
    """y = x W^T with the MoE-front epilogue into out [M, width] (bf16 patterns):
    rows c < valid as FP32 words at bf16 column router_base + 2 (slot + c), rows
    c >= split as bf16 at column base + c - split, the rows between dropped."""
    M, K = x.shape
    N = W.shape[0]
    _rows(W, N, K, "W")
    # the library bounds the columns by the row stride; a column-sliced view
    # is narrower than its stride, so its own width is checked here
    width = 0
    if valid > 0:
        width = router_base + 2 * (slot + valid)
    if split < N:
        width = max(width, base + N - split)
    _rows(out, M, width, "out")
    rc = _lib.wsgemm_moe_front_run(_ptr(x), _row_stride(x), _ptr(W), _row_stride(W), _ptr(out),
                                   _row_stride(out), M, N, K, router_base, slot, base, valid,
                                   split, _stream(stream))
    _check(rc, "wsgemm_moe_front_run")
    return out


def wsgemm_workspace_size(M: int, N: int) -> int:
    return int(_lib.wsgemm_workspace_size(M, N))


def make_gemm_workspace(M: int, N: int, device="cuda") -> torch.Tensor:
    """A workspace for wsgemm_run_ws: torch allocates it, the library arms it."""
    ws = torch.empty(wsgemm_workspace_size(M, N), dtype=torch.uint8, device=device)
    return attnres_oproj_workspace_init(ws)


def wsgemm_run_ws(x, W, y, workspace, stream=None):
    """wsgemm_run with a workspace (K split across workgroups beyond 32 tokens)."""
    M, K = x.shape
    N = W.shape[0]
    _rows(W, N, K, "W")
    _rows(y, M, N, "y")
    rc = _lib.wsgemm_run_ws(_ptr(x), _row_stride(x), _ptr(W), _row_stride(W), _ptr(y),
                            _row_stride(y), M, N, K, ctypes.c_void_p(workspace.data_ptr()),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "wsgemm_run_ws")
    return y


def attnres_run(delta, prefix, blocks, norm, query, out_norm, out, aux=None, *, nb, write=-1,
                has_delta=1, final_boundary=0, eps=1e-6, out_eps=1e-6, stream=None):
    """AttnRes of T = delta.shape[0] tokens; blocks [T, cap, H] (any token / slot strides)."""
    T, H = delta.shape
    _attn_shapes(T, H, prefix, blocks, norm, query, out_norm, out, aux)
    if blocks is None:
        bst_t = bst_b = cap = 0
    else:
        if blocks.stride(-1) != 1:
            raise AttnResError(-1, "block rows must be contiguous")
        bst_t, bst_b, cap = blocks.stride(0), blocks.stride(1), blocks.shape[1]
    rc = _lib.attnres_run(_ptr(delta), _row_stride(delta), _ptr(prefix), _row_stride(prefix),
                          _ptr(blocks), bst_t, bst_b, cap, _ptr(norm), _ptr(query),
                          _ptr(out_norm), _ptr(out), _row_stride(out), _ptr(aux),
                          _row_stride(aux), eps, out_eps, T, H, nb, write, int(has_delta),
                          int(final_boundary), _stream(stream))
    _check(rc, "attnres_run")
    return out, prefix, blocks


def attnres_oproj_workspace_size(M: int, H: int, nb: int) -> int:
    return int(_lib.attnres_oproj_workspace_size(M, H, nb))


def attnres_workspace_status(workspace, stream=None) -> int:
    """Waits for the work enqueued on the stream, then returns 0 when no wait of
    a call on this workspace gave up, EWAIT when one did (that call's outputs
    are invalid and later calls write nothing until the workspace is re-armed
    by attnres_oproj_workspace_init). workspace=None: the library's own array
    of attnres_oproj_run_noalloc on the current device."""
    if workspace is None:
        ptr, nbytes = None, 0
    else:
        ptr, nbytes = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    rc = _lib.attnres_workspace_status(ptr, nbytes, _stream(stream))
    if rc not in (0, EWAIT):
        raise AttnResError(rc, "attnres_workspace_status")
    return rc


workspace_status = attnres_workspace_status


def check_workspace(workspace, stream=None):
    """Raises AttnResError(EWAIT) if a wait of a call on this workspace gave up."""
    _check(attnres_workspace_status(workspace, stream), "attnres_workspace_status")


def attnres_oproj_workspace_init(workspace, stream=None):
    """Arms a workspace once after allocation (see attnres_oproj_workspace_init)."""
    rc = _lib.attnres_oproj_workspace_init(ctypes.c_void_p(workspace.data_ptr()),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(stream))
    _check(rc, "attnres_oproj_workspace_init")
    return workspace


def make_workspace(M: int, H: int, nb: int, device="cuda") -> torch.Tensor:
    """A workspace for attnres_oproj_run: torch allocates it, the library arms it."""
    ws = torch.empty(attnres_oproj_workspace_size(M, H, nb), dtype=torch.uint8, device=device)
    return attnres_oproj_workspace_init(ws)


def attnres_oproj_run(x, W, prefix, blocks, norm, query, out_norm, out, aux, workspace, *, nb,
                      write=-1, has_delta=1, final_boundary=0, eps=1e-6, out_eps=1e-6,
                      stream=None):
    """Fused o-projection + AttnRes: delta = bf16(x W^T), then AttnRes (T = M).

    The call only enqueues work. Its outputs are valid when
    attnres_workspace_status(workspace) returns 0 afterwards (a wait that gave
    up, a safety bound a healthy device never reaches, leaves them invalid)."""
    M, K = x.shape
    H = W.shape[0]
    _rows(W, H, K, "W")
    _attn_shapes(M, H, prefix, blocks, norm, query, out_norm, out, aux)
    if blocks is None:
        bst_t = bst_b = cap = 0
    else:
        if blocks.stride(-1) != 1:
            raise AttnResError(-1, "block rows must be contiguous")
        bst_t, bst_b, cap = blocks.stride(0), blocks.stride(1), blocks.shape[1]
    ws = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.attnres_oproj_run(_ptr(x), _row_stride(x), _ptr(W), _row_stride(W), K, _ptr(prefix),
                                _row_stride(prefix), _ptr(blocks), bst_t, bst_b, cap, _ptr(norm),
                                _ptr(query), _ptr(out_norm), _ptr(out), _row_stride(out),
                                _ptr(aux), _row_stride(aux), eps, out_eps, M, H, nb, write,
                                int(has_delta), int(final_boundary), ws, wsb, _stream(stream))
    _check(rc, "attnres_oproj_run")
    return out, prefix, blocks


def attnres_packed_weights_size(N: int, K: int) -> int:
    return int(_lib.attnres_packed_weights_size(N, K))


def attnres_pack_weights(W, Wp=None, stream=None):
    """W [N, K] in the prepared (tile-major) layout of attnres_oproj_packed_run;
    Wp (uint8 or 16-bit, at least attnres_packed_weights_size(N, K) bytes) is
    allocated here by torch when not given. Returns Wp."""
    N, K = W.shape
    nbytes = attnres_packed_weights_size(N, K)
    if Wp is None:
        Wp = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=W.device)
    have = Wp.numel() * Wp.element_size()
    if have < nbytes:
        raise AttnResError(-1, f"Wp must hold >= {nbytes} bytes, got {have}")
    rc = _lib.attnres_pack_weights(_ptr(W), _row_stride(W), N, K,
                                   ctypes.c_void_p(Wp.data_ptr()), have, _stream(stream))
    _check(rc, "attnres_pack_weights")
    return Wp


def attnres_oproj_packed_run(x, Wp, H, prefix, blocks, norm, query, out_norm, out, aux, workspace,
                             *, nb, write=-1, has_delta=1, final_boundary=0, eps=1e-6,
                             out_eps=1e-6, stream=None):
    """attnres_oproj_run with W [H, K] given as attnres_pack_weights(W)."""
    M, K = x.shape
    _attn_shapes(M, H, prefix, blocks, norm, query, out_norm, out, aux)
    have = Wp.numel() * Wp.element_size()
    if have < attnres_packed_weights_size(H, K):
        raise AttnResError(-1, f"Wp must hold >= {attnres_packed_weights_size(H, K)} bytes")
    if not Wp.is_cuda:
        raise AttnResError(-1, "tensors must be on the GPU")
    bst_t, bst_b, cap = _block_strides(blocks)
    ws = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.attnres_oproj_packed_run(
        _ptr(x), _row_stride(x), ctypes.c_void_p(Wp.data_ptr()), have, K, _ptr(prefix),
        _row_stride(prefix), _ptr(blocks), bst_t, bst_b, cap, _ptr(norm), _ptr(query),
        _ptr(out_norm), _ptr(out), _row_stride(out), _ptr(aux), _row_stride(aux), eps, out_eps, M,
        H, nb, write, int(has_delta), int(final_boundary), ws, wsb, _stream(stream))
    _check(rc, "attnres_oproj_packed_run")
    return out, prefix, blocks


def attnres_oproj_run_noalloc(x, W, prefix, blocks, norm, query, out_norm, out, aux, *, nb,
                              write=-1, has_delta=1, final_boundary=0, eps=1e-6, out_eps=1e-6,
                              stream=None):
    """attnres_oproj_run with the library's own workspace (no allocation by the
    library or here); calls that overlap on one device race."""
    M, K = x.shape
    H = W.shape[0]
    _rows(W, H, K, "W")
    _attn_shapes(M, H, prefix, blocks, norm, query, out_norm, out, aux)
    bst_t, bst_b, cap = _block_strides(blocks)
    rc = _lib.attnres_oproj_run_noalloc(
        _ptr(x), _row_stride(x), _ptr(W), _row_stride(W), K, _ptr(prefix), _row_stride(prefix),
        _ptr(blocks), bst_t, bst_b, cap, _ptr(norm), _ptr(query), _ptr(out_norm), _ptr(out),
        _row_stride(out), _ptr(aux), _row_stride(aux), eps, out_eps, M, H, nb, write,
        int(has_delta), int(final_boundary), _stream(stream))
    _check(rc, "attnres_oproj_run_noalloc")
    return out, prefix, blocks


def _block_strides(blocks):
    if blocks is None:
        return 0, 0, 0
    if blocks.stride(-1) != 1:
        raise AttnResError(-1, "block rows must be contiguous")
    return blocks.stride(0), blocks.stride(1), blocks.shape[1]


def attnres_oproj_ahead_run(x, W, prefix, blocks, norm, query, out_norm, out, aux, workspace,
                            next_norm, next_query, mixture, scal, *, nb, write=-1, has_delta=1,
                            final_boundary=0, eps=1e-6, out_eps=1e-6, next_eps=1e-6,
                            stream=None):
    """attnres_oproj_run that also stores the saved-block statistics of the next
    layer's AttnRes (weights next_norm * next_query, next_eps) over the same
    saved blocks: mixture [M, H] and scal [M, 2] (maximum, exp_sum), float32."""
    M, K = x.shape
    H = W.shape[0]
    _rows(W, H, K, "W")
    _attn_shapes(M, H, prefix, blocks, norm, query, out_norm, out, aux)
    _vec(next_norm, H, "next_norm")
    _vec(next_query, H, "next_query")
    _rows(mixture, M, H, "mixture")
    if scal is not None and scal.numel() < 2 * M:
        raise AttnResError(-1, f"scal must hold >= {2 * M} floats")
    bst_t, bst_b, cap = _block_strides(blocks)
    ws = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if mixture is not None and mixture.stride(-1) != 1:
        raise AttnResError(-1, "mixture rows must be contiguous")
    rc = _lib.attnres_oproj_ahead_run(
        _ptr(x), _row_stride(x), _ptr(W), _row_stride(W), K, _ptr(prefix), _row_stride(prefix),
        _ptr(blocks), bst_t, bst_b, cap, _ptr(norm), _ptr(query), _ptr(out_norm), _ptr(out),
        _row_stride(out), _ptr(aux), _row_stride(aux), eps, out_eps, M, H, nb, write,
        int(has_delta), int(final_boundary), _ptr(next_norm), _ptr(next_query), next_eps,
        _fptr(mixture), 0 if mixture is None else mixture.stride(0), _fptr(scal), ws, wsb,
        _stream(stream))
    _check(rc, "attnres_oproj_ahead_run")
    return out, prefix, blocks, mixture, scal


def attnres_oproj_packed_ahead_run(x, Wp, H, prefix, blocks, norm, query, out_norm, out, aux,
                                   workspace, next_norm, next_query, mixture, scal, *, nb,
                                   write=-1, has_delta=1, final_boundary=0, eps=1e-6, out_eps=1e-6,
                                   next_eps=1e-6, stream=None):
    """attnres_oproj_ahead_run with W [H, K] given as attnres_pack_weights(W)."""
    M, K = x.shape
    _attn_shapes(M, H, prefix, blocks, norm, query, out_norm, out, aux)
    have = Wp.numel() * Wp.element_size()
    if have < attnres_packed_weights_size(H, K):
        raise AttnResError(-1, f"Wp must hold >= {attnres_packed_weights_size(H, K)} bytes")
    if not Wp.is_cuda:
        raise AttnResError(-1, "tensors must be on the GPU")
    _vec(next_norm, H, "next_norm")
    _vec(next_query, H, "next_query")
    _rows(mixture, M, H, "mixture")
    if scal is not None and scal.numel() < 2 * M:
        raise AttnResError(-1, f"scal must hold >= {2 * M} floats")
    if mixture is not None and mixture.stride(-1) != 1:
        raise AttnResError(-1, "mixture rows must be contiguous")
    bst_t, bst_b, cap = _block_strides(blocks)
    ws = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.attnres_oproj_packed_ahead_run(
        _ptr(x), _row_stride(x), ctypes.c_void_p(Wp.data_ptr()), have, K, _ptr(prefix),
        _row_stride(prefix), _ptr(blocks), bst_t, bst_b, cap, _ptr(norm), _ptr(query),
        _ptr(out_norm), _ptr(out), _row_stride(out), _ptr(aux), _row_stride(aux), eps, out_eps, M,
        H, nb, write, int(has_delta), int(final_boundary), _ptr(next_norm), _ptr(next_query),
        next_eps, _fptr(mixture), 0 if mixture is None else mixture.stride(0), _fptr(scal), ws,
        wsb, _stream(stream))
    _check(rc, "attnres_oproj_packed_ahead_run")
    return out, prefix, blocks, mixture, scal


def attnres_post_run(delta, prefix, blocks, norm, query, out_norm, out, aux, mixture, scal, *,
                     nb, write=-1, has_delta=1, final_boundary=0, eps=1e-6, out_eps=1e-6,
                     stream=None):
    """AttnRes post() on carried saved-block statistics (mixture [T, H] and scal
    [T, 2], float32, of nb saved blocks); blocks is only written (slot write)."""
    T, H = delta.shape
    _attn_shapes(T, H, prefix, blocks, norm, query, out_norm, out, aux)
    _rows(mixture, T, H, "mixture")
    if scal is not None and scal.numel() < 2 * T:
        raise AttnResError(-1, f"scal must hold >= {2 * T} floats")
    bst_t, bst_b, cap = _block_strides(blocks)
    if mixture is not None and mixture.stride(-1) != 1:
        raise AttnResError(-1, "mixture rows must be contiguous")
    rc = _lib.attnres_post_run(
        _ptr(delta), _row_stride(delta), _ptr(prefix), _row_stride(prefix), _ptr(blocks), bst_t,
        bst_b, cap, _ptr(norm), _ptr(query), _ptr(out_norm), _ptr(out), _row_stride(out),
        _ptr(aux), _row_stride(aux), _fptr(mixture), 0 if mixture is None else mixture.stride(0),
        _fptr(scal), eps, out_eps, T, H, nb, write, int(has_delta), int(final_boundary),
        _stream(stream))
    _check(rc, "attnres_post_run")
    return out, prefix, blocks
