"""The C-ABI library: it loads without a GPU, exports every entry point the
header declares, and rejects invalid arguments on the host (no HIP call is
made by any case here)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")


@pytest.fixture(scope="module")
def lib():
    from skinny_gemm_attention_amd import _build

    if _build.stale():
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    P, I64, I, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attnres_run.argtypes = [P, I64, P, I64, P, I64, I64, I, P, P, P, P, I64, P, I64, F, F, I, I,
                              I, I, I, I, P]
    L.wsgemm_run.argtypes = [P, I64, P, I64, P, I64, I, I, I, P]
    L.wsgemm_moe_front_run.argtypes = [P, I64, P, I64, P, I64, I, I, I, I, I, I, I, I, P]
    L.wsgemm_workspace_size.argtypes = [I, I]
    L.wsgemm_workspace_size.restype = SZ
    L.wsgemm_run_ws.argtypes = [P, I64, P, I64, P, I64, I, I, I, P, SZ, P]
    L.attnres_oproj_run.argtypes = [P, I64, P, I64, I, P, I64, P, I64, I64, I, P, P, P, P, I64, P,
                                    I64, F, F, I, I, I, I, I, I, P, SZ, P]
    L.attnres_oproj_workspace_size.argtypes = [I, I, I]
    L.attnres_oproj_workspace_size.restype = SZ
    L.attnres_oproj_workspace_init.argtypes = [P, SZ, P]
    L.attnres_oproj_ahead_run.argtypes = [P, I64, P, I64, I, P, I64, P, I64, I64, I, P, P, P, P,
                                          I64, P, I64, F, F, I, I, I, I, I, I, P, P, F, P, I64, P,
                                          P, SZ, P]
    L.attnres_post_run.argtypes = [P, I64, P, I64, P, I64, I64, I, P, P, P, P, I64, P, I64, P, I64,
                                   P, F, F, I, I, I, I, I, I, P]
    L.attnres_oproj_run_noalloc.argtypes = [P, I64, P, I64, I, P, I64, P, I64, I64, I, P, P, P,
                                            P, I64, P, I64, F, F, I, I, I, I, I, I, P]
    L.attnres_packed_weights_size.argtypes = [I, I]
    L.attnres_packed_weights_size.restype = SZ
    L.attnres_pack_weights.argtypes = [P, I64, I, I, P, SZ, P]
    L.attnres_oproj_packed_run.argtypes = [P, I64, P, SZ, I, P, I64, P, I64, I64, I, P, P, P, P,
                                           I64, P, I64, F, F, I, I, I, I, I, I, P, SZ, P]
    L.attnres_oproj_packed_ahead_run.argtypes = [P, I64, P, SZ, I, P, I64, P, I64, I64, I, P, P,
                                                 P, P, I64, P, I64, F, F, I, I, I, I, I, I, P, P,
                                                 F, P, I64, P, P, SZ, P]
    L.attnres_workspace_status.argtypes = [P, SZ, P]
    L.attnres_workspace_status.restype = I
    L.attnres_stream_read.argtypes = [P, SZ, P, P]
    L.attnres_stream_read.restype = I
    L.attnres_strerror.argtypes = [I]
    L.attnres_strerror.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\(", text, flags=re.M)


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) == {"attnres_run", "wsgemm_run", "wsgemm_workspace_size", "wsgemm_run_ws",
                          "wsgemm_moe_front_run",
                          "attnres_oproj_workspace_size",
                          "attnres_oproj_workspace_init", "attnres_oproj_run",
                          "attnres_oproj_ahead_run", "attnres_post_run", "attnres_strerror",
                          "attnres_stream_read", "attnres_workspace_status",
                          "attnres_oproj_run_noalloc", "attnres_packed_weights_size",
                          "attnres_pack_weights", "attnres_oproj_packed_run",
                          "attnres_oproj_packed_ahead_run"}
    for n in names:
        assert hasattr(lib, n), n


def test_binding_names_match_header():
    import skinny_gemm_attention_amd as sga

    for n in declared_functions():
        assert n in sga.EXPORTS and hasattr(sga, n), n


def test_strerror_and_workspace(lib):
    codes = {0: b"success", -1: b"invalid", -2: b"aligned", -3: b"range", -4: b"supported",
             -5: b"workspace", -6: b"HIP", -7: b"gave up"}
    for c, word in codes.items():
        assert word in lib.attnres_strerror(c)
    assert b"unknown" in lib.attnres_strerror(-99)
    # header, bf16 mailbox rows and, beyond 32 tokens, the split-K hand-off
    # (per 64-row group one 16-byte quad per MFMA output quad)
    assert lib.attnres_oproj_workspace_size(32, 7168, 8) == 256 + 32 * 7168 * 2
    assert lib.attnres_oproj_workspace_size(64, 7168, 8) == 256 + 64 * 7168 * 2 + 112 * 1024 * 16
    assert lib.attnres_oproj_workspace_size(33, 8192, 8) == 256 + 33 * 8192 * 2 + 128 * 768 * 16
    assert lib.attnres_oproj_workspace_size(1, 8, 0) == 512
    # host-side rejections of the init call (no launch happens)
    assert lib.attnres_oproj_workspace_init(None, 1024, None) == -5
    assert lib.attnres_oproj_workspace_init(A + 16, 1024, None) == -5
    assert lib.attnres_oproj_workspace_init(A, 128, None) == -5
    assert lib.attnres_oproj_workspace_init(A, 1026, None) == -5


# Fake, 256-byte-aligned addresses: validation only looks at their values.
A = 0x10000
H = 7168


def attn_args(**kw):
    a = dict(delta=A, ld_delta=H, prefix=A, ld_prefix=H, blocks=A, bst_t=9 * H, bst_b=H, cap=9,
             norm=A, query=A, out_norm=A, out=A, ld_out=H, aux=A, ld_aux=H, eps=1e-6,
             out_eps=1e-6, T=4, H=H, nb=8, write=8, has_delta=1, final=0, stream=None)
    a.update(kw)
    return a


def call_attn(lib, a):
    return lib.attnres_run(a["delta"], a["ld_delta"], a["prefix"], a["ld_prefix"], a["blocks"],
                           a["bst_t"], a["bst_b"], a["cap"], a["norm"], a["query"],
                           a["out_norm"], a["out"], a["ld_out"], a["aux"], a["ld_aux"], a["eps"],
                           a["out_eps"], a["T"], a["H"], a["nb"], a["write"], a["has_delta"],
                           a["final"], a["stream"])


@pytest.mark.parametrize("change,code", [
    (dict(delta=None), -1), (dict(prefix=None), -1), (dict(norm=None), -1), (dict(out=None), -1),
    (dict(T=-1), -1), (dict(has_delta=2), -1), (dict(final=3), -1), (dict(eps=-1.0), -1),
    (dict(eps=float("nan")), -1), (dict(ld_delta=H - 8), -1), (dict(ld_out=100), -1),
    (dict(H=7160 + 4), -4), (dict(H=0), -4), (dict(H=8200), -4),
    (dict(nb=9, cap=10, bst_t=10 * H), -3), (dict(nb=-1), -3), (dict(nb=8, cap=7, write=-1, bst_t=7 * H), -3),
    (dict(write=9), -3), (dict(write=-2), -3),
    (dict(blocks=None), -1), (dict(bst_b=H - 8), -1), (dict(bst_t=8 * H), -1),
    (dict(delta=A + 8), -2), (dict(out=A + 2), -2), (dict(aux=A + 4), -2), (dict(blocks=A + 8), -2),
    (dict(ld_out=H + 4), -2), (dict(bst_b=H + 4, bst_t=9 * H + 36), -2),
])
def test_attnres_run_rejects(lib, change, code):
    assert call_attn(lib, attn_args(**change)) == code


def test_attnres_run_empty_is_a_noop(lib):
    assert call_attn(lib, attn_args(T=0)) == 0


def call_gemm(lib, x=A, ldx=1024, W=A, ldw=1024, y=A, ldy=4096, M=8, N=4096, K=1024):
    return lib.wsgemm_run(x, ldx, W, ldw, y, ldy, M, N, K, None)


@pytest.mark.parametrize("change,code", [
    (dict(x=None), -1), (dict(W=None), -1), (dict(y=None), -1), (dict(M=-1), -1), (dict(K=-8), -1),
    (dict(M=65), -3), (dict(N=4), -4), (dict(N=4100), -4), (dict(K=1020, ldx=1024), -4),
    (dict(ldx=1016), -1), (dict(ldy=4088), -1), (dict(x=A + 8), -2), (dict(ldw=1028), -2),
])
def test_wsgemm_run_rejects(lib, change, code):
    assert call_gemm(lib, **change) == code


def test_wsgemm_run_empty_is_a_noop(lib):
    assert call_gemm(lib, M=0) == 0


def call_fused(lib, **kw):
    a = attn_args()
    a.update(x=A, ldx=8192, W=A, ldw=8192, K=8192, ws=A, wsb=256 + 4 * 7168 * 2, M=4)
    a.update(kw)
    return lib.attnres_oproj_run(a["x"], a["ldx"], a["W"], a["ldw"], a["K"], a["prefix"],
                                 a["ld_prefix"], a["blocks"], a["bst_t"], a["bst_b"], a["cap"],
                                 a["norm"], a["query"], a["out_norm"], a["out"], a["ld_out"],
                                 a["aux"], a["ld_aux"], a["eps"], a["out_eps"], a["M"], a["H"],
                                 a["nb"], a["write"], a["has_delta"], a["final"], a["ws"],
                                 a["wsb"], None)


@pytest.mark.parametrize("change,code", [
    (dict(x=None), -1), (dict(W=None), -1), (dict(M=0), -3), (dict(M=65), -3), (dict(K=8190), -4),
    (dict(ldx=4096), -1), (dict(W=A + 8), -2), (dict(ws=None), -5), (dict(wsb=8), -5), (dict(wsb=256 + 4 * 7168 * 2 - 2), -5),
    (dict(ws=A + 16), -5), (dict(nb=9, cap=10, bst_t=10 * H), -3), (dict(H=100), -4),
])
def test_attnres_oproj_run_rejects(lib, change, code):
    assert call_fused(lib, **change) == code


def call_noalloc(lib, **kw):
    a = attn_args()
    a.update(x=A, ldx=8192, W=A, ldw=8192, K=8192, M=4)
    a.update(kw)
    return lib.attnres_oproj_run_noalloc(
        a["x"], a["ldx"], a["W"], a["ldw"], a["K"], a["prefix"], a["ld_prefix"], a["blocks"],
        a["bst_t"], a["bst_b"], a["cap"], a["norm"], a["query"], a["out_norm"], a["out"],
        a["ld_out"], a["aux"], a["ld_aux"], a["eps"], a["out_eps"], a["M"], a["H"], a["nb"],
        a["write"], a["has_delta"], a["final"], None)


@pytest.mark.parametrize("change,code", [
    (dict(x=None), -1), (dict(W=None), -1), (dict(M=0), -3), (dict(M=65), -3), (dict(K=8190), -4),
    (dict(ldx=4096), -1), (dict(W=A + 8), -2), (dict(nb=9, cap=10, bst_t=10 * H), -3),
    (dict(H=100), -4), (dict(H=8200), -4), (dict(prefix=None), -1),
])
def test_attnres_oproj_run_noalloc_rejects(lib, change, code):
    """Every argument is checked before the library's array is looked up or
    armed (no HIP call is made by any case here)."""
    assert call_noalloc(lib, **change) == code


def test_noalloc_array_covers_every_fused_workspace(lib):
    m = re.search(r"#define ATTNRES_NOALLOC_WORKSPACE_BYTES (\d+)", open(HEADER).read())
    biggest = lib.attnres_oproj_workspace_size(64, 8192, 8)
    assert m and int(m.group(1)) == biggest == 3_145_984


def call_ahead(lib, **kw):
    a = attn_args()
    a.update(x=A, ldx=8192, W=A, ldw=8192, K=8192, ws=A, wsb=256 + 4 * 7168 * 2, M=4,
             next_norm=A, next_query=A, next_eps=1e-6, mix=A, ld_mix=H, scal=A)
    a.update(kw)
    return lib.attnres_oproj_ahead_run(
        a["x"], a["ldx"], a["W"], a["ldw"], a["K"], a["prefix"], a["ld_prefix"], a["blocks"],
        a["bst_t"], a["bst_b"], a["cap"], a["norm"], a["query"], a["out_norm"], a["out"],
        a["ld_out"], a["aux"], a["ld_aux"], a["eps"], a["out_eps"], a["M"], a["H"], a["nb"],
        a["write"], a["has_delta"], a["final"], a["next_norm"], a["next_query"], a["next_eps"],
        a["mix"], a["ld_mix"], a["scal"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("change,code", [
    (dict(next_norm=None), -1), (dict(next_query=None), -1), (dict(mix=None), -1),
    (dict(scal=None), -1), (dict(next_eps=-1.0), -1), (dict(next_eps=float("nan")), -1),
    (dict(ld_mix=H - 8), -1), (dict(mix=A + 8), -2), (dict(scal=A + 4), -2),
    (dict(ld_mix=H + 4), -2), (dict(next_norm=A + 2), -2),
    # the attnres_oproj_run checks still apply
    (dict(M=0), -3), (dict(x=None), -1), (dict(ws=None), -5), (dict(H=100), -4),
])
def test_attnres_oproj_ahead_run_rejects(lib, change, code):
    assert call_ahead(lib, **change) == code


def call_post(lib, **kw):
    a = attn_args()
    a.update(mix=A, ld_mix=H, scal=A)
    a.update(kw)
    return lib.attnres_post_run(
        a["delta"], a["ld_delta"], a["prefix"], a["ld_prefix"], a["blocks"], a["bst_t"],
        a["bst_b"], a["cap"], a["norm"], a["query"], a["out_norm"], a["out"], a["ld_out"],
        a["aux"], a["ld_aux"], a["mix"], a["ld_mix"], a["scal"], a["eps"], a["out_eps"], a["T"],
        a["H"], a["nb"], a["write"], a["has_delta"], a["final"], a["stream"])


@pytest.mark.parametrize("change,code", [
    (dict(mix=None), -1), (dict(scal=None), -1), (dict(ld_mix=H - 8), -1),
    (dict(mix=A + 8), -2), (dict(scal=A + 4), -2), (dict(ld_mix=H + 4), -2),
    (dict(nb=9), -3), (dict(nb=-1), -3), (dict(write=9), -3),
    (dict(delta=None), -1), (dict(T=-1), -1), (dict(H=100), -4),
    # blocks are written only: not needed without a written slot ...
    (dict(blocks=None, write=8), -1),
    # ... and nb may exceed cap (the statistics stand in for the blocks):
    # this call fails on the missing delta, not on nb > cap
    (dict(nb=8, cap=1, write=-1, bst_t=H, delta=None), -1),
])
def test_attnres_post_run_rejects(lib, change, code):
    assert call_post(lib, **change) == code


def test_attnres_post_run_empty_is_a_noop(lib):
    assert call_post(lib, T=0) == 0


def test_wsgemm_workspace_size(lib):
    # header, and beyond 32 tokens three parts per 64-row group of one
    # 16-byte quad per MFMA output quad
    assert lib.wsgemm_workspace_size(32, 4096) == 256
    assert lib.wsgemm_workspace_size(64, 4096) == 256 + 3 * 64 * 1024 * 16
    assert lib.wsgemm_workspace_size(33, 1000) == 256 + 3 * 16 * 768 * 16
    assert lib.wsgemm_workspace_size(128, 4096) == 256 + 3 * 64 * 2048 * 16
    assert lib.wsgemm_workspace_size(-1, 8) == 0


def call_gemm_ws(lib, ws=A, wsb=256 + 3 * 64 * 1024 * 16, **kw):
    a = dict(x=A, ldx=1024, W=A, ldw=1024, y=A, ldy=4096, M=64, N=4096, K=1024)
    a.update(kw)
    return lib.wsgemm_run_ws(a["x"], a["ldx"], a["W"], a["ldw"], a["y"], a["ldy"], a["M"],
                             a["N"], a["K"], ws, wsb, None)


@pytest.mark.parametrize("change,code", [
    (dict(ws=None), -5), (dict(ws=A + 16), -5), (dict(wsb=256), -5),
    (dict(x=None), -1), (dict(M=129), -3), (dict(N=4100), -4), (dict(ldy=4088), -1),
    (dict(x=A + 8), -2),
    # beyond 64 tokens only the K split serves: K >= 256 and 2 ceil(N/64) <= 256
    (dict(M=65, K=248, ldx=248, ldw=248), -4), (dict(M=65, N=16392, ldy=16392), -4),
])
def test_wsgemm_run_ws_rejects(lib, change, code):
    assert call_gemm_ws(lib, **change) == code


def test_wsgemm_run_ws_empty_is_a_noop(lib):
    assert call_gemm_ws(lib, M=0, ws=None) == 0


def call_moe(lib, **kw):
    a = dict(x=A, ldx=1024, W=A, ldw=1024, out=A, ld_out=7168, M=8, N=4096, K=1024,
             router_base=3584, slot=0, base=0, valid=384, split=512)
    a.update(kw)
    return lib.wsgemm_moe_front_run(a["x"], a["ldx"], a["W"], a["ldw"], a["out"], a["ld_out"],
                                    a["M"], a["N"], a["K"], a["router_base"], a["slot"],
                                    a["base"], a["valid"], a["split"], None)


@pytest.mark.parametrize("change,code", [
    (dict(valid=520), -3), (dict(split=4104), -3), (dict(split=376), -3), (dict(slot=-1), -3),
    (dict(valid=380), -2), (dict(split=516), -2), (dict(router_base=3585), -2),
    (dict(base=3), -2), (dict(slot=1600), -3), (dict(base=3600), -3),
    (dict(base=100), -3),  # latent columns 100..3683 would overlap the router words
    (dict(out=None), -1), (dict(M=65), -3), (dict(out=A + 8), -2), (dict(ld_out=7164), -2),
])
def test_wsgemm_moe_front_run_rejects(lib, change, code):
    assert call_moe(lib, **change) == code


def test_wsgemm_moe_front_run_empty_is_a_noop(lib):
    assert call_moe(lib, M=0) == 0


def test_stream_read_host_checks(lib):
    """attnres_stream_read rejects bad arguments on the host (nothing is
    launched: the pointers below are never dereferenced)."""
    fake = ctypes.c_void_p(1 << 40)  # 16-byte aligned, never touched
    assert lib.attnres_stream_read(fake, 64, None, None) == -1          # no sink
    assert lib.attnres_stream_read(None, 64, fake, None) == -1          # no source
    assert lib.attnres_stream_read(fake, 40, fake, None) == -2          # bytes % 16
    assert lib.attnres_stream_read(ctypes.c_void_p((1 << 40) + 8), 64, fake, None) == -2
    assert lib.attnres_stream_read(fake, 64, ctypes.c_void_p((1 << 40) + 2), None) == -2


def test_stream_read_sink_words_match_header():
    import skinny_gemm_attention_amd as sga

    m = re.search(r"#define ATTNRES_STREAM_READ_SINK_WORDS (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == sga.STREAM_READ_SINK_WORDS


def test_workspace_status_host_checks(lib):
    """attnres_workspace_status rejects a missing, short or misaligned
    workspace before any HIP call (the pointers are never dereferenced)."""
    fake = 1 << 40
    assert lib.attnres_workspace_status(None, 4096, None) == -5
    assert lib.attnres_workspace_status(ctypes.c_void_p(fake), 255, None) == -5
    assert lib.attnres_workspace_status(ctypes.c_void_p(fake + 16), 4096, None) == -5


def test_error_codes_match_header():
    import skinny_gemm_attention_amd as sga

    text = open(HEADER).read()
    codes = dict((n, int(v)) for n, v in re.findall(r"#define ATTNRES_(E\w+) \((-\d+)\)", text))
    assert codes["EWAIT"] == sga.EWAIT == -7


def test_packed_weights_size(lib):
    """4 ceil(K / 512) planes of 256-byte segments, one per row."""
    assert lib.attnres_packed_weights_size(7168, 4096) == 7168 * 4096 * 2
    assert lib.attnres_packed_weights_size(7168, 1000) == 7168 * 256 * 8
    assert lib.attnres_packed_weights_size(16, 8) == 16 * 256 * 4
    assert lib.attnres_packed_weights_size(16, 0) == 0


def test_pack_weights_host_checks(lib):
    """Every rejection happens on the host (no case here reaches a launch:
    the pointers are never dereferenced)."""
    fake = 1 << 40
    W, Wp = ctypes.c_void_p(fake), ctypes.c_void_p(fake + (1 << 30))
    big = 1 << 30
    assert lib.attnres_pack_weights(None, 4096, 8, 4096, Wp, big, None) == -1
    assert lib.attnres_pack_weights(W, 4000, 8, 4096, Wp, big, None) == -1          # ldw < K
    assert lib.attnres_pack_weights(W, 4096, 8, 4092, Wp, big, None) == -4          # K % 8
    assert lib.attnres_pack_weights(ctypes.c_void_p(fake + 8), 4096, 8, 4096, Wp, big, None) == -2
    assert lib.attnres_pack_weights(W, 4100, 8, 4096, Wp, big, None) == -2          # ldw % 8
    assert lib.attnres_pack_weights(W, 4096, 8, 4096, Wp, 8 * 4096 * 2 - 16, None) == -1
    assert lib.attnres_pack_weights(W, 4096, 0, 4096, Wp, 0, None) == 0            # nothing to do


def call_packed(lib, **kw):
    a = attn_args()
    a.update(x=A, ldx=8192, Wp=A, wpb=7168 * 8192 * 2, K=8192, ws=A, wsb=256 + 4 * 7168 * 2, M=4)
    a.update(kw)
    return lib.attnres_oproj_packed_run(
        a["x"], a["ldx"], a["Wp"], a["wpb"], a["K"], a["prefix"], a["ld_prefix"], a["blocks"],
        a["bst_t"], a["bst_b"], a["cap"], a["norm"], a["query"], a["out_norm"], a["out"],
        a["ld_out"], a["aux"], a["ld_aux"], a["eps"], a["out_eps"], a["M"], a["H"], a["nb"],
        a["write"], a["has_delta"], a["final"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("change,code", [
    (dict(x=None), -1), (dict(Wp=None), -1), (dict(M=0), -3), (dict(M=65), -3),
    (dict(K=8190), -4), (dict(ldx=4096), -1), (dict(Wp=A + 8), -2), (dict(ws=None), -5),
    (dict(wpb=7168 * 8192 * 2 - 256), -1), (dict(H=100), -4),
])
def test_attnres_oproj_packed_run_rejects(lib, change, code):
    assert call_packed(lib, **change) == code


def call_packed_ahead(lib, **kw):
    a = attn_args()
    a.update(x=A, ldx=8192, Wp=A, wpb=7168 * 8192 * 2, K=8192, ws=A, wsb=256 + 4 * 7168 * 2, M=4,
             nn=A, nq=A, neps=1e-6, mix=A, ldm=7168, scal=A)
    a.update(kw)
    return lib.attnres_oproj_packed_ahead_run(
        a["x"], a["ldx"], a["Wp"], a["wpb"], a["K"], a["prefix"], a["ld_prefix"], a["blocks"],
        a["bst_t"], a["bst_b"], a["cap"], a["norm"], a["query"], a["out_norm"], a["out"],
        a["ld_out"], a["aux"], a["ld_aux"], a["eps"], a["out_eps"], a["M"], a["H"], a["nb"],
        a["write"], a["has_delta"], a["final"], a["nn"], a["nq"], a["neps"], a["mix"], a["ldm"],
        a["scal"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("change,code", [
    (dict(x=None), -1), (dict(Wp=None), -1), (dict(M=0), -3), (dict(K=8190), -4),
    (dict(wpb=7168 * 8192 * 2 - 256), -1), (dict(ws=None), -5),
    (dict(nn=None), -1), (dict(nq=None), -1), (dict(mix=None), -1), (dict(scal=None), -1),
    (dict(neps=-1.0), -1), (dict(ldm=7000), -1), (dict(mix=A + 8), -2), (dict(ldm=7172), -2),
    (dict(scal=A + 4), -2),
])
def test_attnres_oproj_packed_ahead_run_rejects(lib, change, code):
    """Host-side rejections only (the fake pointers are never dereferenced)."""
    assert call_packed_ahead(lib, **change) == code

