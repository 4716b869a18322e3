"""The Python binding refuses tensors smaller than the counts it passes to the
C ABI (which sees only pointers and strides): the check runs on the host,
before any pointer is taken, so these tests run without a GPU."""
from __future__ import annotations

import pytest
import torch

import skinny_gemm_attention_amd as sga


def t(*shape, dtype=torch.int16):
    return torch.zeros(*shape, dtype=dtype)


M, K, H, NB, CAP = 4, 64, 128, 2, 3


def attn_args(**over):
    a = dict(prefix=t(M, H), blocks=t(M, CAP, H), norm=t(H), query=t(H), out_norm=t(H),
              out=t(M, H), aux=t(M, H))
    a.update(over)
    return a


@pytest.mark.parametrize("bad,name", [
    (dict(prefix=t(M - 1, H)), "prefix"),
    (dict(out=t(M, H - 8)), "out"),
    (dict(aux=t(M - 1, H)), "aux"),
    (dict(blocks=t(M - 1, CAP, H)), "blocks"),
    (dict(blocks=t(M, CAP, H - 8)), "blocks"),
    (dict(blocks=t(M, H)), "blocks"),
    (dict(norm=t(H - 8)), "norm"),
    (dict(query=t(H // 2)), "query"),
    (dict(out_norm=t(1, H)), "out_norm"),
])
def test_fused_and_attnres_shapes(bad, name):
    a = attn_args(**bad)
    with pytest.raises(sga.AttnResError, match=name):
        sga.attnres_oproj_run(t(M, K), t(H, K), a["prefix"], a["blocks"], a["norm"], a["query"],
                              a["out_norm"], a["out"], a["aux"], t(1024, dtype=torch.uint8), nb=NB)
    with pytest.raises(sga.AttnResError, match=name):
        sga.attnres_run(t(M, H), a["prefix"], a["blocks"], a["norm"], a["query"], a["out_norm"],
                        a["out"], a["aux"], nb=NB)


def test_fused_weight_shape():
    a = attn_args()
    with pytest.raises(sga.AttnResError, match="W"):
        sga.attnres_oproj_run(t(M, K), t(H, K - 8), a["prefix"], a["blocks"], a["norm"], a["query"],
                              a["out_norm"], a["out"], a["aux"], t(1024, dtype=torch.uint8), nb=NB)


def test_lookahead_shapes():
    a = attn_args()
    f32 = torch.float32
    base = (t(M, K), t(H, K), a["prefix"], a["blocks"], a["norm"], a["query"], a["out_norm"],
            a["out"], a["aux"], t(1024, dtype=torch.uint8))
    with pytest.raises(sga.AttnResError, match="next_query"):
        sga.attnres_oproj_ahead_run(*base, t(H), t(H - 8), t(M, H, dtype=f32), t(M, 2, dtype=f32),
                                    nb=NB)
    with pytest.raises(sga.AttnResError, match="mixture"):
        sga.attnres_oproj_ahead_run(*base, t(H), t(H), t(M - 1, H, dtype=f32),
                                    t(M, 2, dtype=f32), nb=NB)
    with pytest.raises(sga.AttnResError, match="scal"):
        sga.attnres_oproj_ahead_run(*base, t(H), t(H), t(M, H, dtype=f32), t(M, dtype=f32), nb=NB)
    with pytest.raises(sga.AttnResError, match="mixture"):
        sga.attnres_post_run(t(M, H), a["prefix"], a["blocks"], a["norm"], a["query"],
                             a["out_norm"], a["out"], a["aux"], t(M, H - 8, dtype=f32),
                             t(M, 2, dtype=f32), nb=NB)


@pytest.mark.parametrize("fn", ["wsgemm_run", "wsgemm_run_ws"])
def test_gemm_shapes(fn):
    ws = (t(1024, dtype=torch.uint8),) if fn == "wsgemm_run_ws" else ()
    with pytest.raises(sga.AttnResError, match="y"):
        getattr(sga, fn)(t(M, K), t(H, K), t(M - 1, H), *ws)
    with pytest.raises(sga.AttnResError, match="W"):
        getattr(sga, fn)(t(M, K), t(H, K - 8), t(M, H), *ws)
    with pytest.raises(sga.AttnResError, match="out"):
        sga.wsgemm_moe_front_run(t(M, K), t(H, K), t(M - 1, 4096), router_base=0, slot=0, base=0,
                                 valid=0, split=0)


def test_well_shaped_cpu_tensors_reach_the_device_check():
    """Correct shapes pass the shape checks; CPU tensors are then refused."""
    a = attn_args()
    with pytest.raises(sga.AttnResError, match="GPU"):
        sga.attnres_oproj_run(t(M, K), t(H, K), a["prefix"], a["blocks"], a["norm"], a["query"],
                              a["out_norm"], a["out"], a["aux"], t(1024, dtype=torch.uint8), nb=NB)


@pytest.mark.parametrize("kw,width", [
    (dict(router_base=64, slot=2, base=0, valid=40, split=48), 64 + 2 * (2 + 40)),  # router end
    (dict(router_base=0, slot=0, base=200, valid=0, split=64), 200 + H - 64),       # latent end
])
def test_moe_front_out_width(kw, width):
    """The MoE-front destination must be as wide as the columns the epilogue
    writes (a column-sliced view is narrower than its row stride)."""
    wide = t(M, 1024)
    with pytest.raises(sga.AttnResError, match="out"):
        sga.wsgemm_moe_front_run(t(M, K), t(H, K), wide[:, :width - 2], **kw)
    with pytest.raises(sga.AttnResError, match="GPU"):  # wide enough: reaches the device check
        sga.wsgemm_moe_front_run(t(M, K), t(H, K), wide[:, :width], **kw)
