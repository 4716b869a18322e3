"""Code-generation check of the LDS-ring kernels (host only: hipcc emits the
gfx950 assembly without a GPU).

The weight stream runs several chunks ahead: each wavefront waits only until
its loads of the chunk it is about to read have landed (``s_waitcnt
vmcnt(n)`` with n > 0). When the compiler's wait bookkeeping believes more
loads are outstanding than the ring's own, it emits ``s_waitcnt vmcnt(0)``
directly before a fragment read of the ring instead, which drains every
chunk in flight on each step (one memory round trip per chunk: 64 tokens,
K = 8192 went from 30.7 to 42.7 us). Unrelated edits elsewhere in a kernel
have set it off, so every ring kernel is checked here.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from skinny_gemm_attention_amd import _build

RING_SOURCES = ["fused.hip", "wsgemm.hip"]
LOOKBACK = 120  # lines: a fragment read this close after a ring load belongs to the stream


def ring_wait_hits(asm: str) -> dict[str, int]:
    """Per kernel: fragment reads (ds_read_b128) preceded directly by a full
    vmcnt(0) wait while a direct-to-LDS load was issued shortly before."""
    hits = {}
    for m in re.finditer(r"^(_ZN7attnres\w*kernel\w*):", asm, flags=re.M):
        end = asm.index(".Lfunc_end", m.end())
        lines = [l for l in asm[m.end():end].splitlines() if l.strip() and not l.lstrip().startswith(";")]
        n = 0
        for i, line in enumerate(lines):
            if "ds_read_b128" not in line or i == 0:
                continue
            prev = lines[i - 1]
            if "s_waitcnt" in prev and re.search(r"\bvmcnt\(0\)", prev):
                if any("global_load_lds" in x for x in lines[max(0, i - LOOKBACK):i]):
                    n += 1
        hits[m.group(1)] = n
    return hits


@pytest.mark.skipif(not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not installed")
@pytest.mark.parametrize("src", RING_SOURCES)
def test_no_full_wait_before_ring_reads(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [_build.HIPCC, *_build.FLAGS, "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    hits = ring_wait_hits(out.read_text())
    assert hits, f"no kernels found in the assembly of {src}"
    bad = {k: v for k, v in hits.items() if v}
    assert not bad, f"{src}: vmcnt(0) directly before ring fragment reads in {bad}"


def test_detector_flags_a_full_wait():
    """The scan itself: a full wait right before a fragment read that follows a
    ring load is reported; a partial wait, or one with no ring load before it,
    is not."""
    body = ("\tglobal_load_lds_dwordx4 v[0:1], off\n"
            "\ts_waitcnt vmcnt(3)\n\tds_read_b128 v[4:7], v2\n"
            "\ts_waitcnt vmcnt(0)\n\tds_read_b128 v[8:11], v2\n")
    asm = ("_ZN7attnres8x_kernelEv:\n" + body + ".Lfunc_end0:\n"
           "_ZN7attnres8y_kernelEv:\n\ts_waitcnt vmcnt(0)\n\tds_read_b128 v[8:11], v2\n.Lfunc_end1:\n")
    assert ring_wait_hits(asm) == {"_ZN7attnres8x_kernelEv": 1, "_ZN7attnres8y_kernelEv": 0}
