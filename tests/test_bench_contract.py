"""bench.py's host-side parts (no GPU): the algorithmic byte counts of the
timed workloads, the one-GPU refusal, and the digest that keys the stored HBM
traffic figures to the kernel sources."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

H = 7168


@pytest.mark.parametrize("cfg,expect", [(0, 14_796_800), (1, 59_746_304), (2, 130_459_648)])
def test_fused_step_bytes(cfg, expect):
    """W, x, three gain rows, and per token: old prefix (read iff has_delta),
    the nb scored blocks, the new prefix, aux, the written slot, the output."""
    w = bench.WORKLOADS[cfg]
    got = bench.algorithmic_bytes(w["M"], w["K"], w["nb"], w["write"], w["has_delta"])
    assert got == expect
    row = 2 * H
    terms = 2 * H * w["K"] + 2 * w["M"] * w["K"] + 3 * row + w["M"] * row * (
        w["has_delta"] + w["nb"] + 1 + 1 + (w["write"] >= 0) + 1)
    assert got == terms


def test_bytes_count_each_tensor_once():
    base = bench.algorithmic_bytes(8, 4096, 4, -1, 1)
    assert bench.algorithmic_bytes(8, 4096, 4, 2, 1) - base == 8 * 2 * H   # the written slot
    assert base - bench.algorithmic_bytes(8, 4096, 4, -1, 0) == 8 * 2 * H  # the old prefix
    assert base - bench.algorithmic_bytes(8, 4096, 4, -1, 1, aux=0) == 8 * 2 * H
    assert bench.algorithmic_bytes(8, 4096, 5, -1, 1) - base == 8 * 2 * H  # one more block


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_digest_ignores_comments_and_spacing():
    a = "int f(int x) {  // the sum\n  return x + 1; /* plus\n one */ }\n"
    b = "int f(int x) { return x + 1; }"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text("return x + 2;") != bench.code_text("return x + 1;")


def test_stored_traffic_records_are_well_formed():
    for (cfg, layout), rec in bench.MEASURED_TRAFFIC.items():
        assert cfg in bench.WORKLOADS and layout in ("prepared", "row-major")
        assert len(rec["digest"]) == 64 and rec["fetch"] > 0 and rec["write"] > 0
        w = bench.WORKLOADS[cfg]
        alg = bench.algorithmic_bytes(w["M"], w["K"], w["nb"], w["write"], w["has_delta"])
        assert 0.9 < (rec["fetch"] + rec["write"]) / alg < 1.5
