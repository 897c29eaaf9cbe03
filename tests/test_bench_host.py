"""Host logic of bench.py (no GPU): the kernel-source digest that keeps committed counters
tied to the code they were taken on, the byte basis a fraction is quoted on, and the
one-GPU refusal."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

KERNEL = """// a comment
__global__ void k(float *p) {  /* block
comment */ p[0] = 1.0f;  // trailing
}
"""


@pytest.fixture
def csrc(tmp_path, monkeypatch):
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "a.hip").write_text(KERNEL)
    (d / "b.hpp").write_text("#pragma once\nconstexpr int N = 4;\n")
    (d / "notes.txt").write_text("not a source")
    monkeypatch.setattr(bench, "CSRC", str(d))
    return d


def test_digest_ignores_comments_and_layout(csrc):
    d0 = bench.sources_digest()
    (csrc / "a.hip").write_text("// another comment\n__global__ void k(float *p)\n{\n"
                                "    p[0] = 1.0f;   /* changed wording */\n}\n")
    assert bench.sources_digest() == d0
    (csrc / "notes.txt").write_text("edited")  # not a kernel source
    assert bench.sources_digest() == d0


@pytest.mark.parametrize("edit", [
    ("a.hip", KERNEL.replace("1.0f", "2.0f")),           # a constant
    ("a.hip", KERNEL.replace("p[0]", "p[1]")),           # an index
    ("b.hpp", "#pragma once\nconstexpr int N = 8;\n"),   # a header
])
def test_digest_follows_code(csrc, edit):
    d0 = bench.sources_digest()
    name, text = edit
    (csrc / name).write_text(text)
    assert bench.sources_digest() != d0


def test_digest_follows_a_new_source(csrc):
    d0 = bench.sources_digest()
    (csrc / "c.hip").write_text("__global__ void q() {}\n")
    assert bench.sources_digest() != d0


def _record(tmp_path, monkeypatch, sha):
    rec = {"sources_sha": sha,
           "workloads": {"w": {"fb": {"bytes": 600, "trans_lane_insts": 4.8e9,
                                      "valu_busy_pct": 50.0}}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    monkeypatch.setattr(bench, "_COUNTERS", None)


def test_fraction_on_counter_bytes_while_the_digest_matches(csrc, tmp_path, monkeypatch):
    _record(tmp_path, monkeypatch, bench.sources_digest())
    out = bench.traffic_fields("w", ("fb",), 1e-6, 400, "minimum", 900)
    assert out["bytes_basis"] == "counters" and out["bytes_per_step"] == 600
    # 600 B in 1 ns = 600 GB/s
    assert out["hbm_gbps"] == pytest.approx(600.0)
    assert out["hbm_frac"] == pytest.approx(600.0 / bench.PEAK_HBM_GBPS, abs=1e-4)
    assert out["trans_util"]["fb"] == pytest.approx(4.8e9 / 1e-9 / bench.PEAK_TRANS_PER_S,
                                                    rel=1e-3)
    assert out["pages_equivalent_bytes"] == 900


def test_fallback_bytes_once_the_code_changed(csrc, tmp_path, monkeypatch):
    _record(tmp_path, monkeypatch, "0" * 16)
    out = bench.traffic_fields("w", ("fb",), 1e-6, 400, "minimum", 900)
    assert out["bytes_basis"] == "minimum" and out["bytes_per_step"] == 400
    assert "trans_util" not in out


def test_fallback_when_a_part_is_missing(csrc, tmp_path, monkeypatch):
    _record(tmp_path, monkeypatch, bench.sources_digest())
    out = bench.traffic_fields("w", ("fwd", "bwd"), 1e-6, 500, "compulsory", 900)
    assert out["bytes_basis"] == "compulsory" and out["bytes_per_step"] == 500


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    text = r.stdout + r.stderr
    assert "one GPU" in text and "--gpus 2" in text
