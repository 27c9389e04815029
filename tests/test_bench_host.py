"""Host-side checks of bench.py (no GPU): the one-GPU contract, the roofline
constants and the guard that retires stored traffic counters when the kernel
code changes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ, **env)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=e, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""  # no JSON line


def test_alu_peak_from_unit_counts():
    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: VALU lane-operations without packed forms
    assert bench.PEAK_VALU_TOPS == pytest.approx(39.3216, rel=1e-12)
    assert bench.PEAK_HBM_GBS == 8000.0
    # the minimum model: 60 VALU lane-ops + 2 transcendentals per composited pair
    assert (bench.VALU_MIN_PER_PAIR, bench.TRANS_PER_PAIR) == (60, 2)
    assert (bench.LDS_RECORD_BYTES, bench.LDS_READS_PER_ENTRY) == (40, 4)


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    code = "__global__ void k(float* p) { p[0] = 1.0f; }\n"
    variants = {
        "plain": code,
        "commented": "// a note\n" + code.replace("{", "{ /* block\ncomment */") + "  // tail\n",
        "spaced": code.replace(" ", "   ").replace("\n", "\n\n"),
        "changed": code.replace("1.0f", "2.0f"),
    }
    hashes = {}
    for name, text in variants.items():
        d = tmp_path / name
        d.mkdir()
        (d / "a.hip").write_text(text)
        (d / "b.hpp").write_text("#pragma once\n")
        monkeypatch.setattr(bench, "ROOT", str(d))
        monkeypatch.setattr(bench, "KERNEL_SOURCES", ["a.hip", "b.hpp"])
        hashes[name] = bench.kernel_source_hash()
    assert hashes["plain"] == hashes["commented"] == hashes["spaced"]
    assert hashes["changed"] != hashes["plain"]


def test_source_hash_covers_the_kernel_sources():
    for rel in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, rel)), rel
    assert len(bench.kernel_source_hash()) == 16
