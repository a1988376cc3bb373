"""Host-side pieces of bench.py, on the CPU: the device-source hash that keys the committed
counter records, the lookups that read them, and the one-GPU guard."""
import importlib.util
import json
import os
import shutil
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_only_drops_comments_and_blank_lines(bench):
    src = "int a; // trailing\n\n/* block\n   over lines */ int b;\n   // whole line\nint c;  \n"
    assert bench._code_only(src) == "int a;\n int b;\nint c;"


def _fake_tree(tmp_path, edit=None):
    csrc = tmp_path / "tiled_stage_software_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "tiled_stage_software_amd", "csrc"), csrc,
                    ignore=shutil.ignore_patterns("*.cpp"))
    if edit:
        f = csrc / "schedule.hpp"
        f.write_text(edit(f.read_text()))
    return str(tmp_path)


def test_hash_ignores_comment_edits_and_sees_code_edits(bench, tmp_path, monkeypatch):
    base = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", _fake_tree(tmp_path / "same"))
    assert bench.kernel_source_hash() == base
    monkeypatch.setattr(bench, "ROOT", _fake_tree(tmp_path / "comment", lambda t: t + "\n// a new comment\n"))
    assert bench.kernel_source_hash() == base
    monkeypatch.setattr(bench, "ROOT", _fake_tree(tmp_path / "code", lambda t: t + "\nconstexpr int kProbe = 1;\n"))
    assert bench.kernel_source_hash() != base


def test_committed_records_match_the_current_sources(bench):
    """The counter records bench.py reads carry the hash of the present device sources and
    the default plan of the headline workload, so the bench line reports their values."""
    h = bench.kernel_source_hash()
    for name in ("traffic_c3.json", "clock_c3.json"):
        with open(os.path.join(ROOT, "profiles", name)) as fh:
            d = json.load(fh)
        assert d["kernel_source_hash"] == h, name
        assert d["plan"] == {"kernel": 3, "tile": 31, "nstage": 2}, name


def test_record_lookups_refuse_other_sources_or_plans(bench):
    plan = types.SimpleNamespace(kernel=3, tile=31, nstage=2)
    h = bench.kernel_source_hash()
    assert bench.traffic_for("c3", h, plan) is not None
    assert bench.clock_for("c3", h, plan) is not None
    assert bench.traffic_for("c3", "0" * 16, plan) is None
    assert bench.clock_for("c3", "0" * 16, plan) is None
    other = types.SimpleNamespace(kernel=3, tile=24, nstage=2)
    assert bench.traffic_for("c3", h, other) is None
    assert bench.clock_for("c3", h, other) is None
    assert bench.traffic_for("c9", h, plan) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
