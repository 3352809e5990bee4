"""Host-side logic of bench.py (no GPU): the one-GPU guard and the rule that
a rocprofv3 traffic record counts only for the kernel sources it was taken
from."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration that is not measured


def _tree(tmp_path, attention_text="kernel A"):
    pkg = tmp_path / "long_context_tabular_amd"
    (pkg / "csrc").mkdir(parents=True)
    (pkg / "csrc" / "attention.hip").write_text(attention_text)
    (pkg / "csrc" / "prep.hip").write_text("prep")
    (pkg / "csrc" / "scaling.h").write_text("scaling")
    (pkg / "build_lib.py").write_text("flags")
    (tmp_path / "profiles").mkdir()
    return pkg


def test_counter_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    pkg = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("context") is None  # no record at all
    rec = tmp_path / "profiles" / "traffic_context_model512k.txt"
    rec.write_text("# comment: ignored\nsource_hash: %s\ncontext.bytes_per_launch: 5.25e10\n"
                   % bench.kernel_source_hash())
    assert bench.counter_traffic("context") == 52_500_000_000
    assert bench.counter_traffic("cached128") is None  # kernel not in the record
    # any change to a hashed file (here the kernel source) retires the record
    (pkg / "csrc" / "attention.hip").write_text("kernel B")
    assert bench.counter_traffic("context") is None
    # and so does a change of the compiler flags' file
    (pkg / "csrc" / "attention.hip").write_text("kernel A")
    assert bench.counter_traffic("context") == 52_500_000_000
    (pkg / "build_lib.py").write_text("other flags")
    assert bench.counter_traffic("context") is None


def test_comment_changes_keep_the_record_and_code_changes_retire_it(tmp_path, monkeypatch):
    src = "// staging\nint f() { return 1; }  // one\n/* block\n comment */\n"
    pkg = _tree(tmp_path, src)
    (pkg / "build_lib.py").write_text("# flags\nFLAGS = ['-O3']\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (pkg / "csrc" / "attention.hip").write_text("// reworded\n\nint f() { return 1; }  // two\n")
    (pkg / "build_lib.py").write_text("# other words\nFLAGS = ['-O3']\n")
    assert bench.kernel_source_hash() == h0
    (pkg / "csrc" / "attention.hip").write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h0
    (pkg / "csrc" / "attention.hip").write_text(src)
    (pkg / "build_lib.py").write_text("FLAGS = ['-O2']\n")
    assert bench.kernel_source_hash() != h0


def test_committed_traffic_record_is_well_formed():
    path = os.path.join(ROOT, "profiles", "traffic_context_model512k.txt")
    if not os.path.exists(path):
        pytest.skip("no committed counter record")
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    assert len(rec["source_hash"]) == 16 and int(rec["source_hash"], 16) >= 0
    assert float(rec["context.bytes_per_launch"]) > 0
    assert float(rec["fetch_factor"]) > 0 and float(rec["write_factor"]) > 0
