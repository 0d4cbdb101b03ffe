"""Host-side checks of bench.py and the committed profile summaries (CPU only).

* Every summary under profiles/ is stamped with one kernel-source hash, and
  every counter target has its summary.
* Each summary gives the command that made it, and that command runs only
  committed files: bench.py under rocprofv3, never a working script.
* read_counters() hands the recorded figures to the benchmark only while the
  stamp matches the sources: a summary with another stamp reads as absent.
* `bench.py --gpus N` with N above 1 exits with a message and status 2.
"""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _summaries():
    return sorted(f for f in os.listdir(PROFILES) if f.endswith(".txt"))


def test_profiles_share_one_stamp_and_cover_every_target():
    stamps = set()
    for f in _summaries():
        m = re.search(r"kernel_source_hash:\s*(\w+)", open(os.path.join(PROFILES, f)).read())
        assert m, f"{f}: no kernel_source_hash stamp"
        stamps.add(m.group(1))
    assert len(stamps) == 1, f"summaries from different sources: {stamps}"
    for stem, _pattern, _what in bench.COUNTER_TARGETS.values():
        assert f"{stem}_counters.txt" in _summaries(), f"no summary for {stem}"


def test_profile_commands_run_committed_files_only():
    for f in _summaries():
        text = open(os.path.join(PROFILES, f)).read()
        assert "rocprofv3" in text and "bench.py" in text, f"{f}: no command recorded"
        assert "_work" not in text, f"{f}: names a working file"


def test_counters_read_only_while_stamp_matches(tmp_path, monkeypatch):
    name = "dense_4096_e4m3"
    stem = bench.COUNTER_TARGETS[name][0]
    text = open(os.path.join(PROFILES, f"{stem}_counters.txt")).read()
    stamp = re.search(r"kernel_source_hash:\s*(\w+)", text).group(1)
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    (tmp_path / f"{stem}_counters.txt").write_text(text.replace(stamp, bench.kernel_source_hash()))
    got = bench.read_counters(name)
    assert got and got["hbm_bytes_per_launch"] > 0 and 0 < got["mfma_busy_fraction"] <= 1
    (tmp_path / f"{stem}_counters.txt").write_text(text.replace(stamp, "0" * 16))
    assert bench.read_counters(name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr
