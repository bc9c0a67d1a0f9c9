"""bench.py's traffic figure, host side: the HBM bytes per launch come from a
committed counter summary only when that summary was taken on the current
kernel source and on the same workload; otherwise the figure is null."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _summary(tmp_path, workload, sha, nbytes=123456789.0):
    path = tmp_path / f"coat_step_multi_{workload}_pmc.json"
    path.write_text(json.dumps({"workload": workload, "source_sha256": sha, "hbm_bytes_per_launch": nbytes}))
    return str(path)


def test_traffic_taken_on_the_current_source_is_reported(tmp_path, monkeypatch):
    path = _summary(tmp_path, "llama13b", bench.kernel_source_hash())
    monkeypatch.setattr(bench, "pmc_file", lambda wl: path)
    assert bench.load_traffic("llama13b", 1.0) == 123456789.0


def test_traffic_from_another_source_is_null(tmp_path, monkeypatch):
    path = _summary(tmp_path, "llama13b", "0" * 64)
    monkeypatch.setattr(bench, "pmc_file", lambda wl: path)
    assert bench.load_traffic("llama13b", 1.0) is None


def test_traffic_of_another_workload_is_null(tmp_path, monkeypatch):
    path = _summary(tmp_path, "llama13b_g32", bench.kernel_source_hash())
    monkeypatch.setattr(bench, "pmc_file", lambda wl: path)
    assert bench.load_traffic("llama13b", 1.0) is None


def test_missing_or_broken_summary_is_null(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "pmc_file", lambda wl: str(tmp_path / "absent.json"))
    assert bench.load_traffic("llama13b", 1.0) is None
    broken = tmp_path / "broken.json"
    broken.write_text("{not json")
    monkeypatch.setattr(bench, "pmc_file", lambda wl: str(broken))
    assert bench.load_traffic("llama13b", 1.0) is None


def test_hash_covers_every_kernel_source_in_order(tmp_path, monkeypatch):
    """Changing any one of the step kernel's sources changes the hash."""
    copies = []
    for src in bench.KERNEL_SRCS:
        dst = tmp_path / os.path.basename(src)
        dst.write_bytes(open(src, "rb").read())
        copies.append(str(dst))
    monkeypatch.setattr(bench, "KERNEL_SRCS", copies)
    base = bench.kernel_source_hash()
    for c in copies:
        original = open(c, "rb").read()
        with open(c, "ab") as f:
            f.write(b"\n")
        assert bench.kernel_source_hash() != base, c
        with open(c, "wb") as f:
            f.write(original)
    assert bench.kernel_source_hash() == base
