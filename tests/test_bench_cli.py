"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal, the
CPU baseline record (the oracle on the host cores) and the gate that drops
counted HBM traffic once the decode sources change."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_cpu_baseline_record_on_the_tiny_workload():
    import bench
    from bit_mla_kv_decode_amd import workloads as W
    rec = bench.cpu_baseline(W.WORKLOADS["tiny_c4r4"], seqs=1)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["host"]["cpu_model"] and rec["host"]["cpus_visible"] >= 1
    assert "1 of 1 sequences (256 tokens)" in rec["sample"]
    assert rec["single_thread"]["value"] > 0


def test_traffic_gate_follows_the_kernel_sources(tmp_path, monkeypatch):
    import bench
    sha = bench.kernel_source_sha256()
    assert re.fullmatch(r"[0-9a-f]{64}", sha)
    prof = tmp_path / "profiles"
    prof.mkdir()
    f = prof / "traffic_k_decode_flat_demo.md"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: sha)
    f.write_text("kernel_source_sha256: %s\ntraffic_bytes_per_launch: 1234\n" % sha)
    assert bench.counted_traffic("demo", "C4R4") == 1234
    f.write_text("kernel_source_sha256: %s\ntraffic_bytes_per_launch: 1234\n" % ("0" * 64))
    assert bench.counted_traffic("demo", "C4R4") is None
    assert bench.counted_traffic("missing", "C4R4") is None


def test_kernel_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    import bench
    def tree(code):
        root = tmp_path / ("t%d" % len(list(tmp_path.iterdir())))
        for rel in bench.KERNEL_SOURCES:
            f = root / rel
            f.parent.mkdir(parents=True, exist_ok=True)
            f.write_text(code)
        return str(root)
    base = "int f(int x) {\n  return x + 1;\n}\n"
    commented = "// header comment\nint f(int x) {  /* inline\n block */\n\n  return x + 1;  // trailing\n}\n"
    changed = "int f(int x) {\n  return x + 2;\n}\n"
    hashes = []
    for code in (base, commented, changed):
        monkeypatch.setattr(bench, "ROOT", tree(code))
        hashes.append(bench.kernel_source_sha256())
    assert hashes[0] == hashes[1] != hashes[2]


def test_traffic_tags_name_workload_format_and_heads():
    import bench
    assert bench.traffic_tag("c4r4_128k") == "c4r4_128k"
    assert bench.traffic_tag("c2r4_32k_outliers", "BF16") == "c2r4_32k_outliers_bf16"
    assert bench.traffic_tag("c4r4_128k", "", 16) == "c4r4_128k_h16"

