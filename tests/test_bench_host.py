"""Host-side checks of bench.py (no GPU): the one-GPU contract and the HBM-traffic bookkeeping."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    rec = {"source_hash": bench.source_hash(), "hbm_bytes_per_launch": 123456789}
    f = tmp_path / "counters.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PMC_FILE", str(f))
    assert bench.measured_traffic() == 123456789
    rec["source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_source_hash_covers_every_kernel_source(tmp_path, monkeypatch):
    """A change to any library source (csrc/, include/) changes the hash, so stale counters are
    dropped and a stale library is refused."""
    dirs = []
    for rel in (("optimizer_step_weight_amd", "csrc"), ("include",)):
        dst = tmp_path.joinpath(*rel)
        dst.mkdir(parents=True)
        src = os.path.join(ROOT, *rel)
        for name in sorted(os.listdir(src)):
            if name.endswith((".h", ".hip", ".cpp")):
                with open(os.path.join(src, name), "rb") as fh:
                    (dst / name).write_bytes(fh.read())
        dirs.append(dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash()
    for d in dirs:
        for name in sorted(os.listdir(d)):
            p = d / name
            old = p.read_bytes()
            p.write_bytes(old + b"\n")
            assert bench.source_hash() != h0, name
            p.write_bytes(old)
    assert bench.source_hash() == h0


def test_committed_counters_describe_the_fused_kernel_at_the_headline_shape():
    with open(bench.PMC_FILE) as fh:
        d = json.load(fh)
    # the write counter must show exactly W (bf16) + m + v (fp32) read-modify-written: no gradient bytes
    N, K = 4096, 14336
    assert d["hbm_write_bytes_per_launch"] == N * K * (2 + 4 + 4)
    assert d["hbm_bytes_per_launch"] == d["hbm_read_bytes_per_launch"] + d["hbm_write_bytes_per_launch"]
    assert d["algorithmic_bytes_per_launch"] == 4096 * (N + K) * 2 + 2 * N * K * (2 + 4 + 4)
