"""Host-side checks of bench.py's contract pieces (no GPU): the one-GPU
refusal, the algorithmic byte count, the counter-summary lookups and the
CPU-baseline object."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_algorithmic_bytes():
    # W once, x once, y once, 2 bytes each (bf16)
    assert bench.algorithmic_bytes(1) == 2 * 1024 * 4096 + 2 * 4096 + 2 * 1024
    assert bench.algorithmic_bytes(16, 8192, 1024) == 2 * (8192 * 1024 + 16 * 1024 + 16 * 8192)


def test_digests_cover_existing_sources_and_are_stable():
    for rel in bench.KERNEL_SOURCES + bench.RING_SOURCES:
        assert os.path.exists(os.path.join(ROOT, rel)), rel
    assert bench.kernel_source_digest() == bench.kernel_source_digest()
    assert len(bench.ring_source_digest()) == 16


def test_traffic_lookup_follows_the_digest(tmp_path, monkeypatch):
    """measured_traffic / ring_traffic read the committed summaries and give
    None once the recorded digest no longer matches the sources."""
    rec = {"kernel_source_digest": bench.kernel_source_digest(),
           "per_m": {"16": {"hbm_bytes_per_launch": 123, "walk": None}}}
    import moe_decode_skinny_amd as sk

    r = sk.skinny_ring_choose(16, bench.N, bench.K, bench.RING)
    now = {**dict(r.gemm._asdict()), "segment": r.segment, "workgroups": r.workgroups,
           "order": r.order}
    other = {**now, "segment": now["segment"] + 1}
    ring = {"kernel_source_digest": bench.ring_source_digest(),
            "per_m": {"16": {"hbm_bytes_per_item": 456, "launch": now},
                      "8": {"hbm_bytes_per_item": 789, "launch": other}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic_unpooler_sweep.json").write_text(json.dumps(rec))
    (tmp_path / "profiles" / "hbm_traffic_ring_unpooler.json").write_text(json.dumps(ring))
    for rel in bench.KERNEL_SOURCES + bench.RING_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    assert bench.measured_traffic(16) == 123
    assert bench.measured_traffic(8) is None
    assert bench.ring_traffic(16) == 456
    assert bench.ring_traffic(16, sk) == 456
    # counters taken at another ring launch than the chooser's are not used
    assert bench.ring_traffic(8, sk) is None
    # a changed kernel source voids both
    src = tmp_path / "moe_decode_skinny_amd" / "csrc" / "device.h"
    src.write_bytes(src.read_bytes() + b"\n")
    assert bench.measured_traffic(16) is None
    assert bench.ring_traffic(16) is None


def test_cpu_baseline_object():
    cb = bench.cpu_baseline(budget_s=0.3)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s"
    assert cb["value"] > 0 and 1 <= cb["cores"] <= 16
    assert "steps of the M=1,2,4,8,16 sweep" in cb["sample"]
