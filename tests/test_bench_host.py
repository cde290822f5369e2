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


def _copy_sources(tmp_path):
    for rel in bench.KERNEL_SOURCES + bench.RING_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        with open(os.path.join(ROOT, rel), "rb") as f:
            dst.write_bytes(f.read())


def test_summary_lookups_follow_the_digest_and_the_launch(tmp_path, monkeypatch):
    """measured_traffic / ring_traffic / traced_call read the committed
    per-shape summaries and give None once the recorded digest no longer
    matches the sources, or the chooser's launch differs from the one
    profiled."""
    import moe_decode_skinny_amd as sk

    walk16 = bench.walk_record(sk, 16, bench.N, bench.K)
    ring16 = bench._ring_launch_record(sk, 16)
    other = {**ring16, "segment": ring16["segment"] + 1}
    traffic = {"kernel_source_digest": bench.kernel_source_digest(),
               "ring_source_digest": bench.ring_source_digest(),
               "entries": [
                   {"shape": "unpooler", "ring": False, "M": 16, "launch": walk16,
                    "hbm_bytes_per_item": 123},
                   {"shape": "unpooler", "ring": False, "M": 8, "launch": walk16,
                    "hbm_bytes_per_item": 5},
                   {"shape": "unpooler", "ring": True, "M": 16, "launch": ring16,
                    "hbm_bytes_per_item": 456},
                   {"shape": "unpooler", "ring": True, "M": 8, "launch": other,
                    "hbm_bytes_per_item": 789}]}
    trace = {"kernel_source_digest": bench.kernel_source_digest(),
             "entries": [{"shape": "unpooler", "M": 16, "launch": walk16, "call_median_us": 5.0,
                          "kernels": [{"kernel": "k", "grid": 1, "n": 901, "median": 5.0,
                                       "p10": 4.9, "p90": 5.2}]}]}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic_shapes.json").write_text(json.dumps(traffic))
    (tmp_path / "profiles" / "kernel_trace_shapes.json").write_text(json.dumps(trace))
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    assert bench.measured_traffic(16) == 123
    assert bench.measured_traffic(16, sk) == 123
    # profiled at another launch than the chooser's M=8 launch
    assert bench.measured_traffic(8, sk) is None
    assert bench.ring_traffic(16, sk) == 456
    assert bench.ring_traffic(8, sk) is None
    t = bench.traced_call(16, sk)
    assert t["median_us"] == 5.0 and t["dispatches"] == 901 and t["p90_us"] == 5.2
    assert bench.traced_call(8, sk) is None
    # a comment or whitespace edit keeps them
    src = tmp_path / "moe_decode_skinny_amd" / "csrc" / "device.h"
    src.write_bytes(src.read_bytes() + b"\n// a comment\n/* another */\n")
    assert bench.measured_traffic(16) == 123 and bench.traced_call(16) is not None
    # a changed kernel source voids all three
    src.write_bytes(src.read_bytes() + b"\nconstexpr int kSomething = 1;\n")
    assert bench.measured_traffic(16) is None
    assert bench.ring_traffic(16) is None
    assert bench.traced_call(16) is None


def _write_csv(path, header, rows):
    import csv

    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_reduces_runs_shape_by_shape(tmp_path):
    """The committed reduction of rocprofv3 CSVs (bench.py --summarize): a
    kernel trace and the four counter passes of one shape, written as the
    profiling runs lay them out, give the per-dispatch quantiles, the
    copy-scaled bytes and the request-size bytes."""
    root = tmp_path / "prof"
    launch = {"path": 3, "splits": 1}
    shape = {"shape": "unpooler", "ring": False, "M": 16, "N": 1024, "K": 4096, "launch": launch,
             "calls": 901, "items_per_call": 1, "us_per_item_replay": 5.1, "copy_mib": 64,
             "kernel_source_digest": "d" * 16, "ring_source_digest": "r" * 16}
    kname = "void skinny::(anonymous namespace)::gemm_blocks_kernel<1, 4, 4, 512>(int)"
    d = root / "trace_unpooler_m16"
    d.mkdir(parents=True)
    (d / "shape.json").write_text(json.dumps(shape))
    head = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
            "Grid_Size_Y", "Grid_Size_Z"]
    rows = [["KERNEL_DISPATCH", kname, 1000 * i, 1000 * i + 4000 + 10 * i, 131072, 1, 1]
            for i in range(101)]
    rows.append(["KERNEL_DISPATCH", "void at::fill_kernel(int)", 0, 99000, 64, 1, 1])
    _write_csv(d / "x" / "run_kernel_trace.csv", head, rows)
    chead = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    copy = "__amd_rocclr_copyBuffer"
    values = {"fetch": [("FETCH_SIZE", 2048.0, 32768.0)],
              "write": [("WRITE_SIZE", 64.0, 65536.0)],
              "rdreq": [("TCC_EA0_RDREQ_32B_sum", 0.0, 0.0), ("TCC_EA0_RDREQ_64B_sum", 10.0, 0.0),
                        ("TCC_EA0_RDREQ_128B_sum", 32768.0, 524288.0),
                        ("TCC_EA0_RDREQ_sum", 32778.0, 524288.0)],
              "dram": [("TCC_EA0_RDREQ_DRAM_32B_sum", 131072.0, 2097152.0),
                       ("TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", 1024.0, 2097152.0)]}
    for pas, cs in values.items():
        d = root / f"{pas}_unpooler_m16"
        d.mkdir(parents=True)
        (d / "shape.json").write_text(json.dumps(shape))
        crow = []
        for name, mine, ref in cs:
            crow.append([copy, 131072, name, ref])
            crow += [[kname, 131072, name, mine]] * 3
        _write_csv(d / "run_counter_collection.csv", chead, crow)
    out = tmp_path / "out"
    out.mkdir()
    bench.summarize_profiles(str(root), str(out))
    tr = json.loads((out / "kernel_trace_shapes.json").read_text())
    e = tr["entries"][0]
    assert tr["kernel_source_digest"] == "d" * 16
    assert [k["kernel"] for k in e["kernels"]] == ["gemm_blocks_kernel<1, 4, 4, 512>"]
    k = e["kernels"][0]
    assert k["n"] == 101 and k["median"] == 4.5 and k["p10"] == 4.1 and k["p90"] == 4.9
    assert e["call_median_us"] == 4.5 and "--profile-shape unpooler:16" in e["command"]
    hb = json.loads((out / "hbm_traffic_shapes.json").read_text())
    t = hb["entries"][0]
    # FETCH 2048 KiB x (64 MiB / 32768 KiB) + WRITE 64 KiB x 1
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["hbm_bytes_per_item"] == 2048 * 1024 * 2 + 64 * 1024
    assert t["read_bytes_from_request_sizes"] == 64 * 10 + 128 * 32768
    assert t["dram_read_bytes"] == 32 * 131072 and t["dram_write_bytes"] == 32 * 1024
    assert t["copy_reference"]["read_bytes_from_request_sizes"] == 64 << 20
    text = (out / "hbm_traffic_shapes.txt").read_text()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "ratio" in text


def test_cpu_baseline_object():
    cb = bench.cpu_baseline(budget_s=0.3)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s"
    assert cb["value"] > 0 and 1 <= cb["cores"] <= 16
    assert "steps of the M=1,2,4,8,16 sweep" in cb["sample"]
    assert set(cb["per_m"]) == {"threads", "1", "2", "4", "8", "16"}
    assert cb["per_m_1_thread"]["16"]["median_us_per_call"] > 0
    assert cb["host"]["nproc"] >= cb["host"]["affinity"] >= 1 and cb["host"]["cpu_model"]
