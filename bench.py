"""Benchmark of the small-M decode GEMM on one MI355X.

Workload: the unpooler shard GEMM sweep y[M, 1024] = x[M, 4096] @ W[1024,
4096]^T for M = 1, 2, 4, 8, 16 (unpooler page, module description), BF16
operands and result with FP32 sums, at the chooser's launch shapes.  One step is one
pass of the sweep: five GEMM launches, each on the next weight of a ring of
distinct layers (60 layers = 480 MiB, twice the 256 MiB Infinity Cache, so no
call finds its weights in a cache).  Inputs are seeded synthetic tensors
already resident in HBM: x ~ N(0, 1), W ~ N(0, 1/K).

Steps run as HIP-graph replays (the decode loop records one pass over the
layer ring, 12 steps = 60 calls, as one graph and replays it: the calls
allocate nothing and never synchronize).  Timing uses
HIP events on the stream the kernels run on.

Output: one JSON line.  `value` is achieved HBM GB/s over the step
(algorithmic bytes 2NK + 2MK + 2MN per call / step time).  `roofline` is for
the dominant kernel (the launch with the largest share of the step), with its
average duration measured here from graph replays of that launch alone over
the ring.  `ring` reports the same sweep through the layer-ring launch
(skinny_gemm_bf16_ring: one persistent launch per M over the 60 layers, the
next layer's weights in flight while one is finished), per item.
`oproj` reports the o_proj shard (N=8192, K=1024) the same two ways, and
`pooler` the pooler shard (N=512) and the full pooler (N=4096) at K=8192.
`epilogue` times the expert-input chain (full-pooler GEMM, RMSNorm -> NVFP4)
and the dual norm.  `ceiling` times, the same way, what one launch reaches by
itself on this device: an empty kernel, and the library's stream reference
reading each 8 MiB weight once (skinny_ceiling_stream); its
`dominant_call_fraction` is that stream's time over the dominant call's.
`cpu_baseline` times the oracle on the host for a bounded sample of the same
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

N, K = 1024, 4096
MS = (1, 2, 4, 8, 16)
RING = 60
PEAK_GBS = 8000.0  # MI355X HBM3E, published


def algorithmic_bytes(M: int, n: int = N, k: int = K) -> int:
    return 2 * n * k + 2 * M * k + 2 * M * n


def log(*a):
    print(*a, file=sys.stderr, flush=True)


HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["moe_decode_skinny_amd/csrc/gemm_mfma.hip", "moe_decode_skinny_amd/csrc/gemm_dot2.hip",
                  "moe_decode_skinny_amd/csrc/gemm_blocks.hip", "moe_decode_skinny_amd/csrc/gemm_ring.hip",
                  "moe_decode_skinny_amd/csrc/dot2_device.h", "moe_decode_skinny_amd/csrc/blocks_device.h",
                  "moe_decode_skinny_amd/csrc/split_reduce.hip", "moe_decode_skinny_amd/csrc/device.h"]


def _code_digest(sources) -> str:
    """sha256 of the sources' code: comments and whitespace removed, so an
    edit of a comment does not mark the profiles of the kernels as stale."""
    import hashlib
    import re

    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(HERE, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_digest() -> str:
    return _code_digest(KERNEL_SOURCES)


RING_SOURCES = ["moe_decode_skinny_amd/csrc/gemm_ring.hip", "moe_decode_skinny_amd/csrc/dot2_device.h",
                "moe_decode_skinny_amd/csrc/blocks_device.h", "moe_decode_skinny_amd/csrc/device.h"]


def ring_source_digest() -> str:
    return _code_digest(RING_SOURCES)


def _summary(name: str):
    try:
        with open(os.path.join(HERE, "profiles", name)) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def _ring_launch_record(sk, M: int, n: int = N, k: int = K) -> dict:
    r = sk.skinny_ring_choose(M, n, k, RING)
    return {**dict(r.gemm._asdict()), "segment": r.segment, "workgroups": r.workgroups,
            "order": r.order}


def ring_traffic(M: int, sk=None):
    """HBM bytes per ring item (unpooler shard) from the committed counter
    summary, or None if the ring kernels, or the launch the ring chooser
    picks, changed since the counters were taken."""
    rec = _summary("hbm_traffic_shapes.json")
    if not rec or rec.get("ring_source_digest") != ring_source_digest():
        return None
    for e in rec["entries"]:
        if e["ring"] and e["shape"] == "unpooler" and e["M"] == M:
            if sk is not None and e["launch"] != _ring_launch_record(sk, M):
                return None
            return e["hbm_bytes_per_item"]
    return None


def measured_traffic(M: int, sk=None, shape: str = "unpooler"):
    """HBM bytes per call of the shape's chooser call from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the plain-copy
    reference), or None when the kernels, or the launch and walk the chooser
    picks, changed since it was taken."""
    rec = _summary("hbm_traffic_shapes.json")
    if not rec or rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    n, k, _ = SHAPES[shape]
    for e in rec["entries"]:
        if (not e["ring"] and not e.get("explicit_launch") and not e.get("l1_only")
                and e["shape"] == shape and e["M"] == M):
            if sk is not None and e["launch"] != walk_record(sk, M, n, k):
                return None
            return e["hbm_bytes_per_item"]
    return None


def traced_call(M: int, sk=None, shape: str = "unpooler"):
    """The kernel-trace figures of the shape's chooser call at M from the
    committed summary (median / p10 / p90 us per dispatch, dispatches), or
    None when the kernels or the chooser's launch changed since."""
    rec = _summary("kernel_trace_shapes.json")
    if not rec or rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    n, k, _ = SHAPES[shape]
    for e in rec["entries"]:
        if e["shape"] == shape and e["M"] == M:
            if sk is not None and e["launch"] != walk_record(sk, M, n, k):
                return None
            ks = e["kernels"]
            return {"median_us": e["call_median_us"],
                    "p10_us": round(sum(kk["p10"] for kk in ks), 3),
                    "p90_us": round(sum(kk["p90"] for kk in ks), 3),
                    "dispatches": min(kk["n"] for kk in ks),
                    "kernels": [kk["kernel"] for kk in ks],
                    "source": "profiles/kernel_trace_shapes.json"}
    return None


def walk_record(sk, M: int, n: int, k: int) -> dict:
    """The launch and walk skinny_gemm_bf16 runs (segment 0: the plain kernel)."""
    w = sk.skinny_choose_walk(M, n, k, 0)
    return {**dict(w.gemm._asdict()), "segment": w.segment, "workgroups": w.workgroups}


# ---------------------------------------------------------------- profiling
# Shapes profiled one per rocprofv3 run, so that rows of a kernel trace or a
# counter collection belong to exactly one (shape, M): the pages' shards, each
# on its own 60-layer weight ring (weight seeds as in the timing below).
SHAPES = {"unpooler": (1024, 4096, 1000), "oproj": (8192, 1024, 7000),
          "pooler_shard": (512, 8192, 7100), "pooler_full": (4096, 8192, 7200)}
TRACE_SET = ([("unpooler", m) for m in MS] + [("oproj", m) for m in (1, 8, 16)]
             + [("pooler_shard", m) for m in (1, 8, 16)] + [("pooler_full", m) for m in (1, 8, 16)])
COUNTER_SET = [("unpooler", m) for m in MS] + [("oproj", 16), ("pooler_shard", 16),
                                                ("pooler_full", 8)]
RING_COUNTER_SET = [("unpooler", m) for m in MS]
# rocprofv3 --pmc passes (each within one run's counter limits: <= 4 TCC).
COUNTER_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "rdreq": ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
              "TCC_EA0_RDREQ_sum"],
    "dram": ["TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"],
    "util": ["MfmaUtil", "VALUBusy"],
    # L1 (TCP) -> L2 read requests and L1 tag accesses: the activation
    # re-reads every workgroup pulls through its compute unit
    "tcp": ["TCP_TCC_READ_REQ_sum", "TCP_TOTAL_CACHE_ACCESSES_sum", "TCP_TOTAL_READ_sum"],
}
# Explicit launches profiled beside the chooser's, to compare the load
# traffic of the 16-token calls: the pooler shard at DOT2 (2 rows, 16 waves
# of 1 chunk) and at the 16-block launch with 4 splits summed in the kernel,
# and the unpooler at the 16-block launch of 4 rows with all tokens in each
# workgroup; the chooser's launches take two token groups instead.
COMPARE_LAUNCHES = [("pooler_shard", 16, "0,1,16,1,1,2"), ("pooler_shard", 16, "3,4,4,4,1,4"),
                    ("unpooler", 16, "3,1,8,4,1,4")]
TRACE_PASSES = 12  # ring passes timed per trace run: 12 x 60 = 720 dispatches of the call
COPY_MIB = 64      # the plain device copy that scales byte counters


def profile_runs(root="gpurun_out/prof"):
    """(run directory, rocprofv3 arguments, bench.py arguments) of every
    profiling run, in order."""
    runs = []
    for name, M in TRACE_SET:
        d = f"{root}/trace_{name}_m{M}"
        runs.append((d, ["--kernel-trace", "--stats"],
                     ["--profile-shape", f"{name}:{M}", "--passes", str(TRACE_PASSES)]))
    for pas in ("fetch", "write", "rdreq", "dram"):
        for name, M in COUNTER_SET:
            d = f"{root}/{pas}_{name}_m{M}"
            runs.append((d, ["--pmc", *COUNTER_PASSES[pas]],
                         ["--profile-shape", f"{name}:{M}", "--passes", "1",
                          "--copy-mib", str(COPY_MIB)]))
        if pas in ("fetch", "write"):
            for name, M in RING_COUNTER_SET:
                d = f"{root}/{pas}_ring_{name}_m{M}"
                runs.append((d, ["--pmc", *COUNTER_PASSES[pas]],
                             ["--profile-shape", f"ring:{name}:{M}", "--passes", "1",
                              "--copy-mib", str(COPY_MIB)]))
    for name, M in [("unpooler", m) for m in MS] + [("pooler_shard", 16)]:
        d = f"{root}/util_{name}_m{M}"
        runs.append((d, ["--pmc", *COUNTER_PASSES["util"]],
                     ["--profile-shape", f"{name}:{M}", "--passes", "1"]))
    for name, M in [("unpooler", 16), ("pooler_shard", 16)]:
        d = f"{root}/tcp_{name}_m{M}"
        runs.append((d, ["--pmc", *COUNTER_PASSES["tcp"]],
                     ["--profile-shape", f"{name}:{M}", "--passes", "1"]))
    for name, M, launch in COMPARE_LAUNCHES:
        tag = launch.replace(",", "")
        for pas in ("fetch", "write", "tcp"):
            d = f"{root}/{pas}_{name}_m{M}_l{tag}"
            runs.append((d, ["--pmc", *COUNTER_PASSES[pas]],
                         ["--profile-shape", f"{name}:{M}", "--launch", launch, "--passes", "1",
                          "--copy-mib", str(COPY_MIB)]))
    return runs


def profile_command(d, prof_args, bench_args) -> str:
    return (f"timeout -s KILL 120 rocprofv3 {' '.join(prof_args)} --output-format csv -d {d} "
            f"-o run -- python3 -u bench.py {' '.join(bench_args)} --profile-out {d}")


def profile_shape(spec: str, passes: int, out_dir: str, copy_mib: int, launch: str = "") -> None:
    """One shape's calls for a profiler run: the chooser's call (skinny_gemm_bf16)
    or, for ring:<shape>:<M>, one 60-item ring launch (skinny_gemm_bf16_ring),
    over the shape's 60-layer weight ring: an eager warm-up, then graphs of
    one ring pass replayed 3 + `passes` times; with `launch` ("path,splits,
    waves,chunks,accs,rows") the GEMM at that explicit launch instead of the
    chooser's.  Writes out_dir/shape.json."""
    import torch

    import moe_decode_skinny_amd as sk
    import synthetic

    parts = spec.split(":")
    ring_launch = parts[0] == "ring"
    name, M = parts[-2], int(parts[-1])
    n, k, wseed = SHAPES[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sk.skinny_init(0)
    if copy_mib:
        src = torch.empty(copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ring = synthetic.device_weight_ring(RING, n, k, dev, base_seed=wseed)
    if ring_launch:
        xs = [synthetic.to_device(synthetic.gemm_inputs(N=16, K=k, seed=900 + i)[0][:M], dev)
              for i in range(RING)]
        ys = [torch.empty((M, n), dtype=torch.bfloat16, device=dev) for _ in range(RING)]
        fn = lambda: sk.skinny_gemm_bf16_ring(xs, ring, ys)
    else:
        x = synthetic.to_device(synthetic.gemm_inputs(N=16, K=k, seed=0)[0][:M], dev)
        y = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        if launch:
            explicit = sk.Launch(*[int(v) for v in launch.split(",")])
            fn = lambda: [sk.skinny_gemm_bf16_launch(x, w, y, explicit) for w in ring]
        else:
            fn = lambda: [sk.skinny_gemm_bf16(x, w, y, 0) for w in ring]
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(passes):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (passes * RING)
    if ring_launch:
        r = sk.skinny_ring_choose(M, n, k, RING)
        rec_launch = {**dict(r.gemm._asdict()), "segment": r.segment,
                      "workgroups": r.workgroups, "order": r.order}
    elif launch:
        rec_launch = {**dict(explicit._asdict()), "segment": 0, "workgroups": 0}
    else:
        rec_launch = walk_record(sk, M, n, k)
    rec = {"shape": name, "ring": ring_launch, "M": M, "N": n, "K": k, "launch": rec_launch,
           "explicit_launch": bool(launch),
           "calls": (4 + passes) * (1 if ring_launch else RING),
           "items_per_call": RING if ring_launch else 1,
           "us_per_item_replay": round(us, 3), "copy_mib": copy_mib,
           "kernel_source_digest": kernel_source_digest(),
           "ring_source_digest": ring_source_digest()}
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "shape.json"), "w") as f:
        json.dump(rec, f)
    print(json.dumps(rec), flush=True)
    del g, ring
    torch.cuda.synchronize()


def _short_kernel(name: str) -> str:
    """'void skinny::(anonymous namespace)::gemm_x<1, 2>(args)' -> 'gemm_x<1, 2>'."""
    head = name.split("(", 1)[0] if "(anonymous namespace)" not in name else \
        name.replace("(anonymous namespace)::", "").split("(", 1)[0]
    head = head.replace("void ", "").replace("skinny::", "").strip()
    return head


def _quantiles(vals):
    v = sorted(vals)
    q = lambda p: v[min(len(v) - 1, max(0, int(round(p * (len(v) - 1)))))]
    return {"n": len(v), "mean": sum(v) / len(v), "median": q(0.5), "p10": q(0.1), "p90": q(0.9)}


def _is_library_kernel(short: str) -> bool:
    return short.startswith(("gemm_", "split_reduce"))


def summarize_profiles(root: str, out_dir: str) -> None:
    """Reduce the rocprofv3 CSVs of the profiling runs under `root` (one run
    directory per shape and pass, each holding shape.json) to the committed
    summaries under `out_dir`: kernel_trace_shapes.{json,txt} and
    hbm_traffic_shapes.{json,txt}."""
    import csv
    import glob

    runs = {os.path.basename(d): d for d, _, _ in profile_runs(root)
            if os.path.exists(os.path.join(d, "shape.json"))}
    cmds = {os.path.basename(d): profile_command(d, p, b) for d, p, b in profile_runs(root)}

    def shape_of(d):
        with open(os.path.join(d, "shape.json")) as f:
            return json.load(f)

    def csv_rows(d, suffix):
        files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no *{suffix} under {d}")
        with open(files[0]) as f:
            return list(csv.DictReader(f))

    # ---- kernel traces
    trace = []
    for key, d in runs.items():
        if not key.startswith("trace_"):
            continue
        sh = shape_of(d)
        durs = {}
        for r in csv_rows(d, "kernel_trace.csv"):
            short = _short_kernel(r["Kernel_Name"])
            if not _is_library_kernel(short):
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            durs.setdefault((short, grid), []).append(us)
        kernels = [{"kernel": kname, "grid": grid, **{q: round(v, 3) if q != "n" else v
                                                      for q, v in _quantiles(ds).items()}}
                   for (kname, grid), ds in sorted(durs.items())]
        trace.append({"shape": sh["shape"], "M": sh["M"], "N": sh["N"], "K": sh["K"],
                      "launch": sh["launch"], "kernels": kernels,
                      "call_median_us": round(sum(kk["median"] for kk in kernels), 3),
                      "replay_us_per_call": sh["us_per_item_replay"], "command": cmds[key]})
    # the kernel-source digests the runs recorded (all runs share one tree)
    digests = {shape_of(d)["kernel_source_digest"] for d in runs.values()
               if os.path.exists(os.path.join(d, "shape.json"))}
    ring_digests = {shape_of(d)["ring_source_digest"] for d in runs.values()
                    if os.path.exists(os.path.join(d, "shape.json"))}
    if len(digests) != 1 or len(ring_digests) != 1:
        raise ValueError(f"runs from different kernel sources: {digests} {ring_digests}")
    digest, ring_digest = digests.pop(), ring_digests.pop()
    with open(os.path.join(out_dir, "kernel_trace_shapes.json"), "w") as f:
        json.dump({"kernel_source_digest": digest, "entries": trace}, f, indent=1)
    lines = ["rocprofv3 kernel traces, one run per shape: the chooser's call over the shape's",
             f"{RING}-layer weight ring (an eager warm-up, then graph replays of one ring pass,",
             f"3 + {TRACE_PASSES} passes: {(4 + TRACE_PASSES) * RING} dispatches of each kernel of "
             "the call); per library kernel and grid: dispatches, mean / median / p10 / p90",
             "duration in us; call = sum of the medians of the call's kernels; replay = event-timed",
             "us per call of the same graph replays in the run (profiler on).",
             f"Reduced with: python bench.py --summarize {root}",
             f"kernel sources digest {digest}", ""]
    for e in trace:
        lines.append(f"{e['shape']} M={e['M']} N={e['N']} K={e['K']}  launch {e['launch']}")
        lines.append(f"  command: {e['command']}")
        for kk in e["kernels"]:
            lines.append(f"  {kk['kernel']:<44} grid {kk['grid']:>8}  n {kk['n']:>4}  mean "
                         f"{kk['mean']:7.3f}  median {kk['median']:7.3f}  p10 {kk['p10']:7.3f}  "
                         f"p90 {kk['p90']:7.3f}")
        lines.append(f"  call median {e['call_median_us']:.3f} us  (replay {e['replay_us_per_call']:.3f}"
                     f" us/call)  {algorithmic_bytes(e['M'], e['N'], e['K']) / e['call_median_us'] / 1e3:.1f}"
                     " GB/s")
        lines.append("")
    with open(os.path.join(out_dir, "kernel_trace_shapes.txt"), "w") as f:
        f.write("\n".join(lines))

    # ---- counters
    def counter_medians(d):
        """{(kernel, grid): {counter: median per dispatch}}, and the copy
        kernel's per-dispatch values."""
        per = {}
        for r in csv_rows(d, "counter_collection.csv"):
            short = _short_kernel(r["Kernel_Name"])
            key = (short, int(r["Grid_Size"]))
            per.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        out, copy, copy_grid = {}, None, -1
        for (kname, grid), cs in per.items():
            med = {c: _quantiles(v)["median"] for c, v in cs.items()}
            # the reference is the largest copy: host-to-device copies of
            # the inputs also run as copy kernels, on small grids
            if "copyBuffer" in kname and grid > copy_grid:
                copy, copy_grid = med, grid
            elif _is_library_kernel(kname):
                out[(kname, grid)] = med
        return out, copy

    traffic = []
    copy_bytes = COPY_MIB << 20
    for key, d in runs.items():
        if not key.startswith("fetch_"):
            continue
        base = key[len("fetch_"):]
        sh = shape_of(d)
        fetch, fcopy = counter_medians(d)
        write, wcopy = counter_medians(runs["write_" + base])
        fscale = copy_bytes / (fcopy["FETCH_SIZE"] * 1024)
        wscale = copy_bytes / (wcopy["WRITE_SIZE"] * 1024)
        rec = {"shape": sh["shape"], "ring": sh["ring"], "M": sh["M"], "N": sh["N"], "K": sh["K"],
               "launch": sh["launch"], "explicit_launch": sh.get("explicit_launch", False),
               "items_per_dispatch": sh["items_per_call"],
               "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
               "kernels": [], "commands": [cmds[key], cmds["write_" + base]]}
        fetch_b = sum(v["FETCH_SIZE"] for v in fetch.values()) * 1024 * fscale
        write_b = sum(v["WRITE_SIZE"] for v in write.values()) * 1024 * wscale
        for kk in sorted(fetch):
            rec["kernels"].append({"kernel": kk[0], "grid": kk[1],
                                   "fetch_kib": fetch[kk]["FETCH_SIZE"],
                                   "write_kib": write.get(kk, {}).get("WRITE_SIZE")})
        items = sh["items_per_call"]
        rec["hbm_bytes_per_item"] = int(round((fetch_b + write_b) / items))
        if ("tcp_" + base) in runs:
            tq, _ = counter_medians(runs["tcp_" + base])
            rec["l1"] = {c.replace("_sum", ""): sum(v.get(c, 0.0) for v in tq.values())
                         for c in COUNTER_PASSES["tcp"]}
            rec["commands"].append(cmds["tcp_" + base])
        if ("rdreq_" + base) in runs:
            rq, rcopy = counter_medians(runs["rdreq_" + base])
            dr, dcopy = counter_medians(runs["dram_" + base])
            req = {c: sum(v.get(c, 0.0) for v in rq.values()) for c in COUNTER_PASSES["rdreq"]}
            rd_bytes = (32 * req["TCC_EA0_RDREQ_32B_sum"] + 64 * req["TCC_EA0_RDREQ_64B_sum"]
                        + 128 * req["TCC_EA0_RDREQ_128B_sum"])
            dram_rd = 32 * sum(v.get("TCC_EA0_RDREQ_DRAM_32B_sum", 0.0) for v in dr.values())
            dram_wr = 32 * sum(v.get("TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", 0.0) for v in dr.values())
            rec["read_requests"] = {c.replace("TCC_EA0_", "").replace("_sum", ""): v
                                    for c, v in req.items()}
            rec["read_bytes_from_request_sizes"] = int(round(rd_bytes))
            rec["dram_read_bytes"] = int(round(dram_rd))
            rec["dram_write_bytes"] = int(round(dram_wr))
            rec["copy_reference"] = {
                "bytes_each_way": copy_bytes,
                "read_bytes_from_request_sizes": int(round(
                    32 * rcopy["TCC_EA0_RDREQ_32B_sum"] + 64 * rcopy["TCC_EA0_RDREQ_64B_sum"]
                    + 128 * rcopy["TCC_EA0_RDREQ_128B_sum"])),
                "dram_read_bytes": int(round(32 * dcopy["TCC_EA0_RDREQ_DRAM_32B_sum"])),
                "dram_write_bytes": int(round(32 * dcopy["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"]))}
            rec["commands"] += [cmds["rdreq_" + base], cmds["dram_" + base]]
        rec["algorithmic_bytes_per_item"] = algorithmic_bytes(sh["M"], sh["N"], sh["K"])
        rec["ratio"] = round(rec["hbm_bytes_per_item"] / rec["algorithmic_bytes_per_item"], 4)
        traffic.append(rec)
    # L1 -> L2 traffic of runs that have no fetch pass of their own
    for key, d in runs.items():
        if key.startswith("tcp_") and ("fetch_" + key[len("tcp_"):]) not in runs:
            sh = shape_of(d)
            tq, _ = counter_medians(d)
            traffic.append({"shape": sh["shape"], "ring": False, "M": sh["M"], "N": sh["N"],
                            "K": sh["K"], "launch": sh["launch"], "l1_only": True,
                            "explicit_launch": sh.get("explicit_launch", False),
                            "l1": {c.replace("_sum", ""): sum(v.get(c, 0.0) for v in tq.values())
                                   for c in COUNTER_PASSES["tcp"]},
                            "commands": [cmds[key]]})
    util = []
    for key, d in runs.items():
        if key.startswith("util_"):
            sh = shape_of(d)
            med, _ = counter_medians(d)
            util.append({"shape": sh["shape"], "M": sh["M"], "launch": sh["launch"],
                         "kernels": [{"kernel": kk[0], "grid": kk[1], **{c: round(v, 2)
                                                                         for c, v in cs.items()}}
                                     for kk, cs in sorted(med.items())],
                         "command": cmds[key]})
    with open(os.path.join(out_dir, "hbm_traffic_shapes.json"), "w") as f:
        json.dump({"kernel_source_digest": digest, "ring_source_digest": ring_digest,
                   "entries": traffic, "utilization": util}, f, indent=1)
    lines = ["HBM traffic per call (per item for ring launches), one rocprofv3 --pmc run per shape",
             "and counter set (program: bench.py --profile-shape; medians over the dispatches):",
             f"  fetch/write: FETCH_SIZE, WRITE_SIZE (KiB per dispatch) scaled by a plain {COPY_MIB} MiB",
             "    device copy in the same run (scale = copy bytes / what the counter reads for it);",
             "  rdreq: read bytes from the request-size counters 32*RDREQ_32B + 64*RDREQ_64B +",
             "    128*RDREQ_128B (TCC_EA0_*_sum), no scale factor;",
             "  dram: 32*TCC_EA0_RDREQ_DRAM_32B_sum and 32*TCC_EA0_WRREQ_WRITE_DRAM_32B_sum;",
             "  util: MfmaUtil and VALUBusy (percent);",
             "  tcp: TCP_TCC_READ_REQ (L1 -> L2 read requests), TCP_TOTAL_CACHE_ACCESSES (L1 tag",
             "    accesses) and TCP_TOTAL_READ, per call: the activation re-reads the workgroups pull.",
             f"Reduced with: python bench.py --summarize {root}",
             f"kernel sources digest {digest}, ring sources digest {ring_digest}", ""]
    for r in traffic:
        tag = "ring item" if r["ring"] else "call"
        lines.append(f"{'ring ' if r['ring'] else ''}{r['shape']} M={r['M']} N={r['N']} K={r['K']}  "
                     f"{'explicit ' if r.get('explicit_launch') else ''}launch {r['launch']}")
        if "l1" in r:
            l1 = r["l1"]
            lines.append(f"  L1 -> L2 read requests {l1['TCP_TCC_READ_REQ']:.0f}, L1 tag accesses "
                         f"{l1['TCP_TOTAL_CACHE_ACCESSES']:.0f}, reads from TA {l1['TCP_TOTAL_READ']:.0f}"
                         " (per call)")
        if r.get("l1_only"):
            for cmd in r["commands"]:
                lines.append(f"  command: {cmd}")
            lines.append("")
            continue
        for kk in r["kernels"]:
            lines.append(f"  {kk['kernel']:<44} grid {kk['grid']:>8}  fetch {kk['fetch_kib']:9.1f} KiB"
                         f"  write {kk['write_kib'] if kk['write_kib'] is not None else float('nan'):8.1f} KiB")
        lines.append(f"  per {tag}: FETCH x{r['fetch_scale']} + WRITE x{r['write_scale']} = "
                     f"{r['hbm_bytes_per_item']} B, algorithmic {r['algorithmic_bytes_per_item']} B, "
                     f"ratio {r['ratio']}")
        if "read_requests" in r:
            rr = r["read_requests"]
            lines.append(f"  read requests 32B {rr['RDREQ_32B']:.0f}  64B {rr['RDREQ_64B']:.0f}  "
                         f"128B {rr['RDREQ_128B']:.0f}  all {rr['RDREQ']:.0f}: "
                         f"{r['read_bytes_from_request_sizes']} B read; DRAM read "
                         f"{r['dram_read_bytes']} B, DRAM write {r['dram_write_bytes']} B")
            c = r["copy_reference"]
            lines.append(f"  copy reference ({c['bytes_each_way']} B each way): request sizes "
                         f"{c['read_bytes_from_request_sizes']} B read, DRAM {c['dram_read_bytes']} B"
                         f" read / {c['dram_write_bytes']} B write")
        for cmd in r["commands"]:
            lines.append(f"  command: {cmd}")
        lines.append("")
    for u in util:
        lines.append(f"utilization {u['shape']} M={u['M']} launch {u['launch']}")
        for kk in u["kernels"]:
            lines.append(f"  {kk['kernel']:<44} grid {kk['grid']:>8}  MfmaUtil {kk.get('MfmaUtil')}"
                         f"  VALUBusy {kk.get('VALUBusy')}")
        lines.append(f"  command: {u['command']}")
        lines.append("")
    with open(os.path.join(out_dir, "hbm_traffic_shapes.txt"), "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_dir}/kernel_trace_shapes.* ({len(trace)} shapes) and "
          f"hbm_traffic_shapes.* ({len(traffic)} shapes, {len(util)} utilization runs)")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s: float = 12.0):
    """The oracle (plain C, binary64) on the host cores for a bounded sample of
    the same sweep: whole steps until the budget is spent, with every host
    thread it may use (at most 16) and then with one thread; and per M the
    median us per call over 3 runs on each thread count."""
    import oracle
    import synthetic

    affinity = len(os.sched_getaffinity(0))
    threads = min(16, affinity)
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=0)
    oracle.gemm_bf16(x[:1], w[:16], threads)  # load the library
    step_bytes = sum(algorithmic_bytes(M) for M in MS)

    def run(nthreads, budget):
        steps, t0 = 0, time.perf_counter()
        while True:
            for M in MS:
                oracle.gemm_bf16(x[:M], w, nthreads)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget or steps >= 5000:
                return steps, el

    def per_m(nthreads, runs=3):
        out = {}
        for M in MS:
            ts = []
            for _ in range(runs):
                t0 = time.perf_counter()
                oracle.gemm_bf16(x[:M], w, nthreads)
                ts.append(time.perf_counter() - t0)
            us = sorted(ts)[len(ts) // 2] * 1e6
            out[str(M)] = {"median_us_per_call": round(us, 1),
                           "GBs": round(algorithmic_bytes(M) / (us * 1e-6) / 1e9, 4)}
        return out

    steps, el = run(threads, budget_s)
    steps1, el1 = run(1, budget_s / 3)
    per_step, per_step1 = el / steps, el1 / steps1
    return {"value": round(step_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} steps of the M=1,2,4,8,16 sweep on one weight "
                      f"({el:.1f} s, {per_step * 1e3:.1f} ms/step)",
            "value_1_thread": round(step_bytes / per_step1 / 1e9, 4),
            "sample_1_thread": f"{steps1} steps ({el1:.1f} s, {per_step1 * 1e3:.1f} ms/step)",
            "per_m": {"threads": threads, **per_m(threads)},
            "per_m_1_thread": per_m(1),
            "host": {"nproc": os.cpu_count(), "affinity": affinity, "cpu_model": _cpu_model()}}


def epilogue_timing(sk, synthetic, dev, stream, reps: int = 50):
    """us/call of the full pooler GEMM (M=8, N=4096, K=8192, on a 16-layer
    ring) and of RMSNorm -> NVFP4 on [8, 4096] (latency-bound: ~92 KB)."""
    import torch

    M, N2, K2 = 8, 4096, 8192
    ring = synthetic.device_weight_ring(16, N2, K2, dev, base_seed=5000)
    xb, _ = synthetic.gemm_inputs(N=16, K=K2, seed=1)
    x = synthetic.to_device(xb[:M], dev)
    y = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
    nw = synthetic.to_device(synthetic.norm_weight(N2, seed=1), dev)
    gs = torch.tensor([100.0], dtype=torch.float32, device=dev)
    a = torch.empty((M, N2 // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((M, N2 // 16), dtype=torch.uint8, device=dev)

    def timed(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for f in fns:
                f()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(fns))

    gemm_us = timed([lambda w=w: sk.skinny_gemm_bf16(x, w, y, 0) for w in ring])
    norm_us = timed([lambda: sk.skinny_rmsnorm_nvfp4(y, nw, 1.0, 1e-6, gs, a, sf)] * 16)
    del ring
    # The dual norm after the o_proj shard (H = 8192) at M = 8.
    H = 8192
    part = torch.randn((M, H), device=dev).to(torch.bfloat16)
    resid = torch.randn((M, H), device=dev)
    vecs = [torch.randn(H, device=dev).to(torch.bfloat16) for _ in range(4)]
    dout = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    dual_us = timed([lambda: sk.skinny_dual_norm(part, resid, vecs[0], 1.0, 1e-6, vecs[1],
                                                 vecs[2], vecs[3], 1.0, 1e-6, dout)] * 16)
    gbytes = algorithmic_bytes(M, N2, K2)
    return {"workload": "full pooler GEMM M=8 N=4096 K=8192 -> RMSNorm -> NVFP4 [8, 4096]",
            "gemm_us_per_call": round(gemm_us, 3),
            "gemm_GBs": round(gbytes / (gemm_us * 1e-6) / 1e9, 1),
            "gemm_launch": dict(sk.skinny_choose(M, N2, K2, 0)._asdict()),
            "norm_nvfp4_us_per_call": round(norm_us, 3),
            "dual_norm_us_per_call": round(dual_us, 3),
            "dual_norm_workload": "M=8, H=8192 (o_proj output), post weight, per-channel alpha"}


def ring_timing(sk, synthetic, dev, stream, ring, reps: int = 10):
    """The layer ring (skinny_gemm_bf16_ring): per-item us when the same
    60-layer unpooler weight ring runs as one 60-item launch per M, each item
    with its own activations, at the ring chooser's launch."""
    import torch

    out = {}
    xb = [synthetic.gemm_inputs(N=16, K=K, seed=900 + i)[0] for i in range(RING)]
    for M in MS:
        xs = [synthetic.to_device(b[:M], dev) for b in xb]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(RING)]
        sk.skinny_gemm_bf16_ring(xs, ring, ys)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            sk.skinny_gemm_bf16_ring(xs, ring, ys)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * RING)
        gbs = algorithmic_bytes(M) / (us * 1e-6) / 1e9
        r = sk.skinny_ring_choose(M, N, K, RING)
        out[str(M)] = {"launch": {**dict(r.gemm._asdict()), "segment": r.segment,
                                  "workgroups": r.workgroups, "order": r.order},
                       "us_per_item": round(us, 3), "GBs": round(gbs, 1),
                       "pct_peak": round(100 * gbs / PEAK_GBS, 2),
                       "hbm_bytes_per_item": ring_traffic(M, sk)}
        del g
    return {"workload": f"unpooler shard GEMM M=1,2,4,8,16, N=1024, K=4096: one "
                        f"{RING}-item skinny_gemm_bf16_ring launch per M over the "
                        f"{RING}-layer weight ring", "per_m": out}


def _graph_us(fn, stream, reps: int = 10) -> float:
    """us per launch of fn() (RING launches) from replays of its graph."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * RING)


def stream_ceiling(sk, dev, stream, ring) -> dict:
    """The stream references of libskinny_ceiling reading each weight of a
    ring once per launch, graphs of RING launches as the calls are timed;
    best of 1, 2, 4, 8 loads per lane: skinny_ceiling_stream (loads only) and
    skinny_ceiling_stream_store (the loads, then the cross-wave combine and
    store a GEMM workgroup ends with)."""
    import torch

    from moe_decode_skinny_amd import ceiling as cl

    nbytes = ring[0].numel() * ring[0].element_size()
    by_l, by_l_store = {}, {}
    for L in (1, 2, 4, 8):
        sinks = [torch.zeros(nbytes // (8192 * L), dtype=torch.int32, device=dev) for _ in ring]
        by_l[L] = _graph_us(lambda: [cl.skinny_ceiling_stream(w, s, L)
                                     for w, s in zip(ring, sinks)], stream)
        del sinks
        outs = [torch.zeros(64 * nbytes // (8192 * L), dtype=torch.int32, device=dev)
                for _ in ring]
        by_l_store[L] = _graph_us(lambda: [cl.skinny_ceiling_stream_store(w, o, L)
                                           for w, o in zip(ring, outs)], stream)
        del outs
    L = min(by_l, key=by_l.get)
    us = by_l[L]
    Ls = min(by_l_store, key=by_l_store.get)
    us_s = by_l_store[Ls]
    return {"bytes": nbytes, "stream_us": round(us, 3),
            "stream_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "stream_pct_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_GBS, 2),
            "stream_loads_per_lane": L, "stream_workgroups": nbytes // (8192 * L),
            "stream_us_by_loads_per_lane": {str(k): round(v, 3) for k, v in by_l.items()},
            "stream_store_us": round(us_s, 3),
            "stream_store_pct_peak": round(100 * nbytes / (us_s * 1e-6) / 1e9 / PEAK_GBS, 2),
            "stream_store_loads_per_lane": Ls,
            "stream_store_us_by_loads_per_lane": {str(k): round(v, 3)
                                                  for k, v in by_l_store.items()}}


def ceiling_timing(sk, dev, stream, ring):
    """What one launch on this device reaches by itself, measured as the calls
    are (graphs of 60 launches over the same 60-layer weight ring): an empty
    kernel, and the stream references reading each 8 MiB weight once (loads
    only, and loads then a GEMM workgroup's combine and store)."""
    from moe_decode_skinny_amd import ceiling as cl

    empty = _graph_us(lambda: [cl.skinny_ceiling_empty(dev) for _ in range(RING)], stream)
    return {"workload": f"one launch per weight of the {RING}-layer unpooler ring",
            "empty_launch_us": round(empty, 3), **stream_ceiling(sk, dev, stream, ring)}


def oproj_timing(sk, synthetic, dev, stream, reps: int = 10):
    """The o_proj shard (N=8192, K=1024, 16 MiB of weights) on its own
    60-layer ring: us per single call (graph of 60 calls) and per ring item
    (one 60-item launch), M = 1..16."""
    out, ceiling = shard_timing(sk, synthetic, dev, stream, 8192, 1024, MS, 7000, 950, reps)
    return {"workload": f"o_proj shard GEMM M=1,2,4,8,16, N=8192, K=1024, {RING}-layer weight "
                        "ring: single calls and one ring launch per M", "per_m": out,
            "stream_ceiling": ceiling}


def pooler_timing(sk, synthetic, dev, stream, reps: int = 5):
    """The pooler shard (N=512, K=8192) and the single-GPU full pooler
    (N=4096, K=8192, 64 MiB of weights), each on its own 60-layer ring, at
    M = 1, 8, 16: us per single call and per ring item."""
    shard, shard_ceiling = shard_timing(sk, synthetic, dev, stream, 512, 8192, (1, 8, 16), 7100,
                                        960, reps)
    full, full_ceiling = shard_timing(sk, synthetic, dev, stream, 4096, 8192, (1, 8, 16), 7200,
                                      970, reps)
    return {"workload": f"pooler shard N=512, K=8192 and full pooler N=4096, K=8192 at "
                        f"M=1,8,16, {RING}-layer weight rings: single calls and one ring "
                        "launch per M", "shard": shard, "full": full,
            "stream_ceiling": {"shard": shard_ceiling, "full": full_ceiling}}


def shard_timing(sk, synthetic, dev, stream, N2, K2, ms, wseed, xseed, reps):
    import torch

    ring = synthetic.device_weight_ring(RING, N2, K2, dev, base_seed=wseed)

    def timed(fn, per):
        # the median of three timings of `reps` replays each
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        g.replay()
        torch.cuda.synchronize()
        runs = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e3 / (reps * per))
        return sorted(runs)[1]

    out = {}
    ceiling = stream_ceiling(sk, dev, stream, ring)
    for M in ms:
        xs = [synthetic.to_device(synthetic.gemm_inputs(N=16, K=K2, seed=xseed + i)[0][:M], dev)
              for i in range(RING)]
        ys = [torch.empty((M, N2), dtype=torch.bfloat16, device=dev) for _ in range(RING)]
        single = timed(lambda: [sk.skinny_gemm_bf16(x, w, y, 0) for x, w, y in zip(xs, ring, ys)],
                       RING)
        item = timed(lambda: sk.skinny_gemm_bf16_ring(xs, ring, ys), RING)
        b = algorithmic_bytes(M, N2, K2)
        out[str(M)] = {"walk": walk_record(sk, M, N2, K2), "us_per_call": round(single, 3),
                       "fraction_of_stream_ceiling": round(ceiling["stream_us"] / single, 4),
                       "fraction_of_stream_store_ceiling": round(
                           ceiling["stream_store_us"] / single, 4),
                       "pct_peak_call": round(100 * b / (single * 1e-6) / 1e9 / PEAK_GBS, 2),
                       "ring_us_per_item": round(item, 3),
                       "pct_peak_ring": round(100 * b / (item * 1e-6) / 1e9 / PEAK_GBS, 2)}
        del xs, ys
    del ring
    torch.cuda.empty_cache()
    return out, ceiling


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="ring passes per launch shape for the per-kernel timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (the reference "
                         "kernel that scales hardware byte counters in a counter run)")
    ap.add_argument("--profile-shape", default="",
                    help="profiling run: <shape>:<M> (shapes: " + ", ".join(SHAPES) +
                         ") runs that shape's chooser call over its weight ring; "
                         "ring:<shape>:<M> its 60-item ring launch")
    ap.add_argument("--passes", type=int, default=TRACE_PASSES,
                    help="profiling run: ring passes replayed after 3 warm ones")
    ap.add_argument("--profile-out", default="", help="profiling run: directory for shape.json")
    ap.add_argument("--launch", default="",
                    help="profiling run: an explicit launch path,splits,waves,chunks,accs,rows")
    ap.add_argument("--profile-commands", action="store_true",
                    help="print the rocprofv3 command of every profiling run and exit")
    ap.add_argument("--summarize", default="",
                    help="reduce the profiling runs under this directory to profiles/*_shapes.*")
    args = ap.parse_args()
    if args.profile_commands:
        for d, p, b in profile_runs():
            print(profile_command(d, p, b))
        return
    if args.summarize:
        summarize_profiles(args.summarize, os.path.join(HERE, "profiles"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this GEMM is one GPU's shard and the "
              "library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.profile_shape:
        profile_shape(args.profile_shape, args.passes, args.profile_out or ".", args.copy_mib,
                      args.launch)
        return

    import torch

    import moe_decode_skinny_amd as sk
    import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sk.skinny_init(0)
    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"device {torch.cuda.get_device_name(dev)}; building the {RING}-layer ring")
    ring = synthetic.device_weight_ring(RING, N, K, dev)
    x_bits, _ = synthetic.gemm_inputs(N=16, K=K, seed=0)
    xs = {M: synthetic.to_device(x_bits[:M], dev) for M in MS}
    ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for M in MS}
    launches = {M: sk.skinny_choose(M, N, K, 0) for M in MS}
    stream = torch.cuda.Stream(dev)

    # The decode loop records one pass over the layer ring as one graph: step
    # i runs the sweep M = 1..16 on layers 5 (i % 12) .. + 4, and a graph
    # holds the 12 steps of a ring pass (60 calls); K steps replay it K // 12
    # times, then a graph of the first K % 12 steps.
    groups = RING // len(MS)

    def record(n_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for gi in range(n_steps):
                for j, M in enumerate(MS):
                    sk.skinny_gemm_bf16(xs[M], ring[gi * len(MS) + j], ys[M], 0)
        return g

    with torch.cuda.stream(stream):
        for M in MS:  # eager warm-up of every launch
            sk.skinny_gemm_bf16(xs[M], ring[0], ys[M], 0)
        torch.cuda.synchronize()
        full = record(groups)
        tails = {r: record(r) for r in {args.steps % groups, args.warmup % groups} if r}
        torch.cuda.synchronize()

        def run_steps(n):
            for _ in range(n // groups):
                full.replay()
            if n % groups:
                tails[n % groups].replay()

        run_steps(args.warmup)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        run_steps(args.steps)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = start.elapsed_time(end) / args.steps

        # Per-launch durations: a graph of one launch shape over the whole ring.
        per_kernel = {}
        for M in MS:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for l in range(RING):
                    sk.skinny_gemm_bf16(xs[M], ring[l], ys[M], 0)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.kernel_reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / (args.kernel_reps * RING)
            per_kernel[M] = us
            del g

        # The expert-input epilogue (pooler page): full-pooler GEMM at M=8,
        # then RMSNorm -> NVFP4 on its output, both timed per call.
        epi = epilogue_timing(sk, synthetic, dev, stream)
        # The same weight ring through the layer-ring launch.
        ring_out = ring_timing(sk, synthetic, dev, stream, ring)
        # The other shard the target names.
        oproj_out = oproj_timing(sk, synthetic, dev, stream)
        # The pooler shapes (K = 8192).
        pooler_out = pooler_timing(sk, synthetic, dev, stream)
        # What a single launch reaches by itself on this device.
        ceiling = ceiling_timing(sk, dev, stream, ring)

    step_bytes = sum(algorithmic_bytes(M) for M in MS)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dom = max(MS, key=lambda M: per_kernel[M])
    ach = algorithmic_bytes(dom) / (per_kernel[dom] * 1e-6) / 1e9
    detail = {str(M): {"launch": dict(launches[M]._asdict()),
                       "walk": walk_record(sk, M, N, K),
                       "us_per_call": round(per_kernel[M], 3),
                       "fraction_of_stream_ceiling": round(ceiling["stream_us"] / per_kernel[M], 4),
                       "fraction_of_stream_store_ceiling": round(
                           ceiling["stream_store_us"] / per_kernel[M], 4),
                       "GBs": round(algorithmic_bytes(M) / (per_kernel[M] * 1e-6) / 1e9, 1),
                       "pct_peak": round(100 * algorithmic_bytes(M) / (per_kernel[M] * 1e-6)
                                         / 1e9 / PEAK_GBS, 2)}
              for M in MS}
    out = {
        "metric": "achieved HBM GB/s (and us/call) of the M=1..16 skinny BF16 GEMM sweep",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "unpooler shard GEMM sweep M=1,2,4,8,16, N=1024, K=4096, "
                               f"{RING}-layer weight ring, chooser launch shapes",
                   "global_batch": list(MS), "parallelism": "single GPU shard"},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_GBS, 4),
                     "traffic": measured_traffic(dom, sk),
                     "kernel": f"M={dom} {walk_record(sk, dom, N, K)}",
                     "bytes_per_launch": algorithmic_bytes(dom),
                     "us_per_launch": round(per_kernel[dom], 3),
                     "traced": traced_call(dom, sk)},
        "per_m": detail,
        "ceiling": {**ceiling,
                    "dominant_call_fraction": round(ceiling["stream_us"] / per_kernel[dom], 4),
                    "dominant_call_fraction_of_stream_store": round(
                        ceiling["stream_store_us"] / per_kernel[dom], 4)},
        "epilogue": epi,
        "ring": ring_out,
        "oproj": oproj_out,
        "pooler": pooler_out,
        "wall_s": round(wall, 6),
        "timed_region_s": round(ms_step * args.steps * 1e-3, 6),
    }
    # Release the device before the host-only part, so nothing holds the GPU
    # while the CPU baseline runs and the process ends with nothing pending.
    del full, tails, ring, xs, ys
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    main()
