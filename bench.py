#!/usr/bin/env python3
"""Throughput of the fused ring all-reduce over p virtual ranks on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--extra]

One step is one collective call over one batch of synthetic rank buffers
already resident in HBM.  The default workload is the largest one: the
row-parallel partial outputs of a tensor-parallel linear layer, p = 8 ranks x
(8, 2048, 4096) bfloat16 (128 MiB per rank), sum all-reduce through
``rr_all_reduce`` -- host validation and planning, the ring chunk plan, and
the single fused kernel that folds every chunk in ring order in float32 and
writes all p outputs (reduce-scatter and all-gather in one pass).

Metric: algorithmic HBM bytes per step / time, bytes = 2 p n s for an
all-reduce (every input read once, every output written once), in GB/s
(10^9 B/s), and its fraction of MI355X's 8 TB/s HBM peak.  Steps rotate over
enough buffer sets that each set is evicted from the 256 MB Infinity Cache by
>= 512 MiB of other traffic before it is used again (cold cache).  A bounded
spin kernel queued before the timed region lets the host run ahead, so host
launch cost does not idle the GPU.

Besides the timed region, the line reports the spread of single launches (a
separate pass with events around every launch), the copy ceilings of the
same machine (a 1 GiB hipMemcpyAsync device-to-device copy and librr's own copy
kernel), and the CPU oracle timed on the host's cores.

Prints ONE JSON line on stdout.  ``--extra`` prints further measurements
(the other workloads and collectives, staged algorithms, cache-hot figures)
as JSON lines on stderr.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "all-reduce effective HBM GB/s (p·N bytes in+out / time) and % of MI355X HBM peak"
HBM_PEAK_GBPS = 8000.0
COLD_BYTES = 512 << 20
DTYPE_TAG = {"int32": "i32", "float32": "f32", "bfloat16": "bf16", "float16": "f16"}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="tp_rowparallel_bf16_p8")
    ap.add_argument("--spread-steps", type=int, default=50,
                    help="launches of the separate per-launch pass (min / median / max); 0 = skip")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy ceilings")
    ap.add_argument("--op", default=None, help="sum, max or min (default: the workload's first op)")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate over (0 = enough for a cold cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extra", action="store_true", help="also measure the other collectives (stderr)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="launch one plain 256 MiB copy (librr's copy kernel) before timing, as the known-size "
                         "reference for HBM byte counters")
    ap.add_argument("--probe-cases", action="store_true",
                    help="run copies of known size (64 MiB to 512 MiB) and one launch pair of each workload's "
                         "collectives, separated by spin-kernel markers, for rocprofv3 --pmc runs; then exit")
    ap.add_argument("--survey", action="store_true",
                    help="measure every collective, float32 and bfloat16, p = 8, at per-rank sizes from 2 to 128 MiB "
                         "(one JSON line per dtype and collective, percent of the HBM peak); then exit")
    ap.add_argument("--ingest-probe", nargs="+", metavar="DB",
                    help="print per-case counter values of --probe-cases runs (rocprofv3 *_results.db files)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH", "WRITE"),
                    help="turn the outputs of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; *_results.db or "
                         "counter_collection.csv) into the traffic record under profiles/, then exit")
    return ap.parse_args(argv)


CALIB_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
# Sources that define the fused all-reduce kernel; the traffic record is
# valid only while their contents are unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "collective_communication_reduction_way_amd", "csrc", f) for f in
                  ("rr_device.h", "rr_kernels.h", "rr_fold_impl.h", "rr_phase.h", "rr_phase_impl.h", "rr_sync.h",
                   "rr_phase_ring.hip", "rr_phase_hier.hip", "rr_phase.cpp")]


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_path(workload):
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def load_traffic(workload):
    """HBM bytes per launch of the fused kernel from the committed counter
    record, or None when there is none or the kernel changed since."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def ingest_pmc(workload, fetch_path, write_path):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the fused kernel, each
    scaled by what the same counter reads for the calibration copy of known
    size (the run's first librr copy dispatch, launched by
    --calibration-copy before anything else of librr), averaged over the
    profiled launches of the fused kernel.  Reads rocprofv3's SQLite output
    (*_results.db, view counters_collection)."""
    import sqlite3

    def dispatches(path, counter):
        con = sqlite3.connect(path)
        rows = con.execute("select dispatch_id, kernel_name, value from counters_collection where counter_name = ? "
                           "order by dispatch_id", (counter,)).fetchall()
        con.close()
        return rows

    rec = {"workload": workload, "kernel_source_sha256": kernel_source_hash(), "counters": {}}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_path), ("WRITE_SIZE", write_path)):
        rows = dispatches(path, counter)
        calib = [v for _, name, v in rows if "k_fanout" in name][:1]
        fused = [v for _, name, v in rows if "k_phase" in name]
        if not calib or not fused:
            raise SystemExit(f"{path}: no calibration-copy or fused-kernel dispatches found")
        calib_kib = calib[0]
        scale = CALIB_BYTES / (calib_kib * 1024.0)
        per_launch = sum(fused) / len(fused) * 1024.0 * scale
        rec["counters"][counter] = {"fused_kib_per_dispatch_mean": sum(fused) / len(fused),
                                    "fused_dispatches": len(fused), "calibration_kib": calib_kib,
                                    "calibration_bytes": CALIB_BYTES, "scale": scale,
                                    "bytes_per_launch": per_launch}
        total += per_launch
    rec["hbm_bytes_per_launch"] = total
    with open(traffic_path(workload), "w", encoding="utf-8") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


PROBE_CASES = [
    # (name, algorithmic read bytes, algorithmic write bytes) per launch
    ("copy_64MiB", 64 << 20, 64 << 20), ("copy_96MiB", 96 << 20, 96 << 20), ("copy_128MiB", 128 << 20, 128 << 20),
    ("copy_256MiB", 256 << 20, 256 << 20), ("copy_512MiB", 512 << 20, 512 << 20),
    ("ar_fp32_p8_8MiB all_reduce", 8 * (8 << 20), 8 * (8 << 20)),
    ("hier_bf16_p8g4_8MiB all_reduce", 8 * (8 << 20), 8 * (8 << 20)),
    ("zero_bucket_fp32_p8 all_reduce", 8 * (96 << 20), 8 * (96 << 20)),
    ("zero_bucket_fp32_p8 reduce_scatter", 8 * (96 << 20), 96 << 20),
    ("zero_bucket_fp32_p8 all_gather", 96 << 20, 8 * (96 << 20)),
    ("zero_bucket_fp32_p8 broadcast", 96 << 20, 8 * (96 << 20)),
    ("tp_rowparallel_bf16_p8 all_reduce", 8 * (128 << 20), 8 * (128 << 20)),
]


def probe_cases():
    """Each case of PROBE_CASES launched twice, after a one-workgroup spin
    kernel that marks where the case's dispatches begin (for --ingest-probe).
    Inputs are drawn on the device: only the bytes matter here.  Copies are
    librr's copy kernel (a broadcast to one rank)."""
    import torch

    import collective_communication_reduction_way_amd as rr

    dev = torch.device("cuda", 0)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)

    def case(fn):
        torch.cuda._sleep(1)  # the marker
        for _ in range(2):
            fn()
        torch.cuda.synchronize()

    for mib in (64, 96, 128, 256, 512):
        src = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        case(lambda: rr.broadcast(src, [dst], root=0))
        del src, dst
        torch.cuda.empty_cache()

    def pair(p, n, dt):
        x = torch.randn((p, n), device=dev, generator=g).to(dt)
        return x, torch.empty_like(x)

    x, y = pair(8, 2097152, torch.float32)
    case(lambda: rr.all_reduce(x, y))
    x, y = pair(8, 4194304, torch.bfloat16)
    case(lambda: rr.all_reduce(x, y, algo="hier", group_size=4))
    del x, y
    torch.cuda.empty_cache()
    x, y = pair(8, 25165824, torch.float32)
    sh = torch.empty((8, 25165824 // 8), device=dev)
    case(lambda: rr.all_reduce(x, y))
    case(lambda: rr.reduce_scatter(x, sh))
    case(lambda: rr.all_gather(sh, y))
    case(lambda: rr.broadcast(x[0], y, root=0))
    del x, y, sh
    torch.cuda.empty_cache()
    x, y = pair(8, 67108864, torch.bfloat16)
    case(lambda: rr.all_reduce(x, y))
    torch.cuda._sleep(1)
    torch.cuda.synchronize()
    print(json.dumps({"probe_cases": [c[0] for c in PROBE_CASES]}), flush=True)
    return 0


def ingest_probe(dbs):
    """Per case of --probe-cases: the librr kernels' counter values (last of
    the case's two launches), each HBM byte counter against the case's
    algorithmic bytes.  TCC_EA0_RDREQ_DRAM_32B / TCC_EA0_WRREQ_WRITE_DRAM_32B
    count 32-byte units (a 64-byte request as 2, a 128-byte one as 4);
    FETCH_SIZE / WRITE_SIZE are KiB."""
    import collections
    import sqlite3

    for db in dbs:
        con = sqlite3.connect(db)
        rows = con.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection "
                           "order by dispatch_id").fetchall()
        con.close()
        disp = collections.OrderedDict()
        for did, kn, cn, v in rows:
            d = disp.setdefault(did, {"k": kn, "c": {}})
            d["c"][cn] = d["c"].get(cn, 0.0) + v
        groups, cur = [], None
        for d in disp.values():
            if "spin_kernel" in d["k"]:
                if cur is not None:
                    groups.append(cur)
                cur = []
            elif cur is not None and "rr::" in d["k"]:
                cur.append(d)
        print(f"== {os.path.basename(db)}")
        for (name, rd, wr), grp in zip(PROBE_CASES, groups):
            kernels = collections.OrderedDict()
            for d in grp:
                kernels.setdefault(d["k"].replace("void rr::(anonymous namespace)::", "").split("(")[0], []).append(d)
            for kname, ds in kernels.items():
                c = ds[-1]["c"]
                cells = []
                for cn, v in sorted(c.items()):
                    if cn in ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", "FETCH_SIZE",
                              "WRITE_SIZE"):
                        unit = 32 if cn.endswith("32B_sum") else 1024
                        ref = rd if ("RDREQ" in cn or cn == "FETCH_SIZE") else wr
                        cells.append(f"{cn}={v:.0f} ({v * unit / ref:.4f}x)")
                    else:
                        cells.append(f"{cn}={v:.0f}")
                print(f"{name:36s} {kname[:48]:48s} " + " ".join(cells))


def busbw_gibps(kind, p, s_bytes, t_seconds):
    """The bandwidth formulas of page "分布式训练/推理", section "带宽怎么核算"
    (all-reduce 2s(p-1)/(p t); reduce-scatter s_in(p-1)/(p t)), in the page's
    printed unit, which is 2^30 bytes per second."""
    if kind == "all_reduce":
        return 2.0 * s_bytes * (p - 1) / (p * t_seconds) / 2 ** 30
    if kind == "reduce_scatter":
        return s_bytes * (p - 1) / (p * t_seconds) / 2 ** 30
    raise ValueError(kind)


class Runner:
    """Pre-marshalled calls of one collective over rotating buffer sets."""

    def __init__(self, rr, torch, spec, coll, op, algo, group, host_x, nsets, stream, hier_kw=None):
        import ctypes

        self.rr, self.torch, self.stream = rr, torch, stream
        self.L = rr.lib()
        hier_kw = hier_kw or {}
        p, n, dtype = spec["p"], spec["n"], spec["dtype"]
        self.p, self.n, self.dtype, self.coll, self.algo = p, n, dtype, coll, algo
        tdt = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16,
               "float16": torch.float16}[dtype]
        dev = torch.device("cuda", 0)
        import numpy as np

        if dtype in ("bfloat16", "float16"):
            host = torch.from_numpy(host_x.view(np.int16)).view(tdt)
        else:
            host = torch.from_numpy(host_x)
        L = n // p
        self.sets = []
        dt = rr.DTYPES[dtype]
        opc = rr.OPS[op]
        sh = stream.cuda_stream
        rows = spec.get("rows", 0)
        cols = n // rows if rows else 0
        for _ in range(nsets):
            if coll in ("all_gather", "gather", "all_gather_dim1"):
                x = host[:, :L].contiguous().to(dev)
                y = torch.empty((p, n), dtype=tdt, device=dev)
            elif coll == "scatter":
                x = host[:1].contiguous().to(dev)
                y = torch.empty((p, L), dtype=tdt, device=dev)
            else:
                x = host.to(dev)
                if coll in ("reduce_scatter", "reduce_scatter_dim1"):
                    y = torch.empty((p, L), dtype=tdt, device=dev)
                elif coll == "reduce":
                    y = torch.empty((1, n), dtype=tdt, device=dev)
                else:
                    y = torch.empty((p, n), dtype=tdt, device=dev)
            ws = None
            need = rr.workspace_size(algo, p, group, n, dtype) if coll == "all_reduce" else 0
            if coll == "all_reduce_hier":
                need = rr.hier_workspace_size(p, group, n, dtype, **hier_kw)
            if need:
                ws = torch.empty(need, dtype=torch.uint8, device=dev)
            send = rr._ptr_array([x[r].data_ptr() for r in range(x.shape[0])])
            recv = rr._ptr_array([y[r].data_ptr() for r in range(y.shape[0])])
            Lb = self.L
            if coll == "all_reduce" and algo == "ring":
                call = (lambda s=send, d=recv: Lb.rr_all_reduce(s, d, p, n, dt, opc, sh))
            elif coll == "all_reduce":
                ap, gp = rr.ALGOS[algo], group
                wp, wb = (ws.data_ptr(), need) if ws is not None else (None, 0)
                call = (lambda s=send, d=recv, ap=ap, gp=gp, wp=wp, wb=wb:
                        Lb.rr_all_reduce_ex(s, d, p, n, dt, opc, ap, gp, wp, wb, sh))
            elif coll == "reduce_scatter":
                call = (lambda s=send, d=recv: Lb.rr_reduce_scatter(s, d, p, n, dt, opc, sh))
            elif coll == "all_gather":
                call = (lambda s=send, d=recv: Lb.rr_all_gather(s, d, p, n, dt, sh))
            elif coll == "reduce":
                yp = y[0].data_ptr()
                call = (lambda s=send, yp=yp: Lb.rr_reduce(s, yp, 0, p, n, dt, opc, sh))
            elif coll == "broadcast":
                xp = x[0].data_ptr()
                call = (lambda xp=xp, d=recv: Lb.rr_broadcast(xp, d, 0, p, n, dt, sh))
            elif coll == "scatter":
                xp = x[0].data_ptr()
                call = (lambda xp=xp, d=recv: Lb.rr_scatter(xp, d, 0, p, n, dt, sh))
            elif coll == "gather":
                yp = y[0].data_ptr()
                call = (lambda s=send, yp=yp: Lb.rr_gather(s, yp, 0, p, n, dt, sh))
            elif coll == "all_reduce_hier":
                fl = rr._hier_flags(hier_kw.get("intra", "reduce"), hier_kw.get("wire_round", False),
                                    hier_kw.get("staged", False))
                wp, wb = (ws.data_ptr(), need) if ws is not None else (None, 0)
                call = (lambda s=send, d=recv, fl=fl, wp=wp, wb=wb:
                        Lb.rr_all_reduce_hier(s, d, p, n, dt, opc, group, fl, wp, wb, sh))
            elif coll == "reduce_scatter_dim1":
                call = (lambda s=send, d=recv: Lb.rr_reduce_scatter_dim1(s, d, p, rows, cols, dt, opc, sh))
            elif coll == "all_gather_dim1":
                call = (lambda s=send, d=recv: Lb.rr_all_gather_dim1(s, d, p, rows, cols, dt, sh))
            else:
                raise ValueError(coll)
            self.sets.append((x, y, ws, send, recv, call))
        base = {"all_reduce_hier": "all_reduce", "reduce_scatter_dim1": "reduce_scatter",
                "all_gather_dim1": "all_gather"}.get(coll, coll)
        self.bytes = rr.algorithmic_bytes(base, p, n, dtype)
        self._ctypes = ctypes

    def step(self, i):
        st = self.sets[i % len(self.sets)][5]()
        if st != 0:
            raise RuntimeError(f"librr call failed: {self.L.rr_last_error().decode()}")


class BucketRunner:
    """Pre-marshalled bucketed all-reduce calls over rotating buffer sets: the
    tensors of a named gradient bucket, one allocation per tensor and rank."""

    def __init__(self, rr, torch, W, name, op, nsets, stream):
        import ctypes

        spec = W.BUCKETS[name]
        self.L = rr.lib()
        p = spec["p"]
        parts = W.bucket_inputs(name)
        counts = [t.shape[1] for t in parts]
        dt, opc, sh = rr.DTYPES[spec["dtype"]], rr.OPS[op], stream.cuda_stream
        cnt = (ctypes.c_size_t * len(counts))(*counts)
        self.sets = []
        for _ in range(nsets):
            xs = [torch.from_numpy(t).to("cuda") for t in parts]
            ys = [torch.empty_like(x) for x in xs]
            send = rr._ptr_array([x[r].data_ptr() for x in xs for r in range(p)])
            recv = rr._ptr_array([y[r].data_ptr() for y in ys for r in range(p)])
            call = (lambda s=send, d=recv: self.L.rr_all_reduce_bucket(s, d, cnt, len(counts), p, dt, opc, sh))
            self.sets.append((xs, ys, send, recv, cnt, call))
        self.bytes = 2 * p * sum(counts) * 4

    def step(self, i):
        st = self.sets[i % len(self.sets)][-1]()
        if st != 0:
            raise RuntimeError(f"librr call failed: {self.L.rr_last_error().decode()}")


def spin_cycles_per_ms(torch, stream):
    """Calibrate torch's bounded spin kernel (used to let the host queue ahead)."""
    try:
        with torch.cuda.stream(stream):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            torch.cuda._sleep(1_000_000)
            b.record(stream)
        stream.synchronize()
        ms = a.elapsed_time(b)
        return 1_000_000 / ms if ms > 0 else None
    except Exception:  # noqa: BLE001 - the spin is an optimisation of the harness only
        return None


def timed(torch, runner, steps, warmup, stream, cycles_per_ms, per_launch=True):
    """Run `warmup` untimed steps, then exactly `steps` timed steps bracketed by
    synchronizations.  Returns (ms_per_step from the region events, mean
    per-launch kernel ms from per-launch events or None, wall seconds)."""
    for i in range(warmup):
        runner.step(i)
    torch.cuda.synchronize()
    # host cost of one step, to size the lead the spin kernel gives the host
    t0 = time.perf_counter()
    for i in range(5):
        runner.step(i)
    host_ms = (time.perf_counter() - t0) / 5 * 1e3
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(stream):
        if cycles_per_ms:
            lead_ms = min(50.0, 1.5 * steps * (host_ms + (0.02 if per_launch else 0.0)) + 0.5)
            torch.cuda._sleep(int(lead_ms * cycles_per_ms))
        start.record(stream)
        for i in range(steps):
            if per_launch:
                evs[i][0].record(stream)
            runner.step(warmup + i)
            if per_launch:
                evs[i][1].record(stream)
        end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    region_ms = start.elapsed_time(end)
    kern = None
    if per_launch:
        kern = sum(a.elapsed_time(b) for a, b in evs) / steps
    return region_ms / steps, kern, wall


def launch_spread(torch, runner, steps, stream, cycles_per_ms):
    """A separate pass (after the timed region, not inside it): `steps`
    launches, each between its own pair of HIP events on the launch stream,
    queued behind a spin so that they run back to back.  Returns min, median,
    max and mean per-launch milliseconds and the GB/s at the median and min."""
    times = []
    for i in range(3):
        runner.step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    with torch.cuda.stream(stream):
        if cycles_per_ms:
            torch.cuda._sleep(int(min(50.0, 0.05 * steps + 1.0) * cycles_per_ms))
        for i in range(steps):
            evs[i][0].record(stream)
            runner.step(i)
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) for a, b in evs)
    med = times[len(times) // 2] if len(times) % 2 else 0.5 * (times[len(times) // 2 - 1] + times[len(times) // 2])
    return {
        "launches": steps, "min_ms": round(times[0], 6), "median_ms": round(med, 6), "max_ms": round(times[-1], 6),
        "mean_ms": round(sum(times) / len(times), 6),
        "GBps_at_median": round(runner.bytes / (med * 1e-3) / 1e9, 2),
        "GBps_at_min": round(runner.bytes / (times[0] * 1e-3) / 1e9, 2),
    }


def copy_ceilings(torch, rr, stream, nbytes=1 << 30, reps=10):
    """What a plain copy reaches on the same machine, as the achievable reference
    for the collectives: a hipMemcpyAsync device-to-device copy of 1 GiB, and
    librr's own copy kernel (a broadcast to one rank: the fan-out kernel with
    one destination) on the same buffers.  GB/s count the bytes read plus the
    bytes written (2 x 1 GiB per copy)."""
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so.7")  # the HIP runtime torch has loaded
    hip.hipMemcpyAsync.restype = ctypes.c_int
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    for b in bufs:
        b.fill_(1)
    L = rr.lib()
    sh = stream.cuda_stream

    def memcpy(i):
        src, dst = bufs[i % 3], bufs[(i + 1) % 3]
        if hip.hipMemcpyAsync(dst.data_ptr(), src.data_ptr(), nbytes, 3, sh) != 0:  # 3: device to device
            raise RuntimeError("hipMemcpyAsync failed")

    def librr_copy(i):
        src, dst = bufs[i % 3], bufs[(i + 1) % 3]
        if L.rr_broadcast(src.data_ptr(), rr._ptr_array([dst.data_ptr()]), 0, 1, nbytes // 4, rr.DTYPES["float32"],
                          sh) != 0:
            raise RuntimeError(L.rr_last_error().decode())

    res = {}
    for name, fn in (("hip_memcpy_d2d_1GiB", memcpy), ("librr_copy_kernel_1GiB", librr_copy)):
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        gbps = 2 * nbytes / (ms * 1e-3) / 1e9
        res[name] = {"GBps": round(gbps, 2), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "ms": round(ms, 6)}
    del bufs
    torch.cuda.empty_cache()
    return res


def cpu_baseline(spec, host_x, op, seconds):
    """Time the oracle's literal ring simulation (as it stands, NumPy, one
    thread) on a bounded sample of the same inputs."""
    import numpy as np

    from oracle import collectives as C

    p, n, dtype = spec["p"], spec["n"], spec["dtype"]
    s = np.dtype(np.uint16 if dtype == "bfloat16" else np.float32).itemsize
    m = min(n, 1 << 21)  # elements per rank in the sample
    sample = np.ascontiguousarray(host_x[:, :m])
    fn = C.all_reduce_hier if spec["coll"] == "all_reduce" and spec["algo"] == "hier" else None
    reps = 0
    t0 = time.perf_counter()
    while True:
        if fn is not None:
            fn(sample, op, dtype, spec["group"])
        else:
            C.all_reduce_ring(sample, op, dtype)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    bytes_per = 2 * p * m * s
    what = "all_reduce_hier" if fn is not None else "all_reduce_ring"
    threaded = None if fn is not None else threaded_formula_fold(sample, op, dtype, min(seconds, 5.0))
    return {
        "value": round(bytes_per * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"oracle.{what} (NumPy, 1 thread) on the first {m} of {n} elements of each of the {p} "
                  f"ranks of the same inputs, {reps} calls in {el:.1f} s",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "numpy": np.__version__,
        "threaded_formula_fold": threaded,
    }


def threaded_formula_fold(sample, op, dtype, seconds):
    """Second CPU timing: the oracle's per-chunk ring-order fold (the steps of
    oracle.all_reduce_fold: to_acc, combine in the order x_{c+1}, ..., x_c,
    finish, from_acc) over pieces of every chunk in a thread pool with one
    worker per CPU of the affinity set (NumPy releases the GIL in its loops);
    every rank's output row is written, as in the all-reduce.  The result is
    checked against oracle.all_reduce_fold before timing."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import collectives as C

    p, m = sample.shape
    threads = len(os.sched_getaffinity(0))
    b = C.chunk_bounds(m, p)
    pieces = []
    for c in range(p):
        lo, hi = b[c], b[c + 1]
        k = max(1, min(threads, (hi - lo) // 4096))
        for j in range(k):
            a0 = lo + (hi - lo) * j // k
            a1 = lo + (hi - lo) * (j + 1) // k
            if a1 > a0:
                pieces.append((c, a0, a1))
    out = np.empty_like(sample)

    def work(piece):
        # the steps of oracle.all_reduce_fold, on one piece of chunk c
        c, a0, a1 = piece
        acc = C.to_acc(sample[(c + 1) % p, a0:a1], dtype)
        for k in range(2, p + 1):
            acc = C.combine(acc, C.to_acc(sample[(c + k) % p, a0:a1], dtype), op)
        out[:, a0:a1] = C.from_acc(C.finish(acc, op, p), dtype)[None, :]

    with ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(work, pieces))
        if not np.array_equal(out.view(np.uint8), C.all_reduce_fold(sample, op, dtype).view(np.uint8)):
            raise RuntimeError("threaded formula fold differs from oracle.all_reduce_fold")
        reps = 0
        t0 = time.perf_counter()
        while True:
            list(pool.map(work, pieces))
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                break
    s = sample.dtype.itemsize
    return {
        "value": round(2 * p * m * s * reps / el / 1e9, 4),
        "unit": "GB/s",
        "threads": threads,
        "sample": f"the steps of oracle.all_reduce_fold over {len(pieces)} pieces of the {p} chunks of the same "
                  f"sample, {threads} worker threads, {reps} calls in {el:.1f} s",
    }


SURVEY_MIB = (2, 4, 6, 8, 10, 12, 16, 20, 24, 28, 32, 40, 48, 64, 96, 128)


def survey(steps):
    """Every collective of the library on synthetic float32 and bfloat16
    inputs, p = 8, at the per-rank sizes of SURVEY_MIB: for each, the rate
    over `steps` timed launches with the cold-cache buffer rotation of the
    bench line, as a fraction of the HBM peak (algorithmic bytes)."""
    import numpy as np
    import torch

    import collective_communication_reduction_way_amd as rr

    stream = torch.cuda.Stream()
    cpm = spin_cycles_per_ms(torch, stream)
    reads_writes = {"all_reduce": 16, "reduce_scatter": 9, "all_gather": 9, "reduce": 9, "broadcast": 16}
    for dtype, esz in (("float32", 4), ("bfloat16", 2)):
        for coll in ("all_reduce", "reduce_scatter", "all_gather", "reduce", "broadcast"):
            row = {}
            for mib in SURVEY_MIB:
                n = (mib << 20) // esz
                spec = dict(p=8, n=n, dtype=dtype)
                x = np.random.default_rng(mib).standard_normal((8, n), dtype=np.float32)
                if dtype == "bfloat16":
                    x = (x.view(np.uint32) >> 16).astype(np.uint16)
                nsets = 1 + math.ceil(COLD_BYTES / (reads_writes[coll] * n * esz))
                r = Runner(rr, torch, spec, coll, "sum", "ring", 0, x, nsets, stream)
                ms, _, _ = timed(torch, r, steps, 5, stream, cpm, per_launch=False)
                row[str(mib)] = round(r.bytes / ms / 1e6 / HBM_PEAK_GBPS * 100, 1)
                del r
                torch.cuda.empty_cache()
            print(json.dumps({"survey": coll, "dtype": dtype, "p": 8, "pct_of_hbm_peak_by_MiB_per_rank": row}),
                  flush=True)
    return 0


def main(argv=None):
    args = parse_args(argv)
    if args.ingest_pmc:
        ingest_pmc(args.workload, *args.ingest_pmc)
        return 0
    if args.ingest_probe:
        ingest_probe(args.ingest_probe)
        return 0
    if args.probe_cases:
        return probe_cases()
    if args.survey:
        return survey(min(args.steps, 40))
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the p virtual ranks live in one GPU's HBM and no collective crosses "
              f"GPUs; --gpus {args.gpus} is not supported (run with --gpus 1).", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import collective_communication_reduction_way_amd as rr
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    spec = W.WORKLOADS[args.workload]
    op = args.op or spec["ops"][0]
    algo = "hier" if spec["algo"] == "hier" else "ring"
    group = spec.get("group", 0)
    p, n, dtype = spec["p"], spec["n"], spec["dtype"]
    host_x = W.make_inputs(args.workload)
    stream = torch.cuda.Stream()  # default priority
    footprint = 2 * p * n * np.dtype(W.STORAGE[dtype]).itemsize
    nsets = args.sets or (1 + math.ceil(COLD_BYTES / footprint))
    runner = Runner(rr, torch, spec, "all_reduce", op, algo, group, host_x, nsets, stream)
    if args.calibration_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        st = rr.lib().rr_broadcast(src.data_ptr(), rr._ptr_array([dst.data_ptr()]), 0, 1, CALIB_BYTES // 4,
                                   rr.DTYPES["float32"], stream.cuda_stream)
        if st != 0:
            raise RuntimeError(rr.lib().rr_last_error().decode())
        stream.synchronize()
        del src, dst
    cpm = spin_cycles_per_ms(torch, stream)
    # The timed region: exactly `steps` steps between HIP events on the launch
    # stream.  One step is one launch of the fused kernel (the workloads have
    # no chunk heads or tails, so no second launch), so the kernel's average
    # launch duration is the region divided by the launches.
    ms_step, _, wall = timed(torch, runner, args.steps, args.warmup, stream, cpm, per_launch=False)
    launch_ms = ms_step
    value = runner.bytes / (ms_step * 1e-3) / 1e9
    achieved = runner.bytes / (launch_ms * 1e-3) / 1e9
    kernel = {"ring": "k_phase / k_phase_batch <..., FoldMode::kRingAll, ...> (phased fused ring all-reduce; "
                      "launches of several rounds take the batched kernel)",
              "hier": "k_phase<..., FoldMode::kHierAll, ...> (phased fused hierarchical all-reduce)"}[algo]
    traffic = load_traffic(args.workload)
    esz = np.dtype(W.STORAGE[dtype]).itemsize
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_TAG[dtype],
        "data": "synthetic",
        "config": {
            "workload": args.workload, "p": p, "n_per_rank": n, "shape_per_rank": list(spec.get("shape", (n,))),
            "op": op, "algo": "ring_fused" if algo == "ring" else f"hier_fused_g{group}",
            "bytes_per_step": runner.bytes, "cold_cache_buffer_sets": nsets,
        },
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / runner.bytes, 5) if traffic else None,
            "kernel": kernel, "launch_ms": round(launch_ms, 6), "launch_ms_from": "timed region / launches",
            "launches_per_step": 1,
        },
        "wall_s_timed_region": round(wall, 4),
        "page_busbw_GiBps": round(busbw_gibps("all_reduce", p, n * esz, ms_step * 1e-3), 2),
    }
    if args.spread_steps > 0:
        out["per_launch"] = launch_spread(torch, runner, args.spread_steps, stream, cpm)
    if not args.no_ceilings:
        out["copy_ceilings"] = copy_ceilings(torch, rr, stream)
    if args.extra:
        extra(args, torch, rr, W, spec, host_x, stream, cpm, op, runner)
    del runner
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, host_x, op, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def workload_lines(args, torch, rr, W, stream, cpm, report):
    """Every workload other than the headline one, each with the collectives
    its configuration names: the int32 p = 4 all-reduce (launch latency per
    call), the 8 MiB fp32 all-reduce, the hierarchical bf16 all-reduce and the
    gradient bucket's all-reduce (sum, max, min), reduce-scatter, all-gather,
    the reduce-scatter -> all-gather pair, and broadcast."""
    import numpy as np

    for name in ("ar_int32_p4_n4096", "ar_fp32_p8_8MiB", "hier_bf16_p8g4_8MiB", "zero_bucket_fp32_p8"):
        if name == args.workload:
            continue
        spec = W.WORKLOADS[name]
        x = W.make_inputs(name)
        p, n, dtype = spec["p"], spec["n"], spec["dtype"]
        esz = np.dtype(W.STORAGE[dtype]).itemsize
        algo = "hier" if spec["algo"] == "hier" else "ring"
        sets = 1 + math.ceil(COLD_BYTES / (2 * p * n * esz))
        for op in spec["ops"]:
            r = Runner(rr, torch, spec, "all_reduce", op, algo, spec.get("group", 0), x, sets, stream)
            report(f"all_reduce_{algo}_{op}", r, 200 if n * esz <= (8 << 20) else 40, True, name)
            if n * esz * p <= (1 << 20):
                # a launch-bound call: also with one buffer set, as a training
                # loop that reuses its buffers calls it (caches and address
                # translations warm), and its host cost per call
                del r
                r = Runner(rr, torch, spec, "all_reduce", op, algo, spec.get("group", 0), x, 1, stream)
                report(f"all_reduce_{algo}_{op}_cache_hot", r, 200, False, name)
                call_latency(torch, r, stream, name)
            del r
            torch.cuda.empty_cache()
        if spec["coll"] == "rs_ag":
            for coll in ("reduce_scatter", "all_gather", "broadcast"):
                fp = {"reduce_scatter": (p + 1) * n * esz, "all_gather": (p + 1) * n * esz,
                      "broadcast": (2 * p) * n * esz}[coll]
                r = Runner(rr, torch, spec, coll, "sum", "ring", 0, x, 1 + math.ceil(COLD_BYTES / fp), stream)
                report(coll, r, 40, True, name)
                del r
                torch.cuda.empty_cache()
            r = PairRunner(rr, torch, spec, x, 2, stream)
            report("reduce_scatter_then_all_gather", r, 40, True, name)
            del r
            torch.cuda.empty_cache()
        del x


def call_latency(torch, runner, stream, name, calls=2000):
    """A launch-bound call: the host time of one librr call (validation, plan
    and launch, through ctypes) over `calls` back-to-back calls, and the GPU
    time per launch from events around 200 launches queued behind a spin."""
    for i in range(20):
        runner.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(calls):
        runner.step(i)
    host_us = (time.perf_counter() - t0) / calls * 1e6
    torch.cuda.synchronize()
    spread = launch_spread(torch, runner, 200, stream, spin_cycles_per_ms(torch, stream))
    print(json.dumps({"extra": "call_latency", "workload": name, "host_us_per_call": round(host_us, 3),
                      "gpu_us_per_launch_median": round(spread["median_ms"] * 1e3, 3),
                      "gpu_us_per_launch_min": round(spread["min_ms"] * 1e3, 3)}), file=sys.stderr, flush=True)


class PairRunner:
    """Reduce-scatter then all-gather of its shards, one step each pair; the
    bytes counted are the all-reduce's 2pns (the pair moves (p+1)ns twice)."""

    def __init__(self, rr, torch, spec, host_x, nsets, stream):
        p, n = spec["p"], spec["n"]
        self.L = rr.lib()
        dt = rr.DTYPES[spec["dtype"]]
        sh = stream.cuda_stream
        self.sets = []
        for _ in range(nsets):
            x = torch.from_numpy(host_x).to("cuda")
            s = torch.empty((p, n // p), dtype=x.dtype, device="cuda")
            y = torch.empty_like(x)
            a = rr._ptr_array([x[r].data_ptr() for r in range(p)])
            b = rr._ptr_array([s[r].data_ptr() for r in range(p)])
            c = rr._ptr_array([y[r].data_ptr() for r in range(p)])
            self.sets.append((x, s, y, a, b, c,
                              lambda a=a, b=b, c=c: (self.L.rr_reduce_scatter(a, b, p, n, dt, 0, sh) or
                                                     self.L.rr_all_gather(b, c, p, n, dt, sh))))
        self.bytes = 2 * p * n * host_x.dtype.itemsize

    def step(self, i):
        if self.sets[i % len(self.sets)][-1]() != 0:
            raise RuntimeError(f"librr call failed: {self.L.rr_last_error().decode()}")


def extra(args, torch, rr, W, spec, host_x, stream, cpm, op, main_runner):
    import numpy as np

    def report(tag, runner, steps, cold, workload=None):
        ms, _, _ = timed(torch, runner, steps, 5, stream, cpm, per_launch=False)
        print(json.dumps({"extra": tag, "workload": workload or args.workload, "cold_cache": cold,
                          "GBps": round(runner.bytes / ms / 1e6, 2), "ms_per_step": round(ms, 6),
                          "us_per_call": round(ms * 1e3, 3),
                          "frac_of_peak": round(runner.bytes / ms / 1e6 / HBM_PEAK_GBPS, 4)}),
              file=sys.stderr, flush=True)

    # cache-hot figure of the main collective: one buffer set, back to back
    hot = Runner(rr, torch, spec, "all_reduce", op, main_runner.algo, spec.get("group", 0), host_x, 1, stream)
    report(f"all_reduce_{main_runner.algo}_cache_hot", hot, args.steps, False)
    del hot
    main_runner.sets.clear()
    torch.cuda.empty_cache()
    workload_lines(args, torch, rr, W, stream, cpm, report)
    # the other collectives, algorithms and layouts on the 8 MiB fp32 workload
    args.workload = "ar_fp32_p8_8MiB"
    spec = W.WORKLOADS[args.workload]
    host_x = W.make_inputs(args.workload)
    op = "sum"
    p, n, dtype = spec["p"], spec["n"], spec["dtype"]
    esz = np.dtype(W.STORAGE[dtype]).itemsize
    nsets = 1 + math.ceil(COLD_BYTES / (2 * p * n * esz))
    main_algo = "ring"
    for coll in ("reduce_scatter", "all_gather", "reduce", "broadcast"):
        fp = {"reduce_scatter": (p + 1) * n * esz, "all_gather": (p + 1) * n * esz, "reduce": (p + 1) * n * esz,
              "broadcast": (2 * p) * n * esz}[coll]
        k = 1 + math.ceil(COLD_BYTES / fp)
        r = Runner(rr, torch, spec, coll, op, "ring", 0, host_x, k, stream)
        report(coll, r, max(10, args.steps // 2), True)
        del r
        torch.cuda.empty_cache()
    for algo, G in (("ring_staged", 0), ("ring_persistent", 0), ("hier", 4), ("hier_staged", 4)):
        if p % max(G, 1):
            continue
        r = Runner(rr, torch, spec, "all_reduce", op, algo, G, host_x, nsets, stream)
        report(f"all_reduce_{algo}" + (f"_g{G}" if G else ""), r, max(10, args.steps // 4), True)
        del r
        torch.cuda.empty_cache()
    # AVG over the same buffers (the DDP gradient average)
    if dtype != "int32":
        r = Runner(rr, torch, spec, "all_reduce", "avg", main_algo, spec.get("group", 0), host_x, nsets,
                   stream)
        report(f"all_reduce_{main_algo}_avg", r, max(10, args.steps // 2), True)
        del r
        torch.cuda.empty_cache()
    # scatter and gather of the rank-sized buffer
    for coll in ("scatter", "gather"):
        k = 1 + math.ceil(COLD_BYTES / (2 * n * esz))
        r = Runner(rr, torch, spec, coll, op, "ring", 0, host_x, k, stream)
        report(coll, r, max(10, args.steps // 2), True)
        del r
        torch.cuda.empty_cache()
    # float16 all-reduce of the same byte size per rank
    if esz == 4:
        spec16 = dict(spec, dtype="float16", n=2 * n)
        x16 = W.random_inputs(7, p, 2 * n, "float16")
        r = Runner(rr, torch, spec16, "all_reduce", "sum", "ring", 0, x16, nsets, stream)
        report("all_reduce_ring_float16", r, max(10, args.steps // 2), True, f"{args.workload} as float16")
        del r, x16
        torch.cuda.empty_cache()
    # hierarchical variants on the hierarchy's workload
    hspec = W.WORKLOADS["hier_bf16_p8g4_8MiB"]
    hx = W.make_inputs("hier_bf16_p8g4_8MiB")
    hsets = 1 + math.ceil(COLD_BYTES / (2 * hspec["p"] * hspec["n"] * 2))
    for tag, kw in (("hier_default", {}), ("hier_intra_ring", dict(intra="ring")),
                    ("hier_wire_round", dict(wire_round=True)),
                    ("hier_intra_ring_wire_round", dict(intra="ring", wire_round=True))):
        r = Runner(rr, torch, hspec, "all_reduce_hier", "sum", "hier", hspec["group"], hx, hsets, stream, hier_kw=kw)
        report(f"all_reduce_{tag}", r, max(10, args.steps // 2), True, "hier_bf16_p8g4_8MiB")
        del r
        torch.cuda.empty_cache()
    del hx
    # bucketed all-reduce of one transformer block's gradients
    br = BucketRunner(rr, torch, W, "gpt2_block_fp32_p8", "avg", 1 + math.ceil(COLD_BYTES / (2 * 8 * 7087872 * 4)),
                      stream)
    report("all_reduce_bucket_avg", br, max(10, args.steps // 2), True, "gpt2_block_fp32_p8")
    del br
    torch.cuda.empty_cache()
    # tensor-parallel layouts at the row-parallel shape (8, 2048, 4096) bf16 per rank
    tspec = dict(W.WORKLOADS["tp_rowparallel_bf16_p8"], rows=8 * 2048)
    tx = W.make_inputs("tp_rowparallel_bf16_p8")
    tsets = 1 + math.ceil(COLD_BYTES / ((tspec["p"] + 1) * tspec["n"] * 2))
    for coll in ("reduce_scatter_dim1", "all_gather_dim1"):
        r = Runner(rr, torch, tspec, coll, "sum", "ring", 0, tx, tsets, stream)
        report(coll, r, max(10, args.steps // 4), True, "tp_rowparallel_bf16_p8")
        del r
        torch.cuda.empty_cache()
    del tx


if __name__ == "__main__":
    sys.exit(main())
