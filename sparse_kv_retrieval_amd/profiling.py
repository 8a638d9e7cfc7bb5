"""Helpers for the rocprofv3 evidence of the selection path.

Usage (each step's output is plain text, suitable for a short summary file):

  python -m sparse_kv_retrieval_amd.profiling copy --mib 1024 --reps 5
      Device-to-device copy of a known size, to calibrate the HBM byte
      counters: run it under `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE)
      and compare the counter with the bytes the copy must move.

  python -m sparse_kv_retrieval_amd.profiling stream --mib 768 --reps 10
      The plain streaming-read kernel (probe.hip, libprobe.so) over a buffer of
      that size: the achievable read rate that the score pass's key stream is
      compared with.

  python -m sparse_kv_retrieval_amd.profiling stats <dir>
      Per-kernel call count and average / min / max duration from a
      `rocprofv3 --kernel-trace --output-format csv` run (its
      *_kernel_trace.csv), as a markdown table.

  python -m sparse_kv_retrieval_amd.profiling pmc <dir> [--kernel REGEX]
      Average value per dispatch of every counter in a `rocprofv3 --pmc`
      run (its *_counter_collection.csv), per kernel.

  python -m sparse_kv_retrieval_amd.profiling traffic --fetch <dir> --write <dir>
      --copy-fetch <dir> --copy-write <dir> --copy-mib M --kernel REGEX
      HBM bytes per dispatch of one kernel: FETCH_SIZE and WRITE_SIZE (KiB
      per dispatch) divided by what the same counters read per byte for the
      plain copy of M MiB.

Nothing here launches the selection kernels; the copy uses torch, the stream
probe its own kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys
from collections import defaultdict


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(run_dir: str) -> list[dict]:
    """Per-kernel durations (ns) from a kernel-trace csv."""
    path = _one(os.path.join(run_dir, "**", "*kernel_trace.csv"))
    durs = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            durs[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = []
    for name, d in durs.items():
        out.append({"kernel": name, "calls": len(d), "avg_us": statistics.mean(d) / 1e3,
                    "min_us": min(d) / 1e3, "max_us": max(d) / 1e3, "total_us": sum(d) / 1e3})
    out.sort(key=lambda x: -x["total_us"])
    return out


def pmc_means(run_dir: str, kernel: str | None = None) -> dict:
    """{(kernel, counter): (median value per dispatch, dispatches)} from a counter-collection csv.

    The median, not the mean: a run may launch a few dispatches of the same kernel
    with other options (the bench's score-writing variant of the selection pass),
    and those must not shift the figure of the timed step's dispatches."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    vals = defaultdict(list)
    rx = re.compile(kernel) if kernel else None
    with open(path) as f:
        for r in csv.DictReader(f):
            if rx and not rx.search(r["Kernel_Name"]):
                continue
            vals[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return {k: (statistics.median(v), len(v)) for k, v in vals.items()}


def _counter(run_dir: str, kernel: str, counter: str) -> float:
    m = {k: v for k, v in pmc_means(run_dir, kernel).items() if k[1] == counter}
    if not m:
        raise KeyError(f"{counter} for /{kernel}/ not in {run_dir}")
    if len(m) > 1:
        raise KeyError(f"/{kernel}/ matches several kernels: {[k[0] for k in m]}")
    return next(iter(m.values()))[0]


def copy_run(mib: int, reps: int) -> None:
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}", flush=True)


PROBE_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libprobe.so")


def stream_read_rate(nbytes: int, reps: int = 10, copies: int = 2) -> dict:
    """Read rate of the plain streaming-read kernel (probe.hip) over `nbytes`, in GB/s.

    `copies` buffers of nbytes each are read in turn, so no launch finds its
    buffer in the 256 MB Infinity Cache when nbytes is large. The probe's
    access patterns (grid-stride or one contiguous range per block, plain or
    non-temporal loads), loads in flight per thread (8 or 16) and blocks per
    compute unit (2, 4, 8) are swept, plus the LDS-ring pattern of the key scan
    (one block of 8 waves per CU); the fastest configuration's median over
    `reps` launches (HIP events on the launch stream, as the kernels are timed) is the ceiling. The
    whole sweep is returned too."""
    import ctypes

    import torch

    from .pipeline import DeviceEvent
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_void_p]
    nbytes = (int(nbytes) + 15) // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    for b in bufs:
        b.fill_(3)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(8 * cus, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    sweep = []
    # (mode, loads in flight, blocks per CU); the LDS-ring mode runs one block of 8 waves per CU
    configs = [(m, u, bpc) for m in (0, 1, 2) for u in (8, 16) for bpc in (2, 4, 8)] + [(3, 8, 1)]
    for mode, u, bpc in configs:
        blocks = bpc * cus

        def launch(i):
            r = fn(bufs[i % copies].data_ptr(), nbytes, sink.data_ptr(), blocks, mode, u,
                   ctypes.c_void_p(st.cuda_stream))
            assert r == 0, r
        for i in range(3):
            launch(i)
        torch.cuda.synchronize()
        us = []
        for i in range(reps):
            e0, e1 = DeviceEvent(timing=True), DeviceEvent(timing=True)
            e0.record(st)
            launch(i)
            e1.record(st)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3)
        us.sort()
        sweep.append({"mode": ["grid_stride", "block_range", "block_range_nt", "lds_ring_nt"][mode],
                      "loads_in_flight": u if mode < 3 else 16,  # the ring: 4 slots x 4 loads per wave
                      "blocks_per_cu": bpc, "median_us": us[len(us) // 2], "min_us": us[0],
                      "GB_per_s": nbytes / (us[len(us) // 2] * 1e-6) / 1e9})
    del bufs
    torch.cuda.empty_cache()
    best = max(sweep, key=lambda r: r["GB_per_s"])
    return {"bytes": nbytes, "GB_per_s": best["GB_per_s"], "median_us": best["median_us"], "best": best,
            "sweep": sweep}


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m sparse_kv_retrieval_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    p = sub.add_parser("pmc")
    p.add_argument("dir")
    p.add_argument("--kernel")
    r = sub.add_parser("stream")
    r.add_argument("--mib", type=int, default=768)
    r.add_argument("--reps", type=int, default=10)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "kernel"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    a = ap.parse_args(argv)

    if a.cmd == "copy":
        copy_run(a.mib, a.reps)
    elif a.cmd == "stream":
        r_ = stream_read_rate(a.mib << 20, a.reps)
        print(f"streaming read of {a.mib} MiB ({r_['bytes']} bytes), median of {a.reps} launches per configuration")
        print("| pattern | loads in flight per thread | blocks per CU | median us | GB/s |")
        print("|---|---:|---:|---:|---:|")
        for c in r_["sweep"]:
            print(f"| {c['mode']} | {c['loads_in_flight']} | {c['blocks_per_cu']} | {c['median_us']:.1f} | "
                  f"{c['GB_per_s']:.0f} |")
        b_ = r_["best"]
        print(f"ceiling: {r_['GB_per_s']:.0f} GB/s ({b_['mode']}, {b_['loads_in_flight']} loads, "
              f"{b_['blocks_per_cu']} blocks per CU)", flush=True)
    elif a.cmd == "stats":
        print("| kernel | calls | avg us | min us | max us |")
        print("|---|---:|---:|---:|---:|")
        for r in kernel_stats(a.dir):
            print(f"| `{r['kernel'][:90]}` | {r['calls']} | {r['avg_us']:.1f} | {r['min_us']:.1f} | {r['max_us']:.1f} |")
    elif a.cmd == "pmc":
        for (k, ctr), (v, n) in sorted(pmc_means(a.dir, a.kernel).items()):
            print(f"{k[:90]}\t{ctr}\t{v:.1f}\t(n={n})")
    else:
        copy_bytes = a.copy_mib << 20
        cf = _counter(a.copy_fetch, r"copyBuffer", "FETCH_SIZE") * 1024 / copy_bytes
        cw = _counter(a.copy_write, r"copyBuffer", "WRITE_SIZE") * 1024 / copy_bytes
        kf = _counter(a.fetch, a.kernel, "FETCH_SIZE") * 1024
        kw = _counter(a.write, a.kernel, "WRITE_SIZE") * 1024
        print(f"copy calibration: FETCH_SIZE reads {cf:.4f} x the copied bytes, WRITE_SIZE {cw:.4f} x")
        print(f"kernel /{a.kernel}/: FETCH_SIZE {kf / 1e6:.2f} MB, WRITE_SIZE {kw / 1e6:.2f} MB per dispatch (raw, median)")
        print(f"traffic_bytes_per_launch: {kf / cf + kw / cw:.0f}")
        print(f"fetch_bytes_per_launch: {kf / cf:.0f}")
        print(f"write_bytes_per_launch: {kw / cw:.0f}")


if __name__ == "__main__":
    main(sys.argv[1:])
