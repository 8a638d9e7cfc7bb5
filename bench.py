#!/usr/bin/env python3
"""Throughput of the LSA memory-indexer selection path on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs
already resident in HBM: project (memory-indexer and native queries), score +
select, OR-union + compact, native top-k inside the subset, and gather of the
union rows. The default workload is three indexer layers x 8 sequences x
125,000 compressed entries (bf16 keys, d_h = 128, n_h = 64). That is the
N = 125K configuration whose key stream (768 MB) does not fit in the 256 MB
Infinity Cache.

Output: one JSON line. `value` is entries scored+selected per second over the
whole step (sum over layers and sequences of N_b, divided by the step time).
Whole steps are timed as Pipeline.run() calls, which launch the gather on a
second stream so that it overlaps both top-k stages. `ms_per_step_graph` is
the same step replayed from a HIP graph, and `ms_per_step_sequential` the five
calls one after another on one stream (with the per-stage events).
`roofline` describes the dominant kernel (score_select), from HIP events on
its stream. `cpu_baseline` is the CPU oracle on a bounded sample of the same
workload.

`golden_labels` reports the label-mining step (lsa_golden_labels) on its own
workload, one lookahead window of 64 tokens x 21 layers x 125K entries: the
window time from HIP events on its stream, the rate against the bytes it must
move (the logits once, the masks written once) and HBM peak, and the oracle's
rate on a few of the window's tokens. `--golden-only` runs just that part.

`train_step` reports one training step of an indexer layer (lsa_train_step)
on 8 sequences x 125K entries with d = 4096, r = 2048: the step time from HIP
events, the rate against the bytes the step must move, and the oracle's rate
on a few of the sequences. `--train-only` runs just that part.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_select_traffic_{}.txt")  # per workload
# what the score_select kernel is built from: a change to any of these invalidates the measured traffic
SCORE_SOURCES = ["csrc/score.hip", "csrc/score_stream.hip", "csrc/cursor.hpp", "csrc/scorer.hpp", "csrc/common.hpp",
                 "csrc/kernels.hpp", "build.py"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def score_source_hash() -> str:
    h = hashlib.sha256()
    for s in SCORE_SOURCES:
        with open(os.path.join(ROOT, "sparse_kv_retrieval_amd", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per score_select launch from the committed PMC summary, if it was taken on these sources."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", " ", "|", "`")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != score_source_hash() or kv.get("workload") != workload:
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_kv_traffic(path: str, workload: str, source_hash: str):
    """traffic_bytes_per_launch from a committed summary, or None when it is missing or stale."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", " ", "|", "`")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") == source_hash and kv.get("workload") == workload:
        return int(kv["traffic_bytes_per_launch"])
    return None


def algorithmic_bytes(w, lengths) -> dict:
    """Bytes the score+select pass must move: every key once, its fp8 scale, one mask bit, plus q and w once per (b, l)."""
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[w.key_dtype]
    per_entry = w.d_h * esz + (4 if w.key_dtype == "fp8" else 0)
    n = int(np.sum(lengths))
    words = int(np.sum((lengths + 63) // 64))
    qw = w.B * (w.n_h * w.d_h + w.n_h) * 4
    total = w.L * (n * per_entry + words * 8 + qw)
    return {"per_entry_bytes": per_entry + 0.125, "bytes_per_launch": total, "entries_per_launch": w.L * n}


PEAK_BF16_FLOPS = 2.5e15  # MI355X dense bf16 matrix cores, published peak


def spread(v) -> dict:
    """Median, p10, p90 and mean of a list of durations."""
    a = np.asarray(v, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(a.mean()), "n": int(a.size)}


def project_rates(w, seconds: float) -> dict:
    """The projection stage (memory-indexer and native queries, 2L layer projections): its weight
    stream against HBM peak, and its matrix-core work against the dense bf16 peak. The work of one
    layer projection is 2 B (d r + r n_h d_h + d n_h) flops; the up-projection's c enters the matrix
    cores as hi + lo, which issues its part twice."""
    proj = 2 * w.L
    wbytes = proj * (w.r * w.d + w.n_h * w.d_h * w.r + w.n_h * w.d) * 2
    flops = proj * 2 * w.B * (w.d * w.r + w.r * w.n_h * w.d_h + w.d * w.n_h)
    issued = proj * 2 * w.B * (w.d * w.r + 2 * w.r * w.n_h * w.d_h + w.d * w.n_h)
    return {"us": seconds * 1e6, "weight_bytes": wbytes, "hbm_GBs": wbytes / seconds / 1e9,
            "hbm_frac": wbytes / seconds / 1e9 / PEAK_HBM_GBS, "flops": flops,
            "mfma_util": flops / seconds / PEAK_BF16_FLOPS, "mfma_util_issued": issued / seconds / PEAK_BF16_FLOPS,
            "note": "B rows per projection: a weight stream, bound by HBM; the matrix-core fraction is small by "
                    "construction"}


def host_facts() -> dict:
    """The host the CPU baselines run on: CPU model, logical CPUs, CPUs this process may use, BLAS threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "blas_threads": int(blas)}


class CpuClock:
    """Wall time and the process's CPU time over a region: cpu / wall is the number of cores it kept busy."""

    def __enter__(self):
        self.t0, self.c0 = time.perf_counter(), os.times()
        return self

    def __exit__(self, *exc):
        c1 = os.times()
        self.wall = time.perf_counter() - self.t0
        self.cpu = (c1.user - self.c0.user) + (c1.system - self.c0.system)
        return False

    @property
    def cores(self) -> int:
        return max(1, int(round(self.cpu / max(self.wall, 1e-9))))


def cpu_baseline(inp, budget_s: float):
    """The CPU oracle as it stands, timed over whole sequences of the same workload until about `budget_s`."""
    from oracle import lsa_oracle as O
    w = inp.workload
    done_entries = 0
    seqs = 0
    # whole sequences, in order, repeating the workload until the budget is spent
    with CpuClock() as clk:
        while time.perf_counter() - clk.t0 < budget_s:
            b = seqs % w.B
            O.run_path(inp, sequences=[b])
            done_entries += int(inp.lengths[b]) * w.L
            seqs += 1
    el = clk.wall
    return {"value": done_entries / el, "unit": "entries/s", "cores": clk.cores, "kind": "oracle",
            "sample": f"{seqs} sequence passes ({seqs / w.B:.2f} x the {w.B} sequences) x {w.L} layers of the "
                      f"{w.name} workload, full path (project, score, select, union, compact, top-k, gather), "
                      f"{el:.1f} s",
            "cpu_seconds": clk.cpu, "host": host_facts()}


def single_scan(steps: int, copies: int = 16) -> dict:
    """score_select on one 125,000-entry sequence of one layer (single_layer_500k: 32 MB of keys),
    timed per launch with HIP events: with the same keys every launch (they stay in the 256 MB
    Infinity Cache), and rotating over `copies` copies of the keys (512 MB), so that every launch
    reads its keys from HBM."""
    import torch
    from sparse_kv_retrieval_amd import lsa
    from sparse_kv_retrieval_amd import synth
    from sparse_kv_retrieval_amd.pipeline import DeviceEvent, Pipeline
    w = synth.WORKLOADS["single_layer_500k"]
    log(f"[bench] single scan: generating {w.name}")
    inp = synth.make(w, with_pool=False)
    p = Pipeline(inp, "cuda:0")
    p.run()
    keys = [p.keys[0]] + [p.keys[0].clone() for _ in range(copies - 1)]
    stream = torch.cuda.current_stream()

    def call(i):
        layers = [dict(q=p.q[0], w=p.g[0], keys=keys[i % copies], key_scale=p.scale[0], mask_out=p.masks[0])]
        lsa.score_select(layers, B=w.B, key_offsets=p.key_off, key_offsets_host=p.key_off_h,
                         mask_word_offsets=p.mwo, mask_word_offsets_host=p.mwo_h, n_h=w.n_h, d_h=w.d_h,
                         key_dtype=w.key_dtype, threshold=w.threshold, stream=stream)

    ab = algorithmic_bytes(w, inp.lengths)
    out = {"workload": w.name, "entries": int(np.sum(inp.lengths)), "bytes_per_launch": ab["bytes_per_launch"],
           "copies_rotated": copies}
    for tag, rot in (("same_keys", False), ("rotated_keys", True)):
        for i in range(3):
            call(i if rot else 0)
        torch.cuda.synchronize()
        us = []
        for i in range(max(steps, 10)):
            e0, e1 = DeviceEvent(timing=True), DeviceEvent(timing=True)
            e0.record(stream)
            call(i + 3 if rot else 0)
            e1.record(stream)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3)
        med = float(np.median(us))
        gbs = ab["bytes_per_launch"] / (med * 1e-6) / 1e9
        out[tag] = {"launch_us": spread(us), "GB_per_s": gbs, "frac": gbs / PEAK_HBM_GBS,
                    "entries_per_s": out["entries"] / (med * 1e-6)}
    del keys, p
    torch.cuda.empty_cache()
    return out


GOLDEN_WORKLOAD = "golden_t64_l21_n125k"
GOLDEN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "golden_segment_traffic_{}.txt")
GOLDEN_SOURCES = ["csrc/golden.hip", "csrc/common.hpp", "csrc/kernels.hpp", "build.py"]


def golden_source_hash() -> str:
    h = hashlib.sha256()
    for s in GOLDEN_SOURCES:
        with open(os.path.join(ROOT, "sparse_kv_retrieval_amd", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def golden_cpu_baseline(inp, budget_s: float) -> dict:
    """The golden-label oracle as it stands, over whole tokens of the window (all layers) until about budget_s."""
    from oracle import golden_oracle as G
    w = inp.workload
    toks = 0
    entries = 0
    with CpuClock() as clk:
        while time.perf_counter() - clk.t0 < budget_s and toks < w.T:
            n = int(inp.n_valid[toks])
            G.votes(inp.logits[toks], n, w.p)
            entries += n * w.L
            toks += 1
    el = clk.wall
    return {"value": entries / el, "unit": "entries/s", "cores": clk.cores, "kind": "oracle",
            "sample": f"{toks} of the {w.T} tokens x {w.L} layers (softmax, nucleus, vote per token), {el:.1f} s",
            "cpu_seconds": clk.cpu}


def golden_measure(steps: int, warmup: int, cpu_budget: float | None) -> dict:
    """Golden-label mining for one lookahead window (lsa_golden_labels), timed with HIP events on its stream."""
    import torch
    from sparse_kv_retrieval_amd import lsa
    from sparse_kv_retrieval_amd import synth_golden as SG
    from sparse_kv_retrieval_amd.pipeline import DeviceEvent
    w = SG.WORKLOADS[GOLDEN_WORKLOAD]
    log(f"[bench] golden labels: generating {w.name}")
    inp = SG.make(w)
    dev = torch.device("cuda")
    logits = torch.from_numpy(inp.logits).to(dev)
    nv = torch.from_numpy(inp.n_valid).to(dev)
    rows, W = w.T * w.L, w.words
    row_mask = torch.empty((rows, W), dtype=torch.int64, device=dev)
    sizes = torch.empty(rows, dtype=torch.int32, device=dev)
    golden = torch.empty(W, dtype=torch.int64, device=dev)
    ws = torch.empty(lsa.golden_workspace_size(w.T, w.L, w.row_stride), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        lsa.golden_labels(logits, row_stride=w.row_stride, T=w.T, L=w.L, n_valid=nv, top_p=w.p, theta=w.theta,
                          row_mask=row_mask, golden=golden, nucleus_size=sizes, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = DeviceEvent(timing=True), DeviceEvent(timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    entries = int(inp.n_valid.astype(np.int64).sum()) * w.L
    # logits read once; row masks, nucleus sizes and the window's label set written once
    alg = entries * 4 + rows * W * 8 + rows * 4 + W * 8
    label = int(np.unpackbits(golden.cpu().numpy().view(np.uint8)).sum())
    sz = sizes.cpu().numpy()
    achieved = alg / (ms * 1e-3) / 1e9
    out = {"workload": w.name, "T": w.T, "L": w.L, "entries_per_row": int(inp.n_valid.max()), "top_p": w.p,
           "theta": w.theta, "us_per_window": ms * 1e3, "entries_per_s": entries / (ms * 1e-3),
           "algorithmic_bytes": alg, "achieved_GBs": achieved, "peak_GBs": PEAK_HBM_GBS,
           "frac": achieved / PEAK_HBM_GBS, "label_set": label,
           "nucleus_size": {"min": int(sz.min()), "mean": float(sz.mean()), "max": int(sz.max())},
           "what": "lsa_golden_labels over one window: every (token, layer) row's top-p nucleus, the layer vote "
                   "per token and the union over the window (four kernels; logits read once)"}
    traffic = read_kv_traffic(GOLDEN_TRAFFIC_FILE.format(w.name), w.name, golden_source_hash())
    out["segment_kernel_traffic"] = traffic
    if cpu_budget:
        log("[bench] golden labels: cpu baseline")
        out["cpu_baseline"] = golden_cpu_baseline(inp, cpu_budget)
    del logits, row_mask, ws
    torch.cuda.empty_cache()
    return out


TRAIN_WORKLOAD = "train_b8"
TRAIN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "train_scan_traffic_{}.txt")
TRAIN_SOURCES = ["csrc/train.hip", "csrc/common.hpp", "csrc/kernels.hpp", "build.py"]


def train_source_hash() -> str:
    h = hashlib.sha256()
    for s in TRAIN_SOURCES:
        with open(os.path.join(ROOT, "sparse_kv_retrieval_amd", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def train_bytes(w, entries: int) -> dict:
    """Bytes one training step must move: the keys and labels once; h and the three weight matrices for
    the projections, W^IUQ a second time for dc = dq W^IUQ (dq exists only after the key scan); the three
    gradients written once."""
    d, r, m, nh = w.d, w.r, w.n_h * w.d_h, w.n_h
    keys = entries * w.d_h * 2 + entries // 8
    weights = w.B * d * 2 + r * d * 2 + 2 * m * r * 2 + nh * d * 2
    grads = (r * d + m * r + nh * d) * 4
    return {"keys_and_labels": keys, "activations_and_weights": weights, "gradients": grads,
            "total": keys + weights + grads}


def train_measure(steps: int, warmup: int, cpu_budget: float | None) -> dict:
    """One indexer-layer training step (lsa_train_step) on its own workload, timed with HIP events."""
    import torch
    from sparse_kv_retrieval_amd import lsa
    from sparse_kv_retrieval_amd import synth
    from sparse_kv_retrieval_amd.pipeline import DeviceEvent
    w = synth.WORKLOADS[TRAIN_WORKLOAD]
    log(f"[bench] training step: generating {w.name}")
    inp = synth.make(w, with_pool=False)
    lab, words = synth.train_labels(inp, 0, 0.02)
    dev = torch.device("cuda")

    def u16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    mw = inp.mem_w[0]
    args = dict(h=u16(inp.h[0]), w_dq=u16(mw.w_dq), w_iuq=u16(mw.w_iuq), w_w=u16(mw.w_w), keys=u16(inp.keys[0]),
                key_offsets=torch.from_numpy(inp.key_offsets).to(dev), key_offsets_host=inp.key_offsets,
                labels=torch.from_numpy(words.view(np.int64)).to(dev),
                mask_word_offsets=torch.from_numpy(inp.mask_word_offsets).to(dev),
                mask_word_offsets_host=inp.mask_word_offsets, B=w.B, d=w.d, r=w.r, n_h=w.n_h, d_h=w.d_h,
                gamma=2.0, alpha=0.25, loss=torch.empty(1, dtype=torch.float32, device=dev),
                g_dq=torch.empty((w.r, w.d), dtype=torch.float32, device=dev),
                g_iuq=torch.empty((w.n_h * w.d_h, w.r), dtype=torch.float32, device=dev),
                g_w=torch.empty((w.n_h, w.d), dtype=torch.float32, device=dev),
                workspace=torch.empty(lsa.train_workspace_size(w.B, inp.key_offsets, w.r), dtype=torch.uint8,
                                      device=dev))
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        lsa.train_step(**args, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = DeviceEvent(timing=True), DeviceEvent(timing=True)
    e0.record(stream)
    for _ in range(steps):
        lsa.train_step(**args, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    entries = int(inp.key_offsets[-1])
    tb = train_bytes(w, entries)
    achieved = tb["total"] / (ms * 1e-3) / 1e9
    scan_bytes = entries * w.d_h * 2 + entries // 8  # the scan kernel: keys and labels once
    out = {"workload": w.name, "B": w.B, "N_per_seq": int(inp.lengths.max()), "d": w.d, "r": w.r, "n_h": w.n_h,
           "d_h": w.d_h, "gamma": 2.0, "alpha": 0.25, "us_per_step": ms * 1e3, "entries_per_s": entries / (ms * 1e-3),
           "loss": float(args["loss"].item()), "algorithmic_bytes": tb, "achieved_GBs": achieved,
           "peak_GBs": PEAK_HBM_GBS, "frac": achieved / PEAK_HBM_GBS,
           "what": "lsa_train_step: projections, one fused MFMA pass over the frozen keys (scores, focal loss, "
                   "dq and dw), the gradient reduction and the three rank-B gradient products",
           "scan_kernel": {"algorithmic_bytes": scan_bytes,
                           "traffic": read_kv_traffic(TRAIN_TRAFFIC_FILE.format(w.name), w.name, train_source_hash())}}
    if cpu_budget:
        log("[bench] training step: cpu baseline")
        from oracle import lsa_oracle as O
        from oracle import train_oracle as TO
        n_seq = 0
        H = O.decode_act(inp.h[0], "bf16")
        Ws = [O.decode_act(m, "bf16") for m in (mw.w_dq, mw.w_iuq, mw.w_w)]
        done = 0
        with CpuClock() as clk:
            while n_seq < w.B and time.perf_counter() - clk.t0 < cpu_budget:
                s0, s1 = int(inp.key_offsets[n_seq]), int(inp.key_offsets[n_seq + 1])
                TO.train_step(H[n_seq:n_seq + 1], *Ws, [O.decode_keys(inp.keys[0][s0:s1], "bf16")], [lab[s0:s1]],
                              w.n_h, w.d_h)
                done += s1 - s0
                n_seq += 1
        el = clk.wall
        out["cpu_baseline"] = {"value": done / el, "unit": "entries/s", "cores": clk.cores,
                               "kind": "oracle",
                               "sample": f"{n_seq} of the {w.B} sequences, each as a one-sequence step "
                                         f"(float64 numpy, decoding included), {el:.1f} s"}
    del args
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="three_layer_b8")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-host-fetch", action="store_true", help="skip the cold-pool (pinned host) fetch measurement")
    ap.add_argument("--no-golden", action="store_true", help="skip the golden-label mining measurement")
    ap.add_argument("--golden-only", action="store_true", help="only the golden-label mining measurement")
    ap.add_argument("--no-train", action="store_true", help="skip the training-step measurement")
    ap.add_argument("--no-single-scan", action="store_true",
                    help="skip the one-sequence scan (single_layer_500k, cache-resident and rotated keys)")
    ap.add_argument("--train-only", action="store_true", help="only the training-step measurement")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (each GPU would score its own "
              "sequences; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_kv_retrieval_amd import synth
    from sparse_kv_retrieval_amd.pipeline import DeviceEvent, Pipeline

    if args.golden_only:
        g = golden_measure(args.steps, args.warmup, None if args.no_cpu_baseline else 3.0)
        print(json.dumps({"golden_labels": g}), flush=True)
        return
    if args.train_only:
        t = train_measure(args.steps, args.warmup, None if args.no_cpu_baseline else 3.0)
        print(json.dumps({"train_step": t}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name}")
    t = time.perf_counter()
    inp = synth.make(w)
    log(f"[bench] generated in {time.perf_counter() - t:.1f}s; uploading")
    p = Pipeline(inp, "cuda:0", with_scores=False)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        p.run()
    torch.cuda.synchronize()

    # Per-stage launch durations: eager calls with HIP events between them, on the launch stream.
    names = ["project", "score_select", "union_compact", "topk", "gather"]
    ev = [[DeviceEvent(timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} eager steps (per stage)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record(stream)
        p.project(); e[1].record(stream)
        p.score_select(); e[2].record(stream)
        p.union_compact(); e[3].record(stream)
        p.topk(); e[4].record(stream)
        p.gather(); e[5].record(stream)
    torch.cuda.synchronize()
    ms_per_step_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_all = {n: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)] for i, n in enumerate(names)}
    stage_ms = {n: float(np.mean(v)) for n, v in stage_all.items()}

    # Whole steps: run() as an application calls it (the gather on a second stream,
    # overlapping the top-k stages), K steps between two synchronisations.
    for _ in range(args.warmup):
        p.run()
    log(f"[bench] timing {args.steps} whole steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        p.run()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # The same step captured once in a HIP graph and replayed (reported alongside).
    graph = p.capture()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_per_step_graph = (time.perf_counter() - t0) * 1e3 / args.steps

    def timed(fn, reps):
        """Per-launch durations (us) of fn() on the launch stream, HIP events around each launch."""
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        out_us = []
        for _ in range(reps):
            e0, e1 = DeviceEvent(timing=True), DeviceEvent(timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out_us.append(e0.elapsed_time(e1) * 1e3)
        return out_us

    # The score pass in its variants: the step's mask-only pass, mask + sigmoid scores (the full
    # pass), the hi-only first pass with per-tile completion, and the wave-pair kernel.
    log("[bench] score pass variants")
    p.scores = [torch.empty(max(p.rows, 1), dtype=torch.float32, device="cuda") for _ in range(w.L)]
    p.masks_scored = [torch.empty(max(p.words, 1), dtype=torch.int64, device="cuda") for _ in range(w.L)]
    variants = {"mask_only": lambda: p.score_select(),
                "mask_and_score": lambda: p.score_with_sigmoid()}
    if w.key_dtype != "f32":
        variants["mask_only_guard"] = lambda: p._score_call(p.masks, None, {"guard": 1}, None)
    variants["mask_only_pair_kernel"] = lambda: p._score_call(p.masks, None, {"kernel": "pairs"}, None)
    score_variants = {k_: spread(timed(f_, args.steps)) for k_, f_ in variants.items()}
    p.scores = p.masks_scored = None

    # Decode steps after the trigger: each layer's union rows of keys packed once, then per step the
    # native query of the step's hidden state and the top-k over the packed subset (lsa_topk_step).
    log("[bench] decode steps")
    p.alloc_steps()
    p.run()
    p.pack_subset_keys()
    hs = synth.step_hidden(inp, 4)
    p.set_step_hidden(hs[0])
    torch.cuda.synchronize()
    pack_us = timed(lambda: p.pack_subset_keys(), 5)
    step_us = timed(lambda: p.step(), args.steps)
    step_topk_us = timed(lambda: p.step_topk(), args.steps)
    union_rows = int(p.count.sum())
    kb = w.d_h * {"f32": 4, "bf16": 2, "fp8": 1}[w.key_dtype] + (4 if w.key_dtype == "fp8" else 0)
    step_bytes = w.L * union_rows * (kb + 4 + 4 + 4) + w.L * w.B * w.k * 8
    st_med = float(np.median(step_topk_us))
    decode_steps = {
        "what": "per decode step: the native query of the step's h (lsa_project_packed) and lsa_topk_step over "
                "each layer's union rows of keys, packed once per trigger (lsa_gather)",
        "subset_rows_per_layer": union_rows, "k": w.k,
        "us_per_step": spread(step_us), "topk_step_us": spread(step_topk_us),
        "pack_once_per_trigger_us": spread(pack_us),
        "us_per_window_of_64_steps": 64 * float(np.median(step_us)),
        "topk_step_bytes": step_bytes, "topk_step_GBs": step_bytes / (st_med * 1e-6) / 1e9,
        "note": "topk_step_bytes: the packed keys (and fp8 scales) once, the list index, the workspace score "
                "written and read, and the k outputs"}
    p.keys_sub = None
    torch.cuda.empty_cache()

    # The plain streaming read of the same number of bytes as the score pass: the achievable ceiling.
    from sparse_kv_retrieval_amd import profiling as PR
    log("[bench] streaming-read reference")
    ab0 = algorithmic_bytes(w, inp.lengths)
    stream_ref = PR.stream_read_rate(ab0["bytes_per_launch"], reps=args.steps)

    host_fetch = None
    if not args.no_host_fetch and inp.pool is not None:
        # The load step from the cold pool: the same union rows read from a pinned
        # host copy of the pool over the host link (lsa_fetch_host). Reported on
        # its own; it is not part of the step above.
        log("[bench] cold-pool fetch")
        a = np.ascontiguousarray(inp.pool)
        p.pool_host = torch.from_numpy(a.view(np.int16)).pin_memory()
        for _ in range(2):
            p.fetch_host()
        torch.cuda.synchronize()
        reps = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            p.fetch_host()
        e1.record(stream)
        torch.cuda.synchronize()
        fms = e0.elapsed_time(e1) / reps
        rows_f = int(min(int(p.count.sum()), p.gather_capacity))
        fbytes = rows_f * w.pool_dim * 2
        host_fetch = {"rows": rows_f, "bytes_read": fbytes, "ms": fms, "GB_per_s": fbytes / (fms * 1e-3) / 1e9,
                      "what": "union rows read from pinned host memory over the host link into HBM (lsa_fetch_host)"}
        p.pool_host = None

    counts = p.count.cpu().numpy()
    rows = int(inp.key_offsets[-1])
    entries = int(np.sum(inp.lengths)) * w.L
    ab = algorithmic_bytes(w, inp.lengths)
    score_s = stage_ms["score_select"] / 1e3
    achieved = ab["bytes_per_launch"] / score_s / 1e9

    traffic = read_traffic(w.name)

    out = {
        "metric": "compressed entries scored+selected/sec and HBM GB/s at N=125K (1 GPU)",
        "value": entries / (ms_per_step / 1e3),
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.key_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "N_per_seq": int(inp.lengths.max()) if w.N else "ragged",
                   "total_entries_per_layer": rows, "key_dtype": w.key_dtype, "n_h": w.n_h, "d_h": w.d_h,
                   "d": w.d, "r": w.r, "k": w.k, "threshold": w.threshold, "pool_row_bytes": w.pool_dim * 2},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "score_stream_kernel" if w.key_dtype in ("bf16", "fp8") else "score_select_kernel",
                     "bytes_per_launch": ab["bytes_per_launch"], "per_entry_bytes": ab["per_entry_bytes"],
                     "avg_launch_us": stage_ms["score_select"] * 1e3,
                     "launch_us": spread([v * 1e3 for v in stage_all["score_select"]]),
                     "stream_read_ceiling_GBs": stream_ref["GB_per_s"],
                     "frac_of_stream_read": achieved / stream_ref["GB_per_s"],
                     "stream_read": {k_: v_ for k_, v_ in stream_ref.items() if k_ != "sweep"}},
        "stages_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "stages_us_spread": {k: spread([x * 1e3 for x in v]) for k, v in stage_all.items()},
        "score_select_variants_us": score_variants,
        "project": project_rates(w, stage_ms["project"] * 1e-3),
        "decode_steps": decode_steps,
        "ms_per_step_sequential": ms_per_step_eager,
        "ms_per_step_graph": ms_per_step_graph,
        "selection": {"union_fraction": float(counts.sum()) / rows, "union_per_seq_mean": float(counts.mean())},
    }
    if host_fetch is not None:
        out["host_fetch"] = host_fetch
    if not args.no_single_scan and args.workload != "single_layer_500k":
        p = None
        torch.cuda.empty_cache()
        out["single_scan"] = single_scan(args.steps)
    if not args.no_golden:
        p = None
        torch.cuda.empty_cache()
        out["golden_labels"] = golden_measure(args.steps, args.warmup, None if args.no_cpu_baseline else 3.0)
    if not args.no_train:
        out["train_step"] = train_measure(args.steps, args.warmup, None if args.no_cpu_baseline else 3.0)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
