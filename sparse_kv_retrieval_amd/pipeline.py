"""Device-resident buffers for one workload, and one pass of the whole path.

`Pipeline(inputs)` copies a seeded input set (from `synth.make`) into HBM and
allocates every output and the top-k workspace once. `run()` then enqueues the
five library calls, with no allocation and no host synchronisation, on the
current stream (the load step on a second stream that forks after the union
and joins at the end):

  lsa_project        memory-indexer and native query/gates for every layer (one call, 2L layers);
                     with bf16 weights, lsa_project_packed on weights packed once at set-up
  lsa_score_select   masks for every (layer, sequence) (score_with_sigmoid: a pass that also
                     writes the sigmoid scores)
  lsa_union_compact  OR over the layers -> ascending index list + count per sequence
  lsa_topk           native top-k inside the union, per (layer, sequence)
                     (run() calls its two stages, lsa_topk_score and lsa_topk_select)
  lsa_gather         the union rows of the compressed-KV pool -> packed compact buffer
                     (with host_pool=True, lsa_fetch_host reads them from a copy of the
                     pool in pinned host memory instead: the cold pool)

After a trigger, alloc_steps() / pack_subset_keys() / step() run the decode steps: each
layer's union rows of keys are packed once (lsa_gather), and every step projects its own
native query and calls lsa_topk_step over them.

This module only wires buffers. All arithmetic happens in the HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import torch

from . import lsa


class DeviceEvent:
    """A HIP event for ordering or timing work on the streams of one device, with no
    system-scope fence when it is recorded or waited on. The fork and join of run() need only
    device-scope ordering (host visibility comes from the caller's own synchronisation), and a
    default event's system-scope fence left the GPU idle for several microseconds at each fork
    and join. As a timing event (timing=True) it adds less to the interval it brackets than a
    default event, for the same reason. The runtime is the one the library is linked against,
    already loaded."""

    _DISABLE_TIMING = 0x2
    _DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    def __init__(self, timing: bool = False):
        if DeviceEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            DeviceEvent._hip = hip
        self._h = ctypes.c_void_p()
        flags = self._DISABLE_SYSTEM_FENCE | (0 if timing else self._DISABLE_TIMING)
        self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(self._h), flags), "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, stream):
        self._check(self._hip.hipEventRecord(self._h, ctypes.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def wait(self, stream):
        """Make `stream` wait for the work before this event's last record."""
        self._check(self._hip.hipStreamWaitEvent(ctypes.c_void_p(stream.cuda_stream), self._h, 0),
                    "hipStreamWaitEvent")

    def elapsed_time(self, end: "DeviceEvent") -> float:
        """Milliseconds from this event to `end` (both recorded with timing=True and complete)."""
        ms = ctypes.c_float()
        self._check(self._hip.hipEventElapsedTime(ctypes.byref(ms), self._h, end._h), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        # at interpreter exit the runtime may already be torn down; the process frees the event
        if self._hip is not None and self._h and not sys.is_finalizing():
            self._hip.hipEventDestroy(self._h)


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint64:
        a = a.view(np.int64)
    return torch.from_numpy(a).to(device)


GUARD_BYTES = 4096
CANARY = 0x5A


class Pipeline:
    def __init__(self, inp, device="cuda", *, with_scores=False, with_topk_scores=True, gather_capacity=None,
                 guard=False, packed=True, overlap=True, host_pool=False, early_fork=True):
        w = inp.workload
        self.w = w
        self.inp = inp
        dev = torch.device(device)
        self.device = dev
        self._guarded = []
        self.guard = guard
        self.overlap = overlap
        self.early_fork = early_fork  # fork the load step before the top-k scoring (else after it)
        self._side = torch.cuda.Stream(device=dev)  # default priority
        self._fork = DeviceEvent()
        self._join = DeviceEvent()
        B, L = w.B, w.L
        self.rows = int(inp.key_offsets[-1])
        self.words = int(inp.mask_word_offsets[-1])
        self.key_off_h = inp.key_offsets.astype(np.int64)
        self.mwo_h = inp.mask_word_offsets.astype(np.int64)
        self.key_off = _dev(self.key_off_h, dev)
        self.mwo = _dev(self.mwo_h, dev)

        self.h = [_dev(inp.h[l], dev) for l in range(L)]
        self.mem = [tuple(_dev(x, dev) for x in (lw.w_dq, lw.w_iuq, lw.w_w)) for lw in inp.mem_w]
        self.nat = [tuple(_dev(x, dev) for x in (lw.w_dq, lw.w_iuq, lw.w_w)) for lw in inp.nat_w]
        # bf16 projection weights are packed once into the matrix-core operand layout
        self.packed = packed and w.act_dtype == "bf16" and B <= 32 and w.r % 64 == 0 and (w.n_h * w.d_h) % 64 == 0
        if self.packed:
            shapes = ((w.r, w.d), (w.n_h * w.d_h, w.r), (w.n_h, w.d))

            def pack(mats):
                out = []
                for m, (rows, K) in zip(mats, shapes):
                    buf = torch.empty(lsa.pack_weights_size(rows, K), dtype=torch.uint8, device=dev)
                    lsa.pack_weights(m, rows, K, buf)
                    out.append(buf)
                return tuple(out)

            self.mem = [pack(m) for m in self.mem]
            self.nat = [pack(m) for m in self.nat]
            torch.cuda.synchronize()
        self.keys = [_dev(inp.keys[l], dev) for l in range(L)]
        self.scale = [None if inp.key_scale[l] is None else _dev(inp.key_scale[l], dev) for l in range(L)]
        self.pool = None if inp.pool is None else _dev(inp.pool, dev)
        # the cold pool: the same rows in pinned host memory, read by lsa_fetch_host
        self.pool_host = None
        if host_pool and inp.pool is not None:
            a = np.ascontiguousarray(inp.pool)
            self.pool_host = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).pin_memory()

        f32, i32, i64, i16 = torch.float32, torch.int32, torch.int64, torch.int16
        out = self._out
        # 2L projection outputs: first L for the memory indexer, next L for the native indexer
        self.c = [out((B, w.r), f32) for _ in range(2 * L)]
        self.q = [out((B, w.n_h, w.d_h), f32) for _ in range(2 * L)]
        self.g = [out((B, w.n_h), f32) for _ in range(2 * L)]
        self.masks = [out((max(self.words, 1),), i64) for _ in range(L)]
        # with_scores: buffers for a separate score pass that also writes the sigmoid scores
        # (score_with_sigmoid); run() itself writes masks only
        self.scores = [out((max(self.rows, 1),), f32) for _ in range(L)] if with_scores else None
        self.masks_scored = [out((max(self.words, 1),), i64) for _ in range(L)] if with_scores else None
        self.score_options = None  # launch options of run()'s score pass (lsa_score_select_ex), None = defaults
        self.idx = out((max(self.rows, 1),), i32)
        self.count = out((B,), i32)
        self.union_mask = out((max(self.words, 1),), i64)
        self.topk_idx = [out((B, w.k), i32) for _ in range(L)]
        self.topk_score = [out((B, w.k), f32) for _ in range(L)] if with_topk_scores else None
        self.topk_count = out((L, B), i32)
        ws = lsa.topk_workspace_size(L, B, self.rows, w.k)
        self.workspace = out((max(ws, 4),), torch.uint8)
        self.gather_capacity = self.rows if gather_capacity is None else int(gather_capacity)
        if self.pool is not None:
            self.gathered = out((max(self.gather_capacity, 1), w.pool_dim), i16)
        # decode steps (allocated by alloc_steps): each layer's union rows of keys packed once per
        # trigger, the step's native query and gates, and the step's top-k outputs
        self.keys_sub = None

    def alloc_steps(self):
        """Buffers of the per-step top-k over the resident subset (lsa_topk_step)."""
        w, L, B = self.w, self.w.L, self.w.B
        f32, i32 = torch.float32, torch.int32
        kdt = {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8}[w.key_dtype]
        self.key_row_bytes = w.d_h * {"f32": 4, "bf16": 2, "fp8": 1}[w.key_dtype]
        self.keys_sub = [self._out((max(self.rows, 1), w.d_h), kdt) for _ in range(L)]
        self.h_step = [self._out((B, w.d), torch.int16 if w.act_dtype == "bf16" else f32) for _ in range(L)]
        self.c_step = [self._out((B, w.r), f32) for _ in range(L)]
        self.q_step = [self._out((B, w.n_h, w.d_h), f32) for _ in range(L)]
        self.g_step = [self._out((B, w.n_h), f32) for _ in range(L)]
        self.step_idx = [self._out((B, w.k), i32) for _ in range(L)]
        self.step_score = [self._out((B, w.k), f32) for _ in range(L)]
        self.step_count = self._out((L, B), i32)

    def _out(self, shape, dtype):
        """An output buffer. With guard=True it sits between two GUARD_BYTES canary bands."""
        n = 1
        for s_ in shape:
            n *= int(s_)
        if not self.guard:
            return torch.empty(shape, dtype=dtype, device=self.device)
        esz = torch.empty(0, dtype=dtype).element_size()
        nbytes = n * esz
        raw = torch.full((GUARD_BYTES + nbytes + GUARD_BYTES,), CANARY, dtype=torch.uint8, device=self.device)
        self._guarded.append((raw, nbytes))
        return raw[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)

    def check_guards(self):
        """Return the indices of output buffers whose canary bands were written."""
        bad = []
        for i, (raw, nbytes) in enumerate(self._guarded):
            head = raw[:GUARD_BYTES]
            tail = raw[GUARD_BYTES + nbytes:]
            if not (bool((head == CANARY).all()) and bool((tail == CANARY).all())):
                bad.append(i)
        return bad

    # ------------------------------------------------------------- stages
    def project(self, stream=None):
        w, L = self.w, self.w.L
        layers = []
        for j in range(2 * L):
            wdq, wiuq, ww = (self.mem if j < L else self.nat)[j % L]
            layers.append(dict(h=self.h[j % L], w_dq=wdq, w_iuq=wiuq, w_w=ww, c_out=self.c[j], q_out=self.q[j],
                               w_out=self.g[j]))
        if self.packed:
            lsa.project_packed(layers, B=w.B, d=w.d, r=w.r, n_h=w.n_h, d_h=w.d_h, stream=stream)
        else:
            lsa.project(layers, B=w.B, d=w.d, r=w.r, n_h=w.n_h, d_h=w.d_h, dtype=w.act_dtype, stream=stream)

    def score_select(self, stream=None):
        """The step's score pass: masks only, with score_options if set."""
        self._score_call(self.masks, None, self.score_options, stream)

    def score_with_sigmoid(self, stream=None, options=None):
        """A score pass that also writes the sigmoid scores (into scores and masks_scored)."""
        self._score_call(self.masks_scored, self.scores, options, stream)

    def _score_call(self, masks, scores, options, stream):
        w = self.w
        layers = [dict(q=self.q[l], w=self.g[l], keys=self.keys[l], key_scale=self.scale[l], mask_out=masks[l],
                       score_out=None if scores is None else scores[l]) for l in range(w.L)]
        lsa.score_select(layers, B=w.B, key_offsets=self.key_off, key_offsets_host=self.key_off_h,
                         mask_word_offsets=self.mwo, mask_word_offsets_host=self.mwo_h, n_h=w.n_h, d_h=w.d_h,
                         key_dtype=w.key_dtype, threshold=w.threshold, options=options, stream=stream)

    def union_compact(self, stream=None):
        w = self.w
        lsa.union_compact(self.masks, B=w.B, key_offsets=self.key_off, key_offsets_host=self.key_off_h,
                          mask_word_offsets=self.mwo, mask_word_offsets_host=self.mwo_h, idx_out=self.idx,
                          count_out=self.count, union_mask_out=self.union_mask, stream=stream)

    def _topk_layers(self):
        w, L = self.w, self.w.L
        return [dict(q=self.q[L + l], w=self.g[L + l], keys=self.keys[l], key_scale=self.scale[l],
                     topk_idx_out=self.topk_idx[l],
                     topk_score_out=None if self.topk_score is None else self.topk_score[l]) for l in range(L)]

    def topk(self, stream=None):
        w = self.w
        lsa.topk(self._topk_layers(), B=w.B, key_offsets=self.key_off, key_offsets_host=self.key_off_h,
                 idx=self.idx, count=self.count, n_h=w.n_h, d_h=w.d_h, key_dtype=w.key_dtype, k=w.k,
                 topk_count_out=self.topk_count, workspace=self.workspace, stream=stream)

    def topk_score_stage(self, stream=None):
        w = self.w
        lsa.topk_score(self._topk_layers(), B=w.B, key_offsets=self.key_off, key_offsets_host=self.key_off_h,
                       idx=self.idx, count=self.count, n_h=w.n_h, d_h=w.d_h, key_dtype=w.key_dtype,
                       workspace=self.workspace, stream=stream)

    def topk_select_stage(self, stream=None):
        w = self.w
        lsa.topk_select(self._topk_layers(), B=w.B, key_offsets=self.key_off, key_offsets_host=self.key_off_h,
                        idx=self.idx, count=self.count, k=w.k, topk_count_out=self.topk_count,
                        workspace=self.workspace, stream=stream)

    def gather(self, stream=None):
        if self.pool is None:
            return
        w = self.w
        lsa.gather(self.pool, row_bytes=w.pool_dim * 2, B=w.B, pool_row_offsets=self.key_off,
                   pool_row_offsets_host=self.key_off_h, idx=self.idx, idx_offsets=self.key_off, count=self.count,
                   out=self.gathered, out_capacity_rows=self.gather_capacity, stream=stream)

    def fetch_host(self, stream=None):
        """The gather's rows, read from the pinned host copy of the pool (lsa_fetch_host)."""
        if self.pool_host is None:
            return
        w = self.w
        lsa.fetch_host(self.pool_host, row_bytes=w.pool_dim * 2, B=w.B, pool_row_offsets=self.key_off,
                       pool_row_offsets_host=self.key_off_h, idx=self.idx, idx_offsets=self.key_off, count=self.count,
                       out=self.gathered, out_capacity_rows=self.gather_capacity, stream=stream)

    # ------------------------------------------------------------- decode steps
    def pack_subset_keys(self, stream=None):
        """Once per trigger: each layer's keys of the union rows, packed in list order (lsa_gather)."""
        w = self.w
        for l in range(w.L):
            lsa.gather(self.keys[l], row_bytes=self.key_row_bytes, B=w.B, pool_row_offsets=self.key_off,
                       pool_row_offsets_host=self.key_off_h, idx=self.idx, idx_offsets=self.key_off, count=self.count,
                       out=self.keys_sub[l], out_capacity_rows=self.rows, stream=stream)

    def set_step_hidden(self, h_step):
        """Copy one decode step's hidden states ([layer] -> [B, d] stored values) into HBM."""
        for l, hl in enumerate(h_step):
            a = np.ascontiguousarray(hl)
            self.h_step[l].copy_(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a))

    def step(self, stream=None):
        """One decode step: the native query and gates of the step's h (lsa_project with the native
        weights), then lsa_topk_step over the packed subset keys."""
        w, L = self.w, self.w.L
        layers = [dict(h=self.h_step[l], w_dq=self.nat[l][0], w_iuq=self.nat[l][1], w_w=self.nat[l][2],
                       c_out=self.c_step[l], q_out=self.q_step[l], w_out=self.g_step[l]) for l in range(L)]
        if self.packed:
            lsa.project_packed(layers, B=w.B, d=w.d, r=w.r, n_h=w.n_h, d_h=w.d_h, stream=stream)
        else:
            lsa.project(layers, B=w.B, d=w.d, r=w.r, n_h=w.n_h, d_h=w.d_h, dtype=w.act_dtype, stream=stream)
        self.step_topk(stream)

    def step_topk(self, stream=None):
        """lsa_topk_step with the step's native query (q_step, g_step) over the packed subset keys."""
        w, L = self.w, self.w.L
        tl = [dict(q=self.q_step[l], w=self.g_step[l], keys=self.keys_sub[l], key_scale=self.scale[l],
                   topk_idx_out=self.step_idx[l], topk_score_out=self.step_score[l]) for l in range(L)]
        lsa.topk_step(tl, B=w.B, key_offsets=self.key_off, key_offsets_host=self.key_off_h, idx=self.idx,
                      count=self.count, n_h=w.n_h, d_h=w.d_h, key_dtype=w.key_dtype, k=w.k,
                      topk_count_out=self.step_count, workspace=self.workspace, stream=stream)

    def load(self, stream=None):
        """The load step: from the host pool when there is one, else from HBM."""
        if self.pool_host is not None:
            self.fetch_host(stream)
        else:
            self.gather(stream)

    def run(self, stream=None):
        """One pass of the path. The load step (gather, or the cold-pool fetch) needs only the
        union list, so it runs on a second stream forked right after the union and compaction,
        overlapping both top-k stages, and joins at the end. (Forking it after the top-k
        scoring instead, so that it overlaps only the selection, is 14 us slower per step on
        the three-layer workload: the scoring and the gather share HBM better than they
        queue. Projecting the native indexer on the second stream while the memory indexer
        scores is 6 us slower per step: score_select is the HBM-bound stage and loses more
        than the projection gains. Projecting it after the union instead, on this stream while
        the load runs on the other, is 24 us slower on the three-layer workload: that phase is
        already bound by HBM, and the split adds a second pair of projection launches.)"""
        main = torch.cuda.current_stream() if stream is None else stream
        self.project(main)
        self.score_select(main)
        self.union_compact(main)
        if self.pool is None or not self.overlap:
            self.topk(main)
            self.load(main)
            return
        if self.early_fork:
            self._fork.record(main)
            self._fork.wait(self._side)
            self.load(self._side)
            self.topk_score_stage(main)
        else:
            self.topk_score_stage(main)
            self._fork.record(main)
            self._fork.wait(self._side)
            self.load(self._side)
        self.topk_select_stage(main)
        self._join.record(self._side)
        self._join.wait(main)

    def capture(self):
        """Record one run() into a HIP graph and return it (replay with .replay()).

        run() allocates nothing and clears nothing with memset, so the graph holds
        exactly the kernel launches of the five calls, with these buffers baked in.
        """
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        return g

    def outputs(self):
        """Every output buffer of run(), for comparisons between runs."""
        out = self.c + self.q + self.g + self.masks + [self.idx, self.count, self.union_mask, self.topk_count]
        out += self.topk_idx
        if self.topk_score is not None:
            out += self.topk_score
        if self.pool is not None:
            out.append(self.gathered)
        return out

    # ------------------------------------------------------------- readback
    def masks_bool(self, l, scored=False):
        """Unpack layer l's mask words (of run(), or of score_with_sigmoid) into one bool array per sequence."""
        words = (self.masks_scored if scored else self.masks)[l][: self.words].cpu().numpy().view(np.uint64)
        return self._unpack(words)

    def union_bool(self):
        return self._unpack(self.union_mask[: self.words].cpu().numpy().view(np.uint64))

    def _unpack(self, words):
        out = []
        bits = np.unpackbits(words.view(np.uint8), bitorder="little")
        for b in range(self.w.B):
            w0, w1 = int(self.mwo_h[b]), int(self.mwo_h[b + 1])
            n = int(self.key_off_h[b + 1] - self.key_off_h[b])
            seg = bits[w0 * 64: w1 * 64]
            out.append((seg[:n].astype(bool), seg[n:].astype(bool)))
        return out
