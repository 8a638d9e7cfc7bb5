"""Comparison of the HIP path with the CPU oracle, to the tolerances the method's target fixes:
  * sigmoid scores within 2e-3 absolute;
  * selected and top-k sets identical, except entries whose oracle logit is within 1e-2 of
    the threshold (logit 0) or of the k-th value;
  * everything integer (compaction, counts, padding) and the gather bit-exact.
Where several results are correct (near-ties), the unique part is compared and the rest is
checked for validity.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import lsa_oracle as O

BAND = 1e-2        # logit band around the threshold / the k-th value
SCORE_TOL = 2e-3   # sigmoid score tolerance


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def proj_tol(c_in, W):
    """Per-output error allowance for a projection: 1e-4 of sum_k |c_k||W_km| plus a tiny floor.

    The kernel accumulates in fp32 and feeds c as bf16 hi + lo (about 2^-17 relative per
    element). The allowance is loose compared with that, but an indexing error would still
    show up as an O(1) relative error."""
    return 1e-4 * (np.abs(c_in) @ np.abs(W).T) + 1e-6


def check_projection(p, inp, ref):
    w = inp.workload
    for l in range(w.L):
        c = p.c[l].cpu().numpy(); q = p.q[l].cpu().numpy(); g = p.g[l].cpu().numpy()
        mw = inp.mem_w[l]
        H = O.decode_act(inp.h[l], w.act_dtype)
        Wdq = O.decode_act(mw.w_dq, w.act_dtype)
        Wiuq = O.decode_act(mw.w_iuq, w.act_dtype)
        Ww = O.decode_act(mw.w_w, w.act_dtype)
        for b in ref:
            rc, rq, rw = ref[b]["c"][l], ref[b]["q"][l], ref[b]["w"][l]
            assert np.all(np.abs(c[b] - rc) <= proj_tol(H[b], Wdq)), f"c mismatch l={l} b={b}"
            assert np.all(np.abs(g[b] - rw) <= proj_tol(H[b], Ww)), f"w mismatch l={l} b={b}"
            tq = proj_tol(rc, Wiuq).reshape(w.n_h, w.d_h)
            assert np.all(np.abs(q[b] - rq) <= tq), f"q mismatch l={l} b={b} max {np.abs(q[b] - rq).max()}"


def check_masks(p, inp, ref, with_scores):
    w = inp.workload
    stats = {"band": 0, "mismatch_in_band": 0, "max_dI": 0.0}
    for l in range(w.L):
        mb = p.masks_bool(l)
        for b in ref:
            m, tail = mb[b]
            assert not tail.any(), f"bits beyond N_b set l={l} b={b}"
            x = ref[b]["x"][l]
            band = np.abs(x) <= BAND
            bad = (m != ref[b]["mask"][l]) & ~band
            assert not bad.any(), f"selection differs outside the band l={l} b={b}: {np.flatnonzero(bad)[:10]}"
            stats["band"] += int(band.sum())
            stats["mismatch_in_band"] += int(((m != ref[b]["mask"][l]) & band).sum())
            # exact-zero rule: every head's dot clearly negative -> logit exactly 0 -> selected
            s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
            if s1 > s0:
                K = O.decode_keys(inp.keys[l][s0:s1], w.key_dtype,
                                  None if inp.key_scale[l] is None else inp.key_scale[l][s0:s1])
                allneg = (K @ ref[b]["q"][l].T).max(axis=1) < -1e-3
                assert m[allneg].all(), f"exact-zero entries not selected l={l} b={b}"
            if with_scores:
                I = p.scores[l][s0:s1].cpu().numpy()
                d = np.abs(I - ref[b]["I"][l])
                stats["max_dI"] = max(stats["max_dI"], float(d.max(initial=0)))
                assert d.max(initial=0) <= SCORE_TOL, f"sigmoid score error {d.max()} l={l} b={b}"
    return stats


def gpu_union_lists(p, inp):
    counts = p.count.cpu().numpy()
    idx = p.idx.cpu().numpy()
    return counts, [idx[inp.key_offsets[b]: inp.key_offsets[b] + counts[b]].astype(np.int64)
                    for b in range(inp.workload.B)]


def check_union(p, inp, ref):
    w = inp.workload
    counts, lists = gpu_union_lists(p, inp)
    ub = p.union_bool()
    masks = [p.masks_bool(l) for l in range(w.L)]
    for b in ref:
        gm = [masks[l][b][0] for l in range(w.L)]
        U = O.union(gm)
        # integer work on the GPU's own masks: bit-exact
        assert np.array_equal(ub[b][0], U) and not ub[b][1].any(), f"union mask b={b}"
        assert np.array_equal(lists[b], O.compact(U)), f"compacted list b={b}"
        assert counts[b] == U.sum()
        # against the oracle's own union, outside the band
        anyband = np.zeros(U.size, bool)
        for l in range(w.L):
            anyband |= np.abs(ref[b]["x"][l]) <= BAND
        assert not ((U != ref[b]["union"]) & ~anyband).any(), f"union differs from the oracle outside the band b={b}"
    return counts, lists


def check_topk(p, inp, ref, lists):
    w = inp.workload
    tk_idx = [t.cpu().numpy() for t in p.topk_idx]
    tk_sc = None if p.topk_score is None else [t.cpu().numpy() for t in p.topk_score]
    tk_cnt = p.topk_count.cpu().numpy()
    # the GPU's fp32 score of every union entry, in list order: [l, key_offsets[b] + i]
    ws = p.workspace[: 4 * w.L * p.rows].cpu().numpy().view(np.float32).reshape(w.L, p.rows)
    for b in ref:
        idx = lists[b]
        s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
        for l in range(w.L):
            K = O.decode_keys(inp.keys[l][s0:s1], w.key_dtype,
                              None if inp.key_scale[l] is None else inp.key_scale[l][s0:s1])
            y = O.logits(ref[b]["qn"][l], ref[b]["wn"][l], K[idx]) if idx.size else np.zeros(0)
            want = O.topk(y, idx, w.k)
            M = idx.size
            n = min(w.k, M)
            assert tk_cnt[l, b] == n, f"topk count l={l} b={b}: {tk_cnt[l, b]} vs {n}"
            got = tk_idx[l][b]
            assert np.all(got[n:] == -1), "padding"
            got = got[:n].astype(np.int64)
            assert np.all(np.diff(got) > 0), "top-k output not ascending"
            assert np.all(np.isin(got, idx)), "top-k picked an entry outside the subset"
            # The integer decision, in the GPU's own precision: its list is exactly the (-y, s)
            # top-k of its own fp32 scores (ties to the lower index).
            y_gpu = ws[l, s0:s0 + M].astype(np.float64)
            assert np.array_equal(got, O.topk(y_gpu, idx, w.k)), f"top-k vs own scores l={l} b={b}"
            if M > w.k:
                kth = np.sort(y)[::-1][w.k - 1]
                yv = dict(zip(idx.tolist(), y.tolist()))
                diff = np.setxor1d(got, want)
                for s in diff:
                    assert abs(yv[int(s)] - kth) <= BAND, f"top-k differs at s={s}: y={yv[int(s)]} kth={kth}"
            else:
                assert np.array_equal(got, want)
            if tk_sc is not None and n:
                yv = dict(zip(idx.tolist(), y.tolist()))
                ys = np.array([yv[int(s)] for s in got])
                assert np.abs(tk_sc[l][b][:n] - ys).max() <= BAND, "top-k scores"
                assert np.all(np.isneginf(tk_sc[l][b][n:]))


def check_gather(p, inp, lists, sample=None, rng=None):
    if inp.pool is None:
        return
    out = p.gathered.cpu().numpy().view(np.uint16)
    off = 0
    for b in range(inp.workload.B):
        idx = lists[b]
        s0 = int(inp.key_offsets[b])
        rows = np.arange(idx.size)
        if sample is not None and idx.size > sample:
            rows = np.sort(rng.choice(idx.size, sample, replace=False))
        exp = inp.pool[s0 + idx[rows]]
        assert np.array_equal(out[off + rows], exp), f"gather b={b}"
        off += idx.size


def full_check(p, inp, with_scores=True):
    ref = O.run_path(inp)
    check_projection(p, inp, ref)
    st = check_masks(p, inp, ref, with_scores)
    counts, lists = check_union(p, inp, ref)
    check_topk(p, inp, ref, lists)
    check_gather(p, inp, lists)
    return st, counts
