"""Comparison of the HIP path with the CPU oracle, to the tolerances the method's target fixes:
  * sigmoid scores within 2e-3 absolute;
  * selected and top-k sets identical, except entries whose oracle logit is within 1e-2 of
    the logit threshold ln(theta/(1-theta)) or of the k-th value;
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


GUARD_BAND = 2e-3  # the two GPU score passes differ only in fp32 summation order


def check_masks(p, inp, ref, with_scores):
    """Masks of run() (the step's mask-only score pass, with its launch options) against the oracle,
    and with_scores: the masks and sigmoid scores of the full pass (score_with_sigmoid), and the
    two passes' masks against each other."""
    w = inp.workload
    thr = O.logit_threshold(w.threshold)
    stats = {"band": 0, "mismatch_in_band": 0, "max_dI": 0.0, "run_vs_scored": 0}
    if with_scores:
        p.score_with_sigmoid()
    for l in range(w.L):
        sets = [("run", p.masks_bool(l))]
        if with_scores:
            sets.append(("scored", p.masks_bool(l, scored=True)))
        for b in ref:
            x = ref[b]["x"][l]
            band = np.abs(x - thr) <= BAND
            s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
            allneg = None
            if s1 > s0:
                K = O.decode_keys(inp.keys[l][s0:s1], w.key_dtype,
                                  None if inp.key_scale[l] is None else inp.key_scale[l][s0:s1])
                allneg = (K @ ref[b]["q"][l].T).max(axis=1) < -1e-3
            for what, mb in sets:
                m, tail = mb[b]
                assert not tail.any(), f"{what}: bits beyond N_b set l={l} b={b}"
                bad = (m != ref[b]["mask"][l]) & ~band
                assert not bad.any(), f"{what}: selection differs outside the band l={l} b={b}: {np.flatnonzero(bad)[:10]}"
                if what == "run":
                    stats["band"] += int(band.sum())
                    stats["mismatch_in_band"] += int(((m != ref[b]["mask"][l]) & band).sum())
                # exact-zero rule: every head's dot clearly negative -> logit exactly 0 -> selected iff 0 >= thr
                if allneg is not None:
                    assert np.array_equal(m[allneg], np.full(int(allneg.sum()), 0.0 >= thr)), \
                        f"{what}: exact-zero entries l={l} b={b}"
            if with_scores:
                diff = sets[0][1][b][0] != sets[1][1][b][0]
                assert not (diff & (np.abs(x - thr) > GUARD_BAND)).any(), f"the two score passes differ l={l} b={b}"
                stats["run_vs_scored"] += int(diff.sum())
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
        thr = O.logit_threshold(w.threshold)
        anyband = np.zeros(U.size, bool)
        for l in range(w.L):
            anyband |= np.abs(ref[b]["x"][l] - thr) <= BAND
        assert not ((U != ref[b]["union"]) & ~anyband).any(), f"union differs from the oracle outside the band b={b}"
    return counts, lists


def check_topk_one(got, got_sc, got_cnt, y_gpu, idx, y, k, what):
    """One (layer, sequence) top-k against the oracle's scores y of the list idx.

    The integer decision is checked in the GPU's own precision: the list must be exactly the
    (-y, s) top-k of the GPU's fp32 scores y_gpu (ties to the lower index). Against the oracle,
    every entry where the two lists differ must have an oracle score within BAND of the k-th."""
    M = idx.size
    n = min(k, M)
    assert got_cnt == n, f"{what}: top-k count {got_cnt} vs {n}"
    assert np.all(got[n:] == -1), f"{what}: padding"
    g = got[:n].astype(np.int64)
    assert np.all(np.diff(g) > 0), f"{what}: top-k output not ascending"
    assert np.all(np.isin(g, idx)), f"{what}: top-k picked an entry outside the subset"
    assert np.array_equal(g, O.topk(y_gpu.astype(np.float64), idx, k)), f"{what}: top-k vs own scores"
    want = O.topk(y, idx, k)
    if M > k:
        kth = np.sort(y)[::-1][k - 1]
        yv = dict(zip(idx.tolist(), y.tolist()))
        for s_ in np.setxor1d(g, want):
            assert abs(yv[int(s_)] - kth) <= BAND, f"{what}: top-k differs at s={s_}: y={yv[int(s_)]} kth={kth}"
    else:
        assert np.array_equal(g, want), f"{what}: top-k"
    if got_sc is not None and n:
        yv = dict(zip(idx.tolist(), y.tolist()))
        ys = np.array([yv[int(s_)] for s_ in g])
        assert np.abs(got_sc[:n] - ys).max() <= BAND, f"{what}: top-k scores"
        assert np.all(np.isneginf(got_sc[n:])), f"{what}: score padding"


def workspace_scores(p):
    """The GPU's fp32 score of every list entry: [l, key_offsets[b] + i]."""
    w = p.w
    return p.workspace[: 4 * w.L * p.rows].cpu().numpy().view(np.float32).reshape(w.L, p.rows)


def check_topk(p, inp, ref, lists):
    w = inp.workload
    tk_idx = [t.cpu().numpy() for t in p.topk_idx]
    tk_sc = None if p.topk_score is None else [t.cpu().numpy() for t in p.topk_score]
    tk_cnt = p.topk_count.cpu().numpy()
    ws = workspace_scores(p)
    for b in ref:
        idx = lists[b]
        s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
        for l in range(w.L):
            K = O.decode_keys(inp.keys[l][s0:s1], w.key_dtype,
                              None if inp.key_scale[l] is None else inp.key_scale[l][s0:s1])
            y = O.logits(ref[b]["qn"][l], ref[b]["wn"][l], K[idx]) if idx.size else np.zeros(0)
            check_topk_one(tk_idx[l][b], None if tk_sc is None else tk_sc[l][b], int(tk_cnt[l, b]),
                           ws[l, s0:s0 + idx.size], idx, y, w.k, f"top-k l={l} b={b}")


def check_step(p, inp, h_step, lists, what):
    """One decode step's top-k (p.step_idx, p.step_score, p.step_count) against the oracle's
    step_topk over the same resident lists."""
    w = inp.workload
    ref = O.step_topk(inp, h_step, lists)
    tk_idx = [t.cpu().numpy() for t in p.step_idx]
    tk_sc = [t.cpu().numpy() for t in p.step_score]
    tk_cnt = p.step_count.cpu().numpy()
    ws = workspace_scores(p)
    for b in range(w.B):
        s0 = int(inp.key_offsets[b])
        idx = lists[b]
        for l in range(w.L):
            _, y = ref[(b, l)]
            check_topk_one(tk_idx[l][b], tk_sc[l][b], int(tk_cnt[l, b]), ws[l, s0:s0 + idx.size], idx, y, w.k,
                           f"{what} l={l} b={b}")


def check_gather(p, inp, lists):
    """Every gathered row, bit for bit, and nothing written past the packed rows' end."""
    if inp.pool is None:
        return
    out = p.gathered.cpu().numpy().view(np.uint16)
    off = 0
    for b in range(inp.workload.B):
        idx = lists[b]
        s0 = int(inp.key_offsets[b])
        assert np.array_equal(out[off:off + idx.size], inp.pool[s0 + idx]), f"gather b={b}"
        off += idx.size


def full_check(p, inp, with_scores=True):
    ref = O.run_path(inp)
    check_projection(p, inp, ref)
    st = check_masks(p, inp, ref, with_scores)
    counts, lists = check_union(p, inp, ref)
    check_topk(p, inp, ref, lists)
    check_gather(p, inp, lists)
    return st, counts
