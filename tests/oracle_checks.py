"""Checks that pin the CPU oracle to things other than itself.

Each `check_*` function takes the oracle module (or a copy with a deliberate
mistake planted in it) and raises AssertionError if that oracle disagrees with
an independent fact: hand-worked integers, exact rational brute force, closed
forms or library conversions. `test_oracle_pins.py` runs them on the real
oracle. `test_oracle_mutations.py` runs them on mutated copies to show that
every plausible mistake is caught by at least one check.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import brute
from sparse_kv_retrieval_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_hand():
    with open(os.path.join(GOLDEN, "hand_example_2head_8entry.json")) as f:
        return json.load(f)


# -------------------------------------------------------------- hand example
def check_hand_scores(O):
    g = load_hand()
    K = np.array(g["keys"], np.float64)
    masks = []
    for lay in g["layers"]:
        x = O.logits(np.array(lay["q"], np.float64), np.array(lay["w"], np.float64), K)
        assert np.array_equal(x, np.array(lay["x"], np.float64)), (x, lay["x"])
        I = O.sigmoid(x)
        assert np.allclose(I, lay["I"], atol=1e-10, rtol=0), (I, lay["I"])
        m = O.select(x, 0.5)
        assert O.compact(m).tolist() == lay["selected"]
        masks.append(m)
    U = O.union(masks)
    assert O.compact(U).tolist() == g["union"]


def check_hand_topk(O):
    g = load_hand()
    K = np.array(g["keys"], np.float64)
    lay = g["layers"][0]
    idx = np.array(g["union"], np.int64)
    y = O.logits(np.array(lay["q"], np.float64), np.array(lay["w"], np.float64), K[idx])
    for k, want in g["topk_with_layer0_query"].items():
        if k == "about":
            continue
        got = O.topk(y, idx, int(k))
        assert got.tolist() == want, (k, got, want)


def check_hand_projection(O):
    p = load_hand()["projection"]
    h = np.array([p["h"]], np.float64)
    W_dq, W_iuq, W_w = (np.array(p[n], np.float64) for n in ("W_dq", "W_iuq", "W_w"))
    # The oracle takes the "out x in" storage layout, i.e. the transposes.
    c, q, w = O.project(h, W_dq.T.copy(), W_iuq.T.copy(), W_w.T.copy(), 1, 2)
    assert np.array_equal(c[0], p["c"]), c
    assert np.array_equal(q[0], np.array(p["q"], np.float64)), q
    assert np.array_equal(w[0], p["w"]), w
    x = O.logits(q[0], w[0], np.array(p["keys"], np.float64))
    assert np.array_equal(x, p["x"]), x
    assert O.compact(O.select(x, 0.5)).tolist() == p["selected"]


# ----------------------------------------------------------- closed forms
def check_sigmoid_closed_forms(O):
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    l3 = math.log(3.0)
    v = O.sigmoid(np.array([l3, -l3, 745.0, -745.0, 40.0]))
    assert abs(v[0] - 0.75) < 1e-15 and abs(v[1] - 0.25) < 1e-15
    assert v[2] == 1.0 and 0.0 <= v[3] < 1e-300 and np.all(np.isfinite(v))
    x = np.linspace(-30, 30, 601)
    assert np.allclose(O.sigmoid(x) + O.sigmoid(-x), 1.0, atol=1e-15)
    assert np.all(np.diff(O.sigmoid(x)) >= 0)


def check_threshold(O):
    assert O.logit_threshold(0.5) == 0.0
    assert abs(O.logit_threshold(0.75) - math.log(3.0)) < 1e-15
    assert abs(O.logit_threshold(0.25) + math.log(3.0)) < 1e-15
    # inclusive at the boundary; sigma is increasing, so I >= theta <=> x >= logit(theta)
    assert O.select(np.array([0.0, -0.0, -1e-300, 1e-300]), 0.5).tolist() == [True, True, False, True]
    rng = np.random.default_rng(7)
    x = rng.normal(0, 3, 4000)
    for th in (0.1, 0.5, 0.9):
        t = math.log(th / (1 - th))
        far = np.abs(x - t) > 1e-9
        assert np.array_equal(O.select(x, th)[far], (O.sigmoid(x) >= th)[far])


# -------------------------------------------------------- decoders
def check_bf16_decode(O):
    import torch
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, 20000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = O.bf16_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[fin], ref[fin])
    assert O.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0001], np.uint16)).tolist() == [1.0, -2.0, 2.0 ** -133]
    assert O.bf16_to_f64(np.array([0x7F7F], np.uint16))[0] == (2 - 2 ** -7) * 2.0 ** 127


def check_e4m3fn(O):
    import torch
    t = O.E4M3FN_TABLE
    # points fixed by the OCP FP8 definition (E4M3: bias 7, no inf, S.1111.111 = NaN)
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1, t[0x80]) == -1
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6 and t[0x0F] == 1.875 * 2.0 ** -6
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    # independent implementation: torch's float8_e4m3fn
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(t[fin], ref[fin])


# ----------------------------------------------------------- brute force
def _tiny_case(rng, n_h, d_h, d, r, N, dtype):
    def act(shape, scale):
        v = (rng.standard_normal(shape) * scale).astype(np.float32)
        return v if dtype == "f32" else synth.f32_to_bf16_bits(v)
    h = act((1, d), 1.0)
    wdq, wiuq, ww = act((r, d), 1 / math.sqrt(d)), act((n_h * d_h, r), 1 / math.sqrt(r)), act((n_h, d), 1 / math.sqrt(d))
    kraw = rng.standard_normal((N, d_h)).astype(np.float32)
    if dtype == "fp8":
        sc = (np.abs(kraw).max(axis=1) / 448.0).astype(np.float32) if N else np.zeros(0, np.float32)
        sc[sc == 0] = 1
        keys = synth.f32_to_e4m3fn_bits(kraw / sc[:, None])
        return h, wdq, wiuq, ww, keys, sc
    keys = kraw if dtype == "f32" else synth.f32_to_bf16_bits(kraw)
    return h, wdq, wiuq, ww, keys, None


def check_brute_force(O, seeds=range(6)):
    """Oracle vs exact rationals on tiny random inputs (f32, bf16, fp8 keys)."""
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        n_h = (1, 2, 4)[seed % 3]
        d_h = (2, 4, 8)[seed % 3]
        d, r = 6, 3 + seed % 3
        kdt = ("f32", "bf16", "fp8")[seed % 3]
        N = (0, 1, 5, 17, 33, 9)[seed % 6]
        L = 2
        masks_o, masks_b, xs_b, lay_q = [], [], [], []
        for l in range(L):
            h, wdq, wiuq, ww, keys, sc = _tiny_case(rng, n_h, d_h, d, r, N, kdt)
            H = O.decode_act(h, "f32" if h.dtype == np.float32 else "bf16")
            Wdq = O.decode_act(wdq, "f32" if wdq.dtype == np.float32 else "bf16")
            Wiuq = O.decode_act(wiuq, "f32" if wiuq.dtype == np.float32 else "bf16")
            Ww = O.decode_act(ww, "f32" if ww.dtype == np.float32 else "bf16")
            K = O.decode_keys(keys, kdt, sc)
            c, q, w = O.project(H, Wdq, Wiuq, Ww, n_h, d_h)
            # exact keys straight from the stored values: the fp8 bytes and scales are decoded
            # by the brute-force module's own field decoder, not by the oracle
            Kb = brute.fp8_keys(keys, sc) if kdt == "fp8" else brute.mat(keys.astype(np.float64) if kdt == "f32"
                                                                         else synth.bf16_bits_to_f32(keys))
            assert np.array_equal(K, np.array([[float(v) for v in row] for row in Kb], np.float64).reshape(K.shape))
            # exact path (math layout = transposes of the stored buffers)
            hb = [brute.frac(v) for v in H[0]]
            cb, qb, wb = brute.project(hb, brute.mat(Wdq.T), brute.mat(Wiuq.T), brute.mat(Ww.T), n_h, d_h)
            assert np.allclose(c[0], [float(v) for v in cb], rtol=1e-12, atol=1e-12)
            assert np.allclose(q[0].ravel(), [float(v) for row in qb for v in row], rtol=1e-11, atol=1e-11)
            assert np.allclose(w[0], [float(v) for v in wb], rtol=1e-12, atol=1e-12)
            # exact logits from the exact q, w
            xb = [brute.logit(qb, wb, key) for key in Kb]
            x = O.logits(q[0], w[0], K)
            scale = 1.0 + max([abs(float(v)) for v in xb] or [0.0])
            assert np.allclose(x, [float(v) for v in xb], rtol=0, atol=1e-9 * scale)
            m = O.select(x, 0.5)
            mb = np.array([brute.selected_half(v) for v in xb], bool)
            decided = np.array([abs(float(v)) > 1e-9 * scale or v == 0 for v in xb], bool)
            assert np.array_equal(m[decided], mb[decided])
            masks_o.append(m)
            masks_b.append(mb)
            xs_b.append(xb)
            lay_q.append((q[0], w[0], K, qb, wb, Kb))
        U = O.union(masks_o)
        idx = O.compact(U)
        ub = [s for s in range(N) if any(mb[s] for mb in masks_b)]
        assert idx.tolist() == ub
        # top-k with layer 0's query inside the union, exact
        q0, w0, K0, qb0, wb0, Kb0 = lay_q[0]
        y = O.logits(q0, w0, K0[idx]) if idx.size else np.zeros(0)
        yb = [brute.logit(qb0, wb0, Kb0[s]) for s in ub]
        for k in (1, 2, 5, 64):
            assert O.topk(y, idx, k).tolist() == brute.topk(yb, ub, k)


# ------------------------------------------------------------ special cases
def check_special_cases(O):
    rng = np.random.default_rng(3)
    K = rng.standard_normal((257, 8))
    q = rng.standard_normal((3, 8))
    # all gates zero: every logit is exactly 0, I = 0.5, everything is selected
    x = O.logits(q, np.zeros(3), K)
    assert np.all(x == 0) and np.all(O.select(x))
    # one head, gate -1: selected iff q.K <= 0
    x = O.logits(q[:1], np.array([-1.0]), K)
    assert np.array_equal(O.select(x), (K @ q[0]) <= 0)
    # one head, gate +1: the logit is ReLU(q.K) >= 0, so everything is selected
    x = O.logits(q[:1], np.array([1.0]), K)
    assert np.all(O.select(x)) and np.array_equal(x, np.maximum(K @ q[0], 0))
    # h = e_i: c is row i of W^DQ (column i of the out x in buffer), exactly
    d, r = 5, 4
    wdq = rng.standard_normal((r, d))
    wiuq = rng.standard_normal((2 * 3, r))
    ww = rng.standard_normal((2, d))
    for i in range(d):
        e = np.zeros((1, d)); e[0, i] = 1.0
        c, _, w = O.project(e, wdq, wiuq, ww, 2, 3)
        assert np.array_equal(c[0], wdq[:, i]) and np.array_equal(w[0], ww[:, i])
    # small integers: everything is exact, so compare with integer arithmetic
    hi = rng.integers(-3, 4, (2, d)); Wd = rng.integers(-2, 3, (r, d)); Wu = rng.integers(-2, 3, (6, r))
    Ww = rng.integers(-2, 3, (2, d))
    c, q2, w2 = O.project(hi.astype(float), Wd.astype(float), Wu.astype(float), Ww.astype(float), 2, 3)
    ci = [[sum(int(hi[b, i]) * int(Wd[n, i]) for i in range(d)) for n in range(r)] for b in range(2)]
    assert np.array_equal(c, np.array(ci, float))
    qi = [[sum(ci[b][n] * int(Wu[m, n]) for n in range(r)) for m in range(6)] for b in range(2)]
    assert np.array_equal(q2.reshape(2, 6), np.array(qi, float))
    wi = [[sum(int(hi[b, i]) * int(Ww[j, i]) for i in range(d)) for j in range(2)] for b in range(2)]
    assert np.array_equal(w2, np.array(wi, float))


def check_union_compact(O):
    rng = np.random.default_rng(5)
    for N in (0, 1, 63, 64, 65, 1000):
        ms = [rng.random(N) < p for p in (0.1, 0.3, 0.05)]
        U = O.union(ms)
        for m in ms:
            assert np.all(U[m])                        # superset of each layer
        assert np.array_equal(O.union(ms[:1]), ms[0])  # L = 1: identity
        assert np.array_equal(O.union(ms + ms), U)     # idempotent
        idx = O.compact(U)
        assert idx.size == int(U.sum())                # count = popcount
        assert np.all(np.diff(idx) > 0)                # strictly ascending
        mem = np.zeros(N, bool); mem[idx] = True
        assert np.array_equal(mem, U)                  # membership <=> bit
        # against the definition written as a loop
        assert idx.tolist() == [s for s in range(N) if any(m[s] for m in ms)]


def check_topk_properties(O):
    rng = np.random.default_rng(9)
    for M in (0, 1, 5, 100, 1000):
        idx = np.sort(rng.choice(5000, M, replace=False)).astype(np.int64)
        y = np.round(rng.standard_normal(M) * 4) / 2          # many ties
        for k in (1, 3, 50, 2048):
            out = O.topk(y, idx, k)
            assert out.size == min(k, M)
            assert np.all(np.diff(out) > 0)
            keep = np.isin(idx, out)
            if keep.any() and (~keep).any():
                assert y[keep].min() >= y[~keep].max()          # dominance
                kth = y[keep].min()
                # at the k-th value, the kept ones are the lowest indices
                tie = y == kth
                assert np.all(idx[tie & keep].max(initial=-1) < idx[tie & ~keep].min(initial=1 << 40))
            if k >= M:
                assert np.array_equal(out, idx)


def check_gather(O):
    rng = np.random.default_rng(11)
    pool = rng.integers(0, 1 << 16, (300, 24), dtype=np.uint16)
    pool[5, :] = 0x7FC1          # NaN pattern as bf16
    pool[6, :] = 0xFF80          # -inf
    idx = np.array([0, 5, 6, 17, 299], np.int64)
    out = O.gather(pool, idx)
    assert out.dtype == np.uint16
    for i, s in enumerate(idx):
        assert out[i].tobytes() == pool[s].tobytes()


def check_same_query_topk(O):
    """If the native query equals the memory-indexer query, the top-k is the top-k of I."""
    rng = np.random.default_rng(13)
    K = rng.standard_normal((500, 8))
    q = rng.standard_normal((4, 8)); w = rng.standard_normal(4)
    x = O.logits(q, w, K)
    idx = O.compact(O.select(x))
    out = O.topk(O.logits(q, w, K[idx]), idx, 10)
    I = O.sigmoid(x)
    # the 10 selected entries with the largest I (ties cannot occur with continuous data)
    best = idx[np.argsort(-I[idx], kind="stable")[:10]]
    assert np.array_equal(out, np.sort(best))


# ------------------------------------------------------------- fp8 scale
def load_json(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def check_fp8_scale_hand(O):
    """e4m3fn bytes times their per-entry scale, against values decoded by hand."""
    g = load_json("fp8_keys_hand.json")
    for case in (g, g["square"]):
        got = O.decode_keys(np.array(case["bytes"], np.uint8), "fp8", np.array(case["scales"], np.float32))
        assert np.array_equal(got, np.array(case["keys"], np.float64)), (got, case["keys"])


# ------------------------------------------------------- whole-path wiring
def hand_inputs(key_dtype="f32", k=2):
    """The run_path_hand.json example as a synthetic-input object (one sequence, two layers)."""
    g = load_json("run_path_hand.json")
    w = synth.Workload("hand_path", 99, B=1, L=2, d=2, r=1, n_h=2, d_h=2, key_dtype=key_dtype, act_dtype="f32",
                       k=k, N=(8,), pool_dim=4)
    f32 = lambda a: np.array(a, np.float32)
    lw = lambda e: synth.LayerWeights(w_dq=f32(e["w_dq"]), w_iuq=f32(e["w_iuq"]), w_w=f32(e["w_w"]))
    if key_dtype == "fp8":
        keys = [np.array(b, np.uint8) for b in g["fp8"]["bytes"]]
        scales = [f32(s) for s in g["fp8"]["scales"]]
    else:
        keys = [f32(k_) for k_ in g["keys"]]
        scales = [None, None]
    pool = (np.arange(8 * 4, dtype=np.uint16).reshape(8, 4) * np.uint16(37) + np.uint16(0x3F00))
    return g, synth.Inputs(workload=w, lengths=np.array([8], np.int64), key_offsets=np.array([0, 8], np.int64),
                           mask_word_offsets=np.array([0, 1], np.int64), h=[f32(g["h"][0:1]), f32(g["h"][1:2])],
                           mem_w=[lw(e) for e in g["mem"]], nat_w=[lw(e) for e in g["nat"]], keys=keys,
                           key_scale=scales, pool=pool)


def check_run_path_hand(O):
    """The whole path on the hand example: which weights and which layer's keys feed each step."""
    for kdt in ("f32", "fp8"):
        for k in ("2", "5", "8"):
            g, inp = hand_inputs(kdt, int(k))
            r = O.run_path(inp)[0]
            for l in range(2):
                assert np.array_equal(r["c"][l], g["mem"][l]["c"]), (kdt, l, r["c"][l])
                assert np.array_equal(r["q"][l], np.array(g["mem"][l]["q"], np.float64)), (kdt, l)
                assert np.array_equal(r["w"][l], g["mem"][l]["w"]), (kdt, l)
                assert np.array_equal(r["x"][l], g["x"][l]), (kdt, l, r["x"][l])
                assert O.compact(r["mask"][l]).tolist() == g["selected"][l], (kdt, l)
                assert np.array_equal(r["qn"][l], np.array(g["nat"][l]["q"], np.float64)), (kdt, l)
                assert np.array_equal(r["wn"][l], g["nat"][l]["w"]), (kdt, l)
                assert np.array_equal(r["y"][l], g["y"][l]), (kdt, l, r["y"][l])
                assert r["topk"][l].tolist() == g["topk"][k][l], (kdt, k, l, r["topk"][l])
            assert r["idx"].tolist() == g["union"], (kdt, r["idx"])
            assert np.array_equal(r["gathered"], inp.pool[g["union"]])


def check_step_topk_hand(O):
    """One decode step's top-k over the resident subset, on the hand example."""
    for kdt in ("f32", "fp8"):
        for k in ("2", "5"):
            g, inp = hand_inputs(kdt, int(k))
            st = g["step"]
            h_step = [np.array([st["h"][l]], np.float32) for l in range(2)]
            r = O.step_topk(inp, h_step, [np.array(g["union"], np.int64)])
            for l in range(2):
                tk, y = r[(0, l)]
                assert np.array_equal(y, st["y"][l]), (kdt, l, y)
                assert tk.tolist() == st["topk"][k][l], (kdt, k, l, tk)


ALL_CHECKS = [
    check_hand_scores, check_hand_topk, check_hand_projection, check_sigmoid_closed_forms,
    check_threshold, check_bf16_decode, check_e4m3fn, check_brute_force, check_special_cases,
    check_union_compact, check_topk_properties, check_gather, check_same_query_topk,
    check_fp8_scale_hand, check_run_path_hand, check_step_topk_hand,
]
