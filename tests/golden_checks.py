"""Checks that pin the golden-label oracle to things other than itself.

Each `check_*` takes the oracle module (or a copy with a planted mistake) and
raises AssertionError when it disagrees with an independent fact: the
hand-worked cases in tests/golden/golden_labels_hand.json, brute force over
subsets of tiny rows, closed forms and invariances of the softmax nucleus, and
set identities of the vote and the window union.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_hand():
    with open(os.path.join(GOLDEN, "golden_labels_hand.json")) as f:
        return json.load(f)


def check_hand_nucleus(G):
    for row in load_hand()["rows"]:
        y = np.array(row["logits"])
        for c in row["cases"]:
            got = np.flatnonzero(G.nucleus(y, c["p"])).tolist()
            assert got == c["nucleus"], (row["what"], c["p"], got, c["nucleus"])


def check_hand_window(G):
    w = load_hand()["window"]
    L = np.array(w["logits"])
    for i, n in enumerate(w["n_valid"]):
        assert G.votes(L[i], n, w["p"]).tolist() == w["votes"][i], (i, G.votes(L[i], n, w["p"]))
    for th, exp in w["golden"].items():
        got = np.flatnonzero(G.golden_labels(L, w["n_valid"], w["p"], int(th))).tolist()
        assert got == exp, (th, got, exp)


def _probs(y):
    e = np.exp(np.asarray(y, np.float64) - np.max(y))
    return e / e.sum()


def check_nucleus_brute_force(G, seeds=range(40)):
    """Tiny rows: the nucleus is the smallest set of entries reaching mass p, made of
    the most probable entries, ties by lower index (checked over all subsets)."""
    for seed in seeds:
        rng = np.random.default_rng(seed)
        n = int(rng.integers(1, 8))
        y = np.round(rng.normal(0, 1.5, n) * 2) / 2  # a half-step grid makes ties common
        P = _probs(y)
        for p in (0.3, 0.6, 0.9):
            # skip rows where some subset sum lies within 1e-9 of p (rounding would decide)
            sums = [sum(P[list(c)]) for k in range(1, n + 1) for c in itertools.combinations(range(n), k)]
            if any(abs(s - p) < 1e-9 for s in sums):
                continue
            kmin = next(k for k in range(1, n + 1)
                        if max(sum(P[list(c)]) for c in itertools.combinations(range(n), k)) >= p)
            got = G.nucleus(y, p)
            S = np.flatnonzero(got)
            assert S.size == kmin, (seed, p, S, kmin)
            assert P[S].sum() >= p
            out = np.flatnonzero(~got)
            for a in S:
                for b in out:
                    assert y[a] > y[b] or (y[a] == y[b] and a < b), (seed, p, a, b)


def check_nucleus_closed_forms(G):
    # uniform logits: ceil(p n) entries, the lowest indices
    for n, p, k in ((10, 0.55, 6), (10, 0.61, 7), (7, 0.6, 5), (1, 0.6, 1), (100, 0.005, 1)):
        got = G.nucleus(np.full(n, 3.25), p)
        assert np.flatnonzero(got).tolist() == list(range(k)), (n, p, np.flatnonzero(got))
    # one entry above p alone
    y = np.array([0.0, 0.0, 9.0, 0.0])
    assert np.flatnonzero(G.nucleus(y, 0.6)).tolist() == [2]
    # adding a constant to every logit changes nothing (softmax is shift invariant)
    rng = np.random.default_rng(11)
    y = rng.normal(0, 2, 300)
    for p in (0.2, 0.6, 0.95):
        assert np.array_equal(G.nucleus(y, p), G.nucleus(y + 37.5, p))
    # scaling the logits up concentrates the mass: the nucleus can only shrink
    for p in (0.3, 0.6, 0.9):
        assert G.nucleus(y * 3, p).sum() <= G.nucleus(y, p).sum()
    # p close to 1 keeps every entry; the mass of the kept entries always reaches p
    assert G.nucleus(y, 1.0 - 1e-12).all()
    for p in (0.1, 0.6, 0.99):
        m = G.nucleus(y, p)
        assert _probs(y)[m].sum() >= p
        # and without its least probable member it would not
        P = _probs(y)
        assert P[m].sum() - P[m].min() < p


def check_votes_union(G):
    rng = np.random.default_rng(5)
    T, L, N = 4, 5, 60
    logits = rng.normal(0, 2.5, (T, L, N))
    n_valid = [45, 50, 55, 60]
    nuc = [[G.nucleus(logits[i, l, :n_valid[i]], 0.6) for l in range(L)] for i in range(T)]
    # theta = 1: the union of every nucleus; theta > L: nothing
    u = np.zeros(N, bool)
    for i in range(T):
        for l in range(L):
            u[:n_valid[i]] |= nuc[i][l]
    assert np.array_equal(G.golden_labels(logits, n_valid, 0.6, 1), u)
    assert not G.golden_labels(logits, n_valid, 0.6, L + 1).any()
    # the window's set is the union of the tokens' sets, and each token's votes count layers
    for th in (2, 3):
        per = np.zeros((T, N), bool)
        for i in range(T):
            v = sum(nuc[i][l].astype(int) for l in range(L))
            assert np.array_equal(G.votes(logits[i], n_valid[i], 0.6), v)
            per[i, :n_valid[i]] = v >= th
        assert np.array_equal(G.golden_labels(logits, n_valid, 0.6, th), per.any(axis=0))
    # a token never labels entries beyond its prefix
    g = G.golden_labels(logits[:1], [20], 0.6, 1)
    assert g.size == 20


def _bounds_by_definition(y, p, eps):
    """sure_in / sure_out of one row, from a plain loop: entries in (-y, s) order, each with the
    exact-order running mass before it; the first entry is always kept."""
    y = [float(v) for v in y]
    P = _probs(np.array(y)) if y else np.zeros(0)
    order = sorted(range(len(y)), key=lambda s: (-y[s], s))
    sure_in, sure_out = np.zeros(len(y), bool), np.zeros(len(y), bool)
    before = 0.0
    for rank, s in enumerate(order):
        sure_in[s] = rank == 0 or before < p - eps
        sure_out[s] = rank > 0 and before >= p + eps
        before += P[s]
    return sure_in, sure_out


def check_bounds_at_zero_eps(G):
    """With no tolerance the bounds are the nucleus and its complement, and the window bounds
    are the label set and its complement."""
    rng = np.random.default_rng(21)
    for n in (1, 2, 7, 50, 333):
        y = np.round(rng.normal(0, 2, n) * 2) / 2
        for p in (0.05, 0.6, 0.97):
            si, so = G.nucleus_bounds(y, p, 0.0)
            nuc = G.nucleus(y, p)
            assert np.array_equal(si, nuc) and np.array_equal(so, ~nuc), (n, p)
    T, L, N = 3, 4, 40
    logits = np.round(rng.normal(0, 2, (T, L, N)) * 2) / 2
    nv = [30, 35, 40]
    for th in (1, 2, 3, 5):
        sg, sn = G.golden_bounds(logits, nv, 0.6, th, 0.0)
        gl = G.golden_labels(logits, nv, 0.6, th)
        assert np.array_equal(sg, gl) and np.array_equal(sn, ~gl), th


def check_bounds_definition(G):
    """With a tolerance, against the definition written as loops: per row, the entries surely in
    or out of the nucleus; per window, an entry is surely golden when some token has at least
    theta layers that surely keep it, and surely not when no token has theta layers that may."""
    rng = np.random.default_rng(22)
    for trial in range(30):
        n = int(rng.integers(1, 12))
        y = np.round(rng.normal(0, 1.2, n) * 2) / 2
        for p in (0.05, 0.3, 0.6, 0.9):
            for eps in (0.02, 0.1):
                si, so = G.nucleus_bounds(y, p, eps)
                wi, wo = _bounds_by_definition(y, p, eps)
                assert np.array_equal(si, wi) and np.array_equal(so, wo), (trial, p, eps, y)
                nuc = G.nucleus(y, p)
                assert not (si & ~nuc).any() and not (so & nuc).any()
    T, L, N = 4, 5, 9
    logits = np.round(rng.normal(0, 1.2, (T, L, N)) * 2) / 2
    nv = [6, 7, 9, 9]
    for th in (1, 2, 3):
        for eps in (0.03, 0.1):
            sg, sn = G.golden_bounds(logits, nv, 0.6, th, eps)
            want_g, maybe = np.zeros(N, bool), np.zeros(N, bool)
            for i in range(T):
                lo, hi = np.zeros(N, int), np.zeros(N, int)
                for l in range(L):
                    wi, wo = _bounds_by_definition(logits[i, l, :nv[i]], 0.6, eps)
                    lo[:nv[i]] += wi
                    hi[:nv[i]] += ~wo
                want_g |= lo >= th
                maybe |= hi >= th
            assert np.array_equal(sg, want_g) and np.array_equal(sn, ~maybe), (th, eps)


ALL = [check_hand_nucleus, check_hand_window, check_nucleus_brute_force, check_nucleus_closed_forms,
       check_votes_union, check_bounds_at_zero_eps, check_bounds_definition]
