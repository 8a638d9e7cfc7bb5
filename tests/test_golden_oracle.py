"""Pins of the golden-label oracle (CPU), and plausible mistakes each caught by a pin."""
import types

import numpy as np
import pytest

from oracle import golden_oracle as G
from tests import golden_checks as C


@pytest.mark.parametrize("check", C.ALL, ids=lambda f: f.__name__)
def test_golden_oracle_pin(check):
    check(G)


def _clone():
    m = types.ModuleType("golden_mutant")
    m.__dict__.update({k: v for k, v in G.__dict__.items() if not k.startswith("__")})
    return m


def _nucleus_with(keep):
    """A nucleus that decides membership with keep(before, cum, p)."""
    def nucleus(y, p):
        y = np.asarray(y, np.float64)
        out = np.zeros(y.size, bool)
        if y.size == 0:
            return out
        e = np.exp(y - y.max())
        P = e / e.sum()
        order = np.lexsort((np.arange(y.size), -y))
        cum = np.cumsum(P[order])
        before = np.concatenate(([0.0], cum[:-1]))
        out[order[keep(before, cum, p)]] = True
        return out
    return nucleus


def _mut_stop_before_crossing(m):  # keeps only entries whose own running sum stays below p
    m.nucleus = _nucleus_with(lambda before, cum, p: cum < p)


def _mut_one_past(m):  # keeps one entry more than needed
    m.nucleus = _nucleus_with(lambda before, cum, p: np.concatenate(([True], before[:-1] < p)))


def _mut_ties_high_index(m):
    def nucleus(y, p):
        y = np.asarray(y, np.float64)
        out = np.zeros(y.size, bool)
        e = np.exp(y - y.max())
        P = e / e.sum()
        order = np.lexsort((-np.arange(y.size), -y))
        before = np.concatenate(([0.0], np.cumsum(P[order])[:-1]))
        out[order[before < p]] = True
        return out
    m.nucleus = nucleus


def _mut_ascending(m):
    orig = G.nucleus
    m.nucleus = lambda y, p: orig(-np.asarray(y, np.float64), p)


def _mut_unnormalised(m):  # probabilities relative to the largest instead of the sum
    def nucleus(y, p):
        y = np.asarray(y, np.float64)
        out = np.zeros(y.size, bool)
        P = np.exp(y - y.max())
        order = np.lexsort((np.arange(y.size), -y))
        before = np.concatenate(([0.0], np.cumsum(P[order])[:-1]))
        out[order[before < p]] = True
        return out
    m.nucleus = nucleus


def _mut_strict_vote(m):
    orig = G.votes
    m.votes = lambda rows, n, p: orig(rows, n, p) - 1


def _mut_whole_row(m):  # ignores the token's prefix
    def votes(rows, n, p):
        rows = np.asarray(rows, np.float64)
        v = np.zeros(rows.shape[1], np.int64)
        for l in range(rows.shape[0]):
            v += m.nucleus(rows[l], p)
        return v[:n]
    m.votes = votes


def _mut_intersection(m):
    def golden_labels(logits, n_valid, p=0.6, theta=3):
        logits = np.asarray(logits)
        N = int(max(n_valid))
        out = np.ones(N, bool)
        for i in range(logits.shape[0]):
            g = np.zeros(N, bool)
            g[:n_valid[i]] = m.votes(logits[i], n_valid[i], p) >= theta
            out &= g
        return out
    m.golden_labels = golden_labels


def _bounds_with(inside, outside, top=True):
    def nucleus_bounds(y, p, eps):
        y = np.asarray(y, np.float64)
        si, so = np.zeros(y.size, bool), np.zeros(y.size, bool)
        if y.size == 0:
            return si, so
        e = np.exp(y - y.max())
        P = e / e.sum()
        order = np.lexsort((np.arange(y.size), -y))
        before = np.concatenate(([0.0], np.cumsum(P[order])[:-1]))
        si[order[inside(before, p, eps)]] = True
        so[order[outside(before, p, eps)]] = True
        if top:
            si[order[0]], so[order[0]] = True, False
        return si, so
    return nucleus_bounds


def _mut_bounds_eps_sign(m):  # the band on the wrong side: decides entries it should leave open
    m.nucleus_bounds = _bounds_with(lambda b, p, e: b < p + e, lambda b, p, e: b >= p - e)


def _mut_bounds_no_top(m):  # forgets that the most probable entry is always kept
    m.nucleus_bounds = _bounds_with(lambda b, p, e: b < p - e, lambda b, p, e: b >= p + e, top=False)


def _golden_bounds_with(hi_from_sure_in=False, strict=False):
    def golden_bounds(logits, n_valid, p, theta, eps):
        logits = np.asarray(logits)
        T, L = logits.shape[0], logits.shape[1]
        N = int(max(n_valid))
        sure_g, maybe_g = np.zeros(N, bool), np.zeros(N, bool)
        for i in range(T):
            n = int(n_valid[i])
            lo, hi = np.zeros(n, np.int64), np.zeros(n, np.int64)
            for l in range(L):
                si, so = m_ref.nucleus_bounds(logits[i, l, :n], p, eps)
                lo += si
                hi += si if hi_from_sure_in else ~so
            sure_g[:n] |= (lo > theta) if strict else (lo >= theta)
            maybe_g[:n] |= hi >= theta
        return sure_g, ~maybe_g
    m_ref = G
    return golden_bounds


def _mut_golden_bounds_maybe_from_sure(m):  # "may be golden" counted from the sure votes only
    m.golden_bounds = _golden_bounds_with(hi_from_sure_in=True)


def _mut_golden_bounds_strict(m):
    m.golden_bounds = _golden_bounds_with(strict=True)


MUTATIONS = [_mut_stop_before_crossing, _mut_one_past, _mut_ties_high_index, _mut_ascending, _mut_unnormalised,
             _mut_strict_vote, _mut_whole_row, _mut_intersection, _mut_bounds_eps_sign, _mut_bounds_no_top,
             _mut_golden_bounds_maybe_from_sure, _mut_golden_bounds_strict]


@pytest.mark.parametrize("mut", MUTATIONS, ids=lambda f: f.__name__)
def test_golden_mutation_is_caught(mut):
    m = _clone()
    mut(m)
    failed = []
    for check in C.ALL:
        try:
            check(m)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"{mut.__name__} passed every pin"
