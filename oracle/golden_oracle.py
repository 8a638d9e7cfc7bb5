"""CPU oracle for golden-label mining (TEST INFRASTRUCTURE ONLY).

Plain, slow float64 reference for the label-mining step that produces the
indexer's training targets. Only the tests, the smoke check and the CPU
baseline of bench.py may import it; the product path never does, and it
shares no code with the HIP library.

Sources (section names of the pages):
  [HYPER] hyper.ai digest of FlashMemory-DeepSeek-V4, section "数据集"
          (Dataset): the three-step denoising (softmax of the raw indexer
          logits, a 0.6 nucleus threshold, a cross-layer majority vote over
          all 21 CSA layers with at least three layers agreeing) and the
          window construction (per-token golden sets, then a union over the
          future window of tau tokens).
  [BLOG]  marsggbo.github.io write-up, §4.1 "Golden Label 怎么造": for every
          token i in [t, t+tau-1], the raw indexer logits of the 21 CSA layers;
          per layer softmax + top-p (p = 0.6) instead of a fixed top-k; an
          entry is golden if at least 3 layers select it; the union over the
          window is the positive set.
  [GIST]  gist.science summary, §2.2 "Curadoria de Dados e Rotulagem": softmax
          normalisation, top-p thresholding (p = 0.6) per layer, majority vote
          with theta = 3 of L layers.

Readings where the pages leave a step open (also listed with the design
notes):
  G1  The inputs are the raw per-layer indexer logits y[i][l][s] of token i
      over the compressed entries s that precede it. Token i sees the prefix
      s < n[i] of the entries (the window's later tokens see a few more).
  G2  Softmax over that prefix, per (token, layer).
  G3  Top-p is the nucleus: the shortest prefix of the entries, ordered by
      descending probability, whose cumulative probability reaches p
      (inclusive: the entry that makes the sum reach p is kept).
  G4  Ties in probability are ordered by the lower entry index first, as in
      the native top-k order (-y, s).
  G5  Entry s is golden for token i when at least theta layers keep it.
  G6  The label set of the window is the union (OR) of the tokens' golden
      sets. Defaults: tau = 64 tokens, 21 layers, p = 0.6, theta = 3.
"""
from __future__ import annotations

import numpy as np


def softmax(y: np.ndarray) -> np.ndarray:
    """Probabilities of a 1-D logit vector (float64, max subtracted first)."""
    y = np.asarray(y, dtype=np.float64)
    e = np.exp(y - y.max())
    return e / e.sum()


def nucleus_order(y: np.ndarray) -> np.ndarray:
    """Entry indices by descending logit, equal logits by ascending index (G4)."""
    y = np.asarray(y, dtype=np.float64)
    return np.lexsort((np.arange(y.size), -y))


def nucleus(y: np.ndarray, p: float) -> np.ndarray:
    """Boolean mask of the top-p nucleus of one (token, layer) row (G2, G3, G4).

    An entry is kept when the probability mass of the entries before it in the
    nucleus order is still below p; the first entry is always kept.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.size, dtype=bool)
    if y.size == 0:
        return out
    P = softmax(y)
    order = nucleus_order(y)
    before = np.concatenate(([0.0], np.cumsum(P[order])[:-1]))
    out[order[before < p]] = True
    return out


def nucleus_bounds(y: np.ndarray, p: float, eps: float):
    """(sure_in, sure_out) masks for a comparison with a tolerance on the mass.

    An entry whose preceding mass lies within eps of p may go either way under
    rounding; it is in neither mask. Everything else is decided.
    """
    y = np.asarray(y, dtype=np.float64)
    sure_in = np.zeros(y.size, dtype=bool)
    sure_out = np.zeros(y.size, dtype=bool)
    if y.size == 0:
        return sure_in, sure_out
    P = softmax(y)
    order = nucleus_order(y)
    before = np.concatenate(([0.0], np.cumsum(P[order])[:-1]))
    sure_in[order[before < p - eps]] = True
    sure_out[order[before >= p + eps]] = True
    sure_in[order[0]] = True  # the top entry is always kept
    sure_out[order[0]] = False
    return sure_in, sure_out


def votes(rows: np.ndarray, n: int, p: float) -> np.ndarray:
    """Layer votes per entry for one token: rows[l] are its logits, prefix n (G5)."""
    rows = np.asarray(rows, dtype=np.float64)
    v = np.zeros(n, dtype=np.int64)
    for l in range(rows.shape[0]):
        v += nucleus(rows[l, :n], p)
    return v


def golden_labels(logits: np.ndarray, n_valid, p: float = 0.6, theta: int = 3) -> np.ndarray:
    """Union over the window's tokens of the entries kept by >= theta layers (G1-G6).

    logits: [T, L, N] raw indexer logits (rows may be longer than n_valid[i]).
    Returns a bool mask over max(n_valid) entries.
    """
    logits = np.asarray(logits)
    T = logits.shape[0]
    N = int(max(n_valid)) if T else 0
    out = np.zeros(N, dtype=bool)
    for i in range(T):
        n = int(n_valid[i])
        out[:n] |= votes(logits[i], n, p) >= theta
    return out


def golden_bounds(logits: np.ndarray, n_valid, p: float, theta: int, eps: float):
    """(sure_golden, sure_not): the union's entries decided whatever the rounding.

    Per token, the vote count of an entry lies between the number of layers
    that surely keep it and the number that may keep it.
    """
    logits = np.asarray(logits)
    T, L = logits.shape[0], logits.shape[1]
    N = int(max(n_valid)) if T else 0
    sure_g = np.zeros(N, dtype=bool)
    maybe_g = np.zeros(N, dtype=bool)
    for i in range(T):
        n = int(n_valid[i])
        lo = np.zeros(n, dtype=np.int64)
        hi = np.zeros(n, dtype=np.int64)
        for l in range(L):
            si, so = nucleus_bounds(logits[i, l, :n], p, eps)
            lo += si
            hi += ~so
        sure_g[:n] |= lo >= theta
        maybe_g[:n] |= hi >= theta
    return sure_g, ~maybe_g


def nucleus_sizes(logits: np.ndarray, n_valid, p: float) -> np.ndarray:
    """[T, L] number of entries in each row's nucleus."""
    logits = np.asarray(logits)
    T, L = logits.shape[0], logits.shape[1]
    out = np.zeros((T, L), dtype=np.int64)
    for i in range(T):
        for l in range(L):
            out[i, l] = int(nucleus(logits[i, l, :int(n_valid[i])], p).sum())
    return out
