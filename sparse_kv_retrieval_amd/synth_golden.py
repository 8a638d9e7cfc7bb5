"""Seeded synthetic indexer logits for golden-label mining.

This module only draws random numbers and lays them out in memory: it forms no
softmax, nucleus, vote or union. The CPU oracle (through the tests and the
bench's CPU leg) and the HIP path both read what it makes.

The pages describe the inputs of the label step (the hyper.ai digest,
"数据集", and the marsggbo write-up, §4.1): for each token of a lookahead
window of tau tokens, the raw indexer logits of every one of the 21 CSA layers
over the compressed entries that precede the token. The backbone that produces
them is not available, so the logits here are a stand-in with the structure
the method is meant to denoise:

* Token i of the window sees n_valid[i] = N0 + i // 4 entries (one compressed
  entry per 4 tokens, the CSA compression this build assumes elsewhere).
* Background: y = SIGMA_BG * z with z ~ N(0, 1), independent per token, layer
  and entry.
* A set R of R_SIZE entries that the whole window needs, each with a strength
  a_s ~ U(A_LO, A_HI); in each (token, layer) row an entry of R is active with
  probability P_ON and then adds a_s to its logit. Every token also has OWN
  entries of its own, drawn from its prefix, under the same rule.
* Single-layer noise: SPUR entries per (token, layer) row, at uniform positions,
  add U(A_LO, A_HI). One layer alone cannot make them golden.
* Rows are stored with a stride of row_stride floats (a multiple of 64); the
  slots at or beyond n_valid[i] hold PAD, a value that would dominate any
  softmax it entered, so reading past the prefix cannot go unnoticed.

With the defaults, about half the layers' nuclei are entries of R or OWN, the
vote keeps a few hundred entries per token and the window's label set has a few
hundred to a thousand entries: the range the digest reports after denoising
(100 to 1,000 positives per window, down from about 10,000).

Variants for edge cases: `quantum` rounds every logit to a multiple of it
(many exact ties); `mode="flat"` makes every logit equal; `mode="narrow"` puts
every logit inside one narrow interval (more entries share the crossing region
than any fixed-size candidate list holds).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SIGMA_BG = 1.0
A_LO, A_HI = 6.0, 10.0
P_ON = 0.6
PAD = 1.0e4


@dataclass(frozen=True)
class GoldenWorkload:
    name: str
    wid: int
    T: int                   # tokens in the window (tau)
    L: int                   # layers voting
    N0: int                  # entries seen by the window's first token
    p: float = 0.6
    theta: int = 3
    r_size: int = 512
    own: int = 8
    spur: int = 16
    quantum: float = 0.0
    mode: str = "mix"        # "mix" | "flat" | "narrow"
    n_valid: tuple = ()      # explicit per-token prefixes (overrides N0 + i // 4)
    seed: int = 0

    def prefixes(self) -> np.ndarray:
        if self.n_valid:
            assert len(self.n_valid) == self.T
            return np.asarray(self.n_valid, dtype=np.int32)
        return (self.N0 + np.arange(self.T) // 4).astype(np.int32)

    @property
    def row_stride(self) -> int:
        n = int(max(1, self.prefixes().max()))
        return (n + 63) // 64 * 64

    @property
    def words(self) -> int:
        return self.row_stride // 64


WORKLOADS = {
    w.name: w
    for w in (
        # one lookahead window: 64 tokens x 21 layers x 125K entries (a 500K-token context at 4:1)
        GoldenWorkload("golden_t64_l21_n125k", 10, T=64, L=21, N0=125_000, seed=10),
        GoldenWorkload("golden_small", 11, T=8, L=5, N0=3_000, r_size=64, own=4, spur=8, seed=11),
        GoldenWorkload("golden_ragged", 12, T=6, L=4, N0=0,
                       n_valid=(0, 1, 2, 63, 64, 5_000), r_size=32, own=2, spur=4, seed=12),
        GoldenWorkload("golden_ties", 13, T=4, L=5, N0=2_000, quantum=0.5, r_size=64, own=4, spur=8, seed=13),
        GoldenWorkload("golden_flat", 14, T=2, L=3, N0=10_000, mode="flat", seed=14),
        GoldenWorkload("golden_narrow", 15, T=2, L=3, N0=20_000, mode="narrow", seed=15),
    )
}


def _rng(w: GoldenWorkload, *tags) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, w.wid, *tags])))


@dataclass
class GoldenInputs:
    workload: GoldenWorkload
    logits: np.ndarray       # float32 [T, L, row_stride]
    n_valid: np.ndarray      # int32 [T]


def make(w: GoldenWorkload) -> GoldenInputs:
    T, L, S = w.T, w.L, w.row_stride
    n = w.prefixes()
    y = np.full((T, L, S), PAD, dtype=np.float32)
    g = _rng(w, 0)
    if w.mode == "flat":
        for i in range(T):
            y[i, :, :n[i]] = 1.5
        return GoldenInputs(w, y, n)
    if w.mode == "narrow":
        for i in range(T):
            y[i, :, :n[i]] = (1.0 + g.uniform(0.0, 0.1, size=(L, int(n[i])))).astype(np.float32)
        return GoldenInputs(w, y, n)
    n0 = int(max(1, n.min()))
    R = g.choice(n0, size=min(w.r_size, n0), replace=False)
    aR = g.uniform(A_LO, A_HI, size=R.size)
    for i in range(T):
        ni = int(n[i])
        if ni == 0:
            continue
        gi = _rng(w, 1, i)
        row = gi.standard_normal(size=(L, ni), dtype=np.float32) * np.float32(SIGMA_BG)
        own = gi.choice(ni, size=min(w.own, ni), replace=False)
        a_own = gi.uniform(A_LO, A_HI, size=own.size)
        ids = np.concatenate([R[R < ni], own])
        amp = np.concatenate([aR[R < ni], a_own])
        on = gi.random(size=(L, ids.size)) < P_ON
        for l in range(L):
            np.add.at(row[l], ids[on[l]], amp[on[l]].astype(np.float32))
            sp = gi.integers(0, ni, size=w.spur)
            np.add.at(row[l], sp, gi.uniform(A_LO, A_HI, size=w.spur).astype(np.float32))
        if w.quantum:
            row = (np.round(row / w.quantum) * w.quantum).astype(np.float32)
        y[i, :, :ni] = row
    return GoldenInputs(w, y, n)
