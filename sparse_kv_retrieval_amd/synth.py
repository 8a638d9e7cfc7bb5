"""Seeded synthetic inputs for the LSA memory-indexer selection path.

This module only draws random numbers and lays them out in memory. It holds
none of the method's arithmetic: it never forms the low-rank query, the gates,
a score, a selection or a top-k. Both the CPU oracle (through the tests and the
bench's CPU leg) and the HIP path read what it makes, so it is the only thing
the two sides share.

What the pages fix and what is a stand-in
-----------------------------------------
The pages (FlashMemory-DeepSeek-V4 write-up, "3.1 Memory Indexer math") give
the shapes of the operation: a hidden state h_t of width d, a down-projection
W^DQ to rank r (r = 2048 in the hyper.ai digest, "Method"), an up-projection
W^IUQ to n_h indexer heads, head gates from W^w, and one frozen compressed index
key K_s per entry. They give no weights, no keys and no datasets. The sizes
below (d, n_h, d_h, N, k, the 4:1 compression that turns a token count into N)
are the workload definitions this build runs, not numbers from the pages.

The synthetic structure stands in for a trained indexer:

* h carries one "massive activation" channel, h[0] = KAPPA, the same for every
  sequence; all other channels are N(0, 1).
* Row 0 of W^DQ is C_SPIKE / KAPPA times a random unit vector a_l in R^r, so the
  latent c has a fixed component of length C_SPIKE along a_l.
* W^IUQ adds, for head j, a rank-one term alpha * pol_j * a_l (x) u_l, where u_l
  is a random unit vector in R^{d_h} and pol_j = +1 for the first half of the
  heads and -1 for the rest. Each head's query then points along pol_j * u_l
  with strength about Q_SPIKE.
* Row 0 of W^w is GATE_POS / KAPPA for positive-polarity heads and
  -GATE_NEG / KAPPA for the others, so positive heads get a gate near +GATE_POS
  and negative heads a gate near -GATE_NEG. Everything else is N(0, 1/fan_in).
* A fraction `planted` of each layer's keys (positions drawn per sequence and
  per layer) is sqrt(d_h) * (RHO * u_l + sqrt(1 - RHO^2) * z), where z is a
  unit vector orthogonal to u_l. The other keys are N(0, I).

With these values, about 99.9 % of planted keys and about 1 % of background keys
score I >= 0.5. The background rate stands in for the ~8.4 % leakage that the
write-up reports for context-independent queries ("6.1"). The native
Lightning-Indexer weights that drive the per-step top-k use the same
construction with independent noise, so they also favour planted keys.

Storage: bf16 values are uint16 bit patterns (round to nearest even), fp8 keys
are OCP e4m3fn bytes with one fp32 scale per entry, and weights are stored
"out x in" (row n of the W^DQ buffer is column n of W^DQ).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

KAPPA = 4.0        # value of the massive-activation channel h[0] (exact in bf16)
C_SPIKE = 8.0      # length of the fixed latent component along a_l
Q_SPIKE = 3.0      # per-head query strength along +-u_l
GATE_POS = 1.0     # mean gate of positive-polarity heads
GATE_NEG = 6.0     # mean gate magnitude of negative-polarity heads
RHO = 0.5          # cosine between a planted key and u_l

KEY_DTYPES = ("f32", "bf16", "fp8")


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtypes and the planting rule."""
    name: str
    wid: int                 # workload id, part of every seed
    B: int                   # sequences
    L: int                   # indexer layers
    d: int                   # hidden width
    r: int                   # inner rank of W^DQ
    n_h: int                 # indexer heads
    d_h: int                 # head dim = key dim
    key_dtype: str           # "f32" | "bf16" | "fp8"
    act_dtype: str           # "f32" | "bf16" (h and weights)
    k: int                   # top-k inside the subset
    N: tuple = ()            # entries per sequence (fixed lengths)
    ragged_tokens: tuple = ()  # (lo, hi) log-uniform token range, N = tokens // 4
    planted: float = 0.0     # planted fraction per layer; 0 = plain N(0,1) keys, no spikes
    random_init: bool = False  # indexer weights and h without the spikes (keys still planted)
    threshold: float = 0.5
    pool_dim: int = 512      # bf16 latent width of the compressed-KV pool rows
    seed: int = 0

    @property
    def structured(self) -> bool:
        return self.planted > 0.0


# The workloads this build runs (entry counts assume 4:1 CSA compression).
WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_f32", 0, B=1, L=1, d=256, r=64, n_h=4, d_h=32,
                 key_dtype="f32", act_dtype="f32", k=32, N=(1024,),
                 planted=0.0, pool_dim=64, seed=0),
        Workload("single_layer_500k", 1, B=1, L=1, d=4096, r=2048, n_h=64, d_h=128,
                 key_dtype="bf16", act_dtype="bf16", k=2048, N=(125_000,),
                 planted=0.135, seed=1),
        Workload("three_layer_b8", 2, B=8, L=3, d=4096, r=2048, n_h=64, d_h=128,
                 key_dtype="bf16", act_dtype="bf16", k=2048, N=(125_000,) * 8,
                 planted=0.05, seed=2),
        Workload("fp8_1m", 3, B=4, L=3, d=4096, r=2048, n_h=64, d_h=128,
                 key_dtype="fp8", act_dtype="bf16", k=2048, N=(250_000,) * 4,
                 planted=0.10, seed=3),
        Workload("ragged_b32", 4, B=32, L=3, d=4096, r=2048, n_h=64, d_h=128,
                 key_dtype="bf16", act_dtype="bf16", k=2048,
                 ragged_tokens=(16_384, 524_288), planted=0.05, seed=4),
        # one indexer layer being trained from random initialisation against frozen planted keys
        Workload("train_b8", 5, B=8, L=1, d=4096, r=2048, n_h=64, d_h=128,
                 key_dtype="bf16", act_dtype="bf16", k=2048, N=(125_000,) * 8,
                 planted=0.05, random_init=True, seed=5),
    )
}


def scaled(w: Workload, *, N=None, B=None, k=None, name=None) -> Workload:
    """A smaller copy of `w` with the same structure (for parity tests)."""
    changes = {}
    if B is not None:
        changes["B"] = B
    if N is not None:
        bb = changes.get("B", w.B)
        changes["N"] = tuple(N) if isinstance(N, (tuple, list)) else (int(N),) * bb
        changes["ragged_tokens"] = ()
        changes["B"] = len(changes["N"])
    elif B is not None and w.N:
        changes["N"] = (w.N[0],) * B
    if k is not None:
        changes["k"] = k
    changes["name"] = name or (w.name + "_scaled")
    return dataclasses.replace(w, **changes)


# ---------------------------------------------------------------- encodings
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 as OCP e4m3fn bytes (nearest even, saturating at +-448)."""
    import torch
    t = torch.from_numpy(np.clip(np.asarray(x, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- generator
def _rng(w: Workload, *tags) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, w.wid, *tags])))


def lengths(w: Workload) -> np.ndarray:
    """Entries per sequence (int64 [B])."""
    if w.N:
        assert len(w.N) == w.B
        return np.asarray(w.N, dtype=np.int64)
    lo, hi = w.ragged_tokens
    g = _rng(w, 900)
    toks = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=w.B))).astype(np.int64)
    return toks // 4


def _store_act(w: Workload, x: np.ndarray) -> np.ndarray:
    return x.astype(np.float32) if w.act_dtype == "f32" else f32_to_bf16_bits(x.astype(np.float32))


@dataclass
class LayerWeights:
    """One indexer layer's weights in "out x in" storage (f32 or bf16 bits)."""
    w_dq: np.ndarray    # [r, d]          = (W^DQ)^T
    w_iuq: np.ndarray   # [n_h*d_h, r]    = (W^IUQ)^T
    w_w: np.ndarray     # [n_h, d]        = (W^w)^T


@dataclass
class Inputs:
    workload: Workload
    lengths: np.ndarray            # int64 [B]
    key_offsets: np.ndarray        # int64 [B+1] rows
    mask_word_offsets: np.ndarray  # int64 [B+1] u64 words, region b = ceil(N_b/64) words
    h: list                        # per layer: [B, d] (f32 or bf16 bits)
    mem_w: list                    # per layer: LayerWeights (memory indexer)
    nat_w: list                    # per layer: LayerWeights (native Lightning Indexer)
    keys: list                     # per layer: [rows, d_h] (f32, bf16 bits, or e4m3fn bytes)
    key_scale: list                # per layer: [rows] f32 (fp8 only) else None
    pool: np.ndarray               # [rows, pool_dim] bf16 bits (compressed-KV latents)
    planted: list = dataclasses.field(default_factory=list)  # per layer: bool [rows]


def _layer_weights(w: Workload, g: np.random.Generator, a, u) -> LayerWeights:
    d, r, nh, dh = w.d, w.r, w.n_h, w.d_h
    wdq = g.standard_normal((r, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    wiuq = g.standard_normal((nh * dh, r), dtype=np.float32) * np.float32(1.0 / math.sqrt(r))
    ww = g.standard_normal((nh, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    if w.structured and not w.random_init:
        pol = np.where(np.arange(nh) < nh // 2, 1.0, -1.0)
        wdq[:, 0] = (C_SPIKE / KAPPA) * a
        alpha = Q_SPIKE / C_SPIKE
        # rank-one spike per head: column block j of W^IUQ gains alpha*pol_j * a (x) u
        spike = alpha * (pol[:, None] * u[None, :]).reshape(nh * dh)
        wiuq += np.outer(spike, a).astype(np.float32)
        ww[:, 0] = np.where(pol > 0, GATE_POS, -GATE_NEG) / KAPPA
    return LayerWeights(_store_act(w, wdq), _store_act(w, wiuq), _store_act(w, ww))


def _unit(g: np.random.Generator, n: int) -> np.ndarray:
    v = g.standard_normal(n)
    return v / np.linalg.norm(v)


def make(w: Workload, *, with_pool: bool = True) -> Inputs:
    """Generate every input of one workload, deterministically from its seed."""
    n = lengths(w)
    B, L, dh = w.B, w.L, w.d_h
    key_offsets = np.zeros(B + 1, np.int64)
    key_offsets[1:] = np.cumsum(n)
    words = (n + 63) // 64
    mwo = np.zeros(B + 1, np.int64)
    mwo[1:] = np.cumsum(words)
    rows = int(key_offsets[-1])

    hs, mem, nat, keys, scales, planted = [], [], [], [], [], []
    for l in range(L):
        gl = _rng(w, 1, l)
        a = _unit(gl, w.r)
        u = _unit(gl, dh)
        mem.append(_layer_weights(w, _rng(w, 2, l), a, u))
        nat.append(_layer_weights(w, _rng(w, 3, l), a, u))
        hl = np.empty((B, w.d), np.float32)
        for b in range(B):
            hl[b] = _rng(w, 4, l, b).standard_normal(w.d, dtype=np.float32)
        if w.structured and not w.random_init:
            hl[:, 0] = KAPPA
        hs.append(_store_act(w, hl))

        if w.key_dtype == "f32":
            kl = np.empty((rows, dh), np.float32)
        elif w.key_dtype == "bf16":
            kl = np.empty((rows, dh), np.uint16)
        else:
            kl = np.empty((rows, dh), np.uint8)
        sl = np.empty(rows, np.float32) if w.key_dtype == "fp8" else None
        pl = np.zeros(rows, bool)
        for b in range(B):
            g = _rng(w, 5, l, b)
            nb = int(n[b])
            kb = g.standard_normal((nb, dh), dtype=np.float32)
            if w.structured and nb > 0:
                m = int(round(w.planted * nb))
                pos = np.sort(g.choice(nb, size=m, replace=False))
                z = g.standard_normal((m, dh))
                z -= np.outer(z @ u, u)
                z /= np.linalg.norm(z, axis=1, keepdims=True)
                kb[pos] = (math.sqrt(dh) * (RHO * u[None, :] + math.sqrt(1 - RHO * RHO) * z)).astype(np.float32)
                pl[key_offsets[b] + pos] = True
            s0, s1 = key_offsets[b], key_offsets[b + 1]
            if w.key_dtype == "f32":
                kl[s0:s1] = kb
            elif w.key_dtype == "bf16":
                kl[s0:s1] = f32_to_bf16_bits(kb)
            else:
                amax = np.abs(kb).max(axis=1) if nb else np.zeros(0, np.float32)
                sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
                kl[s0:s1] = f32_to_e4m3fn_bits(kb / sc[:, None])
                sl[s0:s1] = sc
        keys.append(kl)
        scales.append(sl)
        planted.append(pl)

    pool = None
    if with_pool:
        pool = np.empty((rows, w.pool_dim), np.uint16)
        for b in range(B):
            g = _rng(w, 6, b)
            pool[key_offsets[b]:key_offsets[b + 1]] = g.integers(
                0, 1 << 16, size=(int(n[b]), w.pool_dim), dtype=np.uint16)
    return Inputs(w, n, key_offsets, mwo, hs, mem, nat, keys, scales, pool, planted)


# ---------------------------------------------------------------- decode steps
def step_hidden(inp: Inputs, steps: int) -> list:
    """Hidden states of `steps` decode steps after the trigger: [step][layer] -> [B, d].

    Each step's h is drawn like the trigger's (the massive-activation channel
    plus N(0, 1) noise), from its own seed, and stored in the workload's
    activation dtype. They feed the native indexer's per-step query."""
    w = inp.workload
    out = []
    for t in range(steps):
        per = []
        for l in range(w.L):
            hl = np.empty((w.B, w.d), np.float32)
            for b in range(w.B):
                hl[b] = _rng(w, 8, t, l, b).standard_normal(w.d, dtype=np.float32)
            if w.structured and not w.random_init:
                hl[:, 0] = KAPPA
            per.append(_store_act(w, hl))
        out.append(per)
    return out


# ---------------------------------------------------------------- training labels
def pack_mask_words(bits: np.ndarray, key_offsets: np.ndarray, mask_word_offsets: np.ndarray) -> np.ndarray:
    """Lay out per-entry booleans [rows] as the selection path's u64 mask words.

    Entry s of sequence b is bit s % 64 of word mask_word_offsets[b] + s // 64;
    bits past N_b are 0."""
    B = len(key_offsets) - 1
    out = np.zeros(int(mask_word_offsets[-1]), np.uint64)
    for b in range(B):
        s0, s1 = int(key_offsets[b]), int(key_offsets[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        padded = np.zeros(((n + 63) // 64) * 64, np.uint8)
        padded[:n] = bits[s0:s1]
        words = np.packbits(padded, bitorder="little").view(np.uint64)
        out[int(mask_word_offsets[b]):int(mask_word_offsets[b + 1])] = words
    return out


def train_labels(inp: Inputs, layer: int = 0, flip: float = 0.02):
    """Golden labels for a training step on one layer's keys.

    The labels are the layer's planted entries (the keys the structured indexer
    is built to favour), with a fraction `flip` of all entries toggled at random
    so that both classes hold entries the current weights get wrong. Returns
    (bool [rows], u64 mask words in the selection path's layout)."""
    w = inp.workload
    rows = int(inp.key_offsets[-1])
    g = _rng(w, 7, layer)
    lab = inp.planted[layer].copy() if inp.planted else np.zeros(rows, bool)
    lab ^= g.random(rows) < flip
    return lab, pack_mask_words(lab, inp.key_offsets, inp.mask_word_offsets)
