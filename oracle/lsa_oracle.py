"""CPU oracle for the LSA memory-indexer selection path (TEST INFRASTRUCTURE ONLY).

This is a plain, slow implementation that is meant to be obviously correct. It
exists only to check the HIP library. The only code allowed to import it is the
tests, the smoke check in `__graft_entry__` and the CPU-baseline leg of
`bench.py`. The product path never calls it. It shares no code with the HIP
path: it has its own dtype decoding, its own projection and its own selection
logic. All arithmetic is float64 on the stored input values.

Sources. Section names refer to these pages:
  [BLOG]  "arXiv'26 | FlashMemory-DeepSeek-V4: 用 13.5% 的显存干 100% 的活,
          超长上下文推理的 less is more" (marsggbo.github.io). The formulas are
          in §3.1 "Memory Indexer 的数学", in order: the down-projection
          c = h W^DQ, the up-projection q = c W^IUQ, the head-routing weights
          w = h W^w, the lookahead index score I, and the rule that entries
          with I >= 0.5 are loaded. §2.2 describes the native Lightning Indexer
          (inner product, ReLU, top-k). §3.2 describes the two-level selection.
          §4.2 covers the three indexer layers and OR-mode routing.
  [HYPER] hyper.ai digest "FlashMemory-DeepSeek-V4 …", section "方法" (Method):
          threshold "reach or exceed 0.5", load C^MemComp, native top-k inside
          it, and OR-union over layers 10/12/20.
  [GIST]  gist.science "Resumo Técnico: FlashMemory-DeepSeek-V4 via Lookahead
          Sparse Attention", §2.1 (I >= 0.5 fetch; top-k inside the subset)
          and §2.4 (OR union).

Readings where the pages leave a step open, numbered as in the design notes'
list (R10-R14 there are about the GPU side and the workloads).
  R1  The per-head ReLU stays inside the sum and the sigmoid wraps the head sum
      ([BLOG] §3.1 score formula). The threshold replaces the native top-k.
  R2  The gates are linear: w = h W^w, with no softmax and no 1/sqrt scale.
  R3  Each layer has its own W^DQ, W^IUQ, W^w and its own h.
  R4  There is one key per entry per layer, shared by all heads (K_s has no head
      index).
  R5  Selection is inclusive: I >= theta. Because sigma is strictly increasing,
      this is tested as x >= ln(theta/(1-theta)), so the sigmoid's rounding
      never decides membership. With theta = 0.5 the test is x >= 0.
  R6  The top-k score is the native Lightning-Indexer form, with no sigmoid
      ([BLOG] §2.2). The order is (-y, s): ties go to the lower entry index.
      With fewer than k candidates, all are kept. The output is ascending.
  R7  The compacted list is in ascending entry order.
  R8  For fp8 keys, K_s = scale_s * e4m3fn(K8_s). Scales are positive, so the
      scale commutes with the ReLU.
  R15 At every decode step after a trigger, the native indexer's own query for
      that step (its projections of the step's hidden state) ranks the entries
      of the subset loaded at the trigger, with that layer's keys ([BLOG] §3.2
      second level; [HYPER] 方法). The subset is an input of the step.
"""
from __future__ import annotations

import math

import numpy as np

# ------------------------------------------------------------------ decoding


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly.

    A bfloat16 value is the upper half of an IEEE float32, so the pattern is
    shifted into the high 16 bits and reinterpreted.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(byte: int) -> float:
    """Value of one OCP FP8 E4M3 ("fn") byte, from the format's definition.

    The layout is 1 sign bit, 4 exponent bits (bias 7) and 3 mantissa bits.
    Exponent field 0 gives subnormals m/8 * 2^(1-7). The all-ones exponent
    field is used for normal numbers, except S.1111.111, which is NaN. There
    are no infinities.
    """
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(i) for i in range(256)], dtype=np.float64)


def e4m3fn_to_f64(bytes_: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(bytes_, dtype=np.uint8)]


def decode_act(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored activation/weight values -> float64 ("f32" or "bf16" bits)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(x)
    raise ValueError(dtype)


def decode_keys(keys: np.ndarray, dtype: str, scale=None) -> np.ndarray:
    """Stored keys -> float64 K (R8 for fp8: K = scale * e4m3fn(K8))."""
    if dtype == "fp8":
        return e4m3fn_to_f64(keys) * np.asarray(scale, np.float32).astype(np.float64)[:, None]
    v = decode_act(keys, dtype)
    assert np.all(np.isfinite(v)), "keys must be finite"
    return v


# ------------------------------------------------------------- the method


def project(h, w_dq, w_iuq, w_w, n_h: int, d_h: int):
    """Indexer query and gates for one layer ([BLOG] §3.1, the three projections).

    All inputs are float64 here. The weight buffers use the "out x in" layout,
    so W^DQ = w_dq.T, W^IUQ = w_iuq.T and W^w = w_w.T.
      c = h W^DQ                  [B, r]
      q = c W^IUQ, viewed [B, n_h, d_h] (head j = columns j*d_h ... (j+1)*d_h-1)
      w = h W^w                   [B, n_h]
    """
    h = np.atleast_2d(h)
    c = h @ w_dq.T
    q = (c @ w_iuq.T).reshape(h.shape[0], n_h, d_h)
    w = h @ w_w.T
    return c, q, w


def logits(q: np.ndarray, w: np.ndarray, K: np.ndarray) -> np.ndarray:
    """x_s = sum_j w_j * ReLU(q_j . K_s) for one (sequence, layer).

    This is the argument of the sigmoid in the lookahead index score
    ([BLOG] §3.1). It is also the native Lightning-Indexer score ([BLOG] §2.2),
    which is the same head-gated ReLU sum with no sigmoid. Shapes: q [n_h, d_h],
    w [n_h], K [N, d_h] -> x [N].
    """
    dots = K @ q.T                      # [N, n_h]: q_j . K_s
    return np.maximum(dots, 0.0) @ w    # gate-weighted head sum


def sigmoid(x: np.ndarray) -> np.ndarray:
    """I = 1 / (1 + exp(-x)), written so it does not overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def logit_threshold(theta: float) -> float:
    """ln(theta/(1-theta)): the logit at which I equals theta (R5)."""
    if not (0.0 < theta < 1.0):
        raise ValueError("threshold must lie in (0, 1)")
    return math.log(theta / (1.0 - theta))


def select(x: np.ndarray, theta: float = 0.5) -> np.ndarray:
    """Keep entry s when I_s >= theta ([BLOG] §3.1 loading rule; [HYPER] 方法)."""
    return np.asarray(x) >= logit_threshold(theta)


def union(masks) -> np.ndarray:
    """OR-mode routing: fetch s if any indexer layer selects it ([BLOG] §4.2; [HYPER] 方法)."""
    out = np.zeros_like(np.asarray(masks[0], dtype=bool))
    for m in masks:
        out |= np.asarray(m, dtype=bool)
    return out


def compact(mask: np.ndarray) -> np.ndarray:
    """Ascending index list of the set entries (R7): the subset C^MemComp."""
    return np.flatnonzero(np.asarray(mask, dtype=bool)).astype(np.int64)


def topk(y: np.ndarray, idx: np.ndarray, k: int) -> np.ndarray:
    """Native top-k inside the subset ([BLOG] §3.2; R6).

    `y` holds the scores of the subset members and `idx` their entry indices,
    aligned. Order by (-y, s), keep the first min(k, M) entries, and return
    them in ascending entry order.
    """
    y = np.asarray(y, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    order = np.lexsort((idx, -y))       # primary key -y, then s
    keep = idx[order[: min(int(k), idx.size)]]
    return np.sort(keep)


def gather(pool: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Load the selected rows: out[i] = pool[idx[i]], bytewise ([HYPER] 方法, C^MemComp loaded)."""
    return np.asarray(pool)[np.asarray(idx, dtype=np.int64)]


# ----------------------------------------------------------- whole path


def run_path(inp, *, sequences=None, layers=None, want_scores=True):
    """The whole selection path for the given sequences of one synthetic input set.

    Steps: project, score, select, OR, compact, top-k, gather. Returns a dict
    keyed by sequence b. Each value holds per-layer q, w, logits, sigmoid
    scores, masks, native scores, the union list and the top-k lists, plus the
    gathered rows. The union always runs over all layers. `layers` only limits
    which layers' top-k are computed.
    """
    w = inp.workload
    B, L = w.B, w.L
    seqs = range(B) if sequences is None else sequences
    lays = range(L) if layers is None else layers
    out = {}
    for b in seqs:
        s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
        per = {"q": [], "w": [], "c": [], "x": [], "I": [], "mask": [], "K": []}
        for l in range(L):
            hl = decode_act(inp.h[l][b:b + 1], w.act_dtype)
            mw = inp.mem_w[l]
            c, q, g = project(hl, decode_act(mw.w_dq, w.act_dtype), decode_act(mw.w_iuq, w.act_dtype),
                              decode_act(mw.w_w, w.act_dtype), w.n_h, w.d_h)
            sc = None if inp.key_scale[l] is None else inp.key_scale[l][s0:s1]
            K = decode_keys(inp.keys[l][s0:s1], w.key_dtype, sc)
            x = logits(q[0], g[0], K)
            per["c"].append(c[0]); per["q"].append(q[0]); per["w"].append(g[0])
            per["x"].append(x)
            per["I"].append(sigmoid(x) if want_scores else None)
            per["mask"].append(select(x, w.threshold))
            per["K"].append(K)
        U = union(per["mask"])
        idx = compact(U)
        tk, ys, qn, wn = {}, {}, {}, {}
        for l in lays:
            hl = decode_act(inp.h[l][b:b + 1], w.act_dtype)
            nw = inp.nat_w[l]
            _, qn_, wn_ = project(hl, decode_act(nw.w_dq, w.act_dtype), decode_act(nw.w_iuq, w.act_dtype),
                                  decode_act(nw.w_w, w.act_dtype), w.n_h, w.d_h)
            y = logits(qn_[0], wn_[0], per["K"][l][idx])
            ys[l], qn[l], wn[l] = y, qn_[0], wn_[0]
            tk[l] = topk(y, idx, w.k)
        del per["K"]
        per.update(union=U, idx=idx, topk=tk, y=ys, qn=qn, wn=wn)
        if inp.pool is not None:
            per["gathered"] = gather(inp.pool[s0:s1], idx)
        out[b] = per
    return out


def step_topk(inp, h_step, lists, *, layers=None):
    """The native top-k of one decode step over the resident subset (R15).

    `h_step[l]` holds the step's hidden states [B, d] (stored values) for
    layer l, and `lists[b]` the subset of sequence b (ascending entry indices,
    loaded at the trigger). For every sequence b and layer l: q', w' are the
    native indexer's projections of the step's h ([BLOG] §3.1 forms with the
    native weights), y_s = sum_j w'_j ReLU(q'_j . K^l_s) for s in the subset,
    and the k best by (-y, s), ascending. Returns {(b, l): (topk, y)}.
    """
    w = inp.workload
    out = {}
    lays = range(w.L) if layers is None else layers
    for b in range(w.B):
        s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
        idx = np.asarray(lists[b], dtype=np.int64)
        for l in lays:
            nw = inp.nat_w[l]
            hl = decode_act(h_step[l][b:b + 1], w.act_dtype)
            _, qn, wn = project(hl, decode_act(nw.w_dq, w.act_dtype), decode_act(nw.w_iuq, w.act_dtype),
                                decode_act(nw.w_w, w.act_dtype), w.n_h, w.d_h)
            sc = None if inp.key_scale[l] is None else inp.key_scale[l][s0:s1][idx]
            K = decode_keys(inp.keys[l][s0:s1][idx], w.key_dtype, sc)
            y = logits(qn[0], wn[0], K) if idx.size else np.zeros(0)
            out[(b, l)] = (topk(y, idx, w.k), y)
    return out
