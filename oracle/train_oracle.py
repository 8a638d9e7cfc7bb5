"""CPU oracle for the memory indexer's training step (TEST INFRASTRUCTURE ONLY).

Plain float64 forward and backward for one indexer layer: the three
projections, the lookahead score, a focal binary cross-entropy against golden
labels, and the gradients of the three trained matrices. Only the tests, the
smoke check and the CPU baseline of bench.py may import it; the product path
never does, and it shares no code with the HIP library.

Sources (section names of the pages):
  [BLOG]  marsggbo.github.io write-up, "4. 训练" (training): the compressed
          index keys are fixed, only the query side's low-rank projections
          W^DQ, W^IUQ and W^w are trained, with Focal Loss; the score is the
          §3.1 formula.
  [HYPER] hyper.ai digest, "方法" (Method): the keys are precomputed and
          frozen; the projections are trained with binary cross-entropy on the
          predicted lookahead scores; random initialisation; focal loss keeps
          the easy negatives from dominating the gradient.
  [GIST]  gist.science summary: binary cross-entropy made focal, to lower the
          weight of easy negatives.

Readings where the pages leave a step open (also listed with the design notes):
  T1  The trained score is the selection score: I_s = sigmoid(x_s) with
      x_s = sum_j w_j ReLU(q_j . K_s), q = (h W^DQ) W^IUQ, w = h W^w.
  T2  The focal loss is the usual form with p = I_s: -alpha (1-p)^gamma log p
      for a golden entry and -(1-alpha) p^gamma log(1-p) for the others.
      The pages give no constants; gamma = 2 and alpha = 0.25 are the defaults
      (the form's own paper's values), both arguments.
  T3  The loss is the mean over every entry of every sequence of the batch.
  T4  Only W^DQ, W^IUQ and W^w get gradients; h and the keys are inputs.
      Weights are stored "out x in" as in the selection path (row n of the
      W^DQ buffer is column n of W^DQ), and so are the gradients.
"""
from __future__ import annotations

import numpy as np


def log_sigmoid(x: np.ndarray) -> np.ndarray:
    """log(sigmoid(x)) = -log(1 + exp(-x)), without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return -np.logaddexp(0.0, -x)


def focal_terms(x: np.ndarray, y: np.ndarray, gamma: float, alpha: float) -> np.ndarray:
    """Per-entry focal loss of logits x against 0/1 labels y (T2)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=bool)
    lp, lq = log_sigmoid(x), log_sigmoid(-x)  # log p, log(1 - p)
    p, q = np.exp(lp), np.exp(lq)
    return np.where(y, -alpha * q ** gamma * lp, -(1.0 - alpha) * p ** gamma * lq)


def focal_grad(x: np.ndarray, y: np.ndarray, gamma: float, alpha: float) -> np.ndarray:
    """d(focal term)/dx, from dp/dx = p (1 - p):
    golden: alpha (1-p)^gamma (gamma p log p - (1 - p));
    other:  (1-alpha) p^gamma (p - gamma (1 - p) log(1 - p))."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=bool)
    lp, lq = log_sigmoid(x), log_sigmoid(-x)
    p, q = np.exp(lp), np.exp(lq)
    pos = alpha * q ** gamma * (gamma * p * lp - q)
    neg = (1.0 - alpha) * p ** gamma * (p - gamma * q * lq)
    return np.where(y, pos, neg)


def train_step(h, w_dq, w_iuq, w_w, keys, labels, n_h: int, d_h: int, gamma: float = 2.0, alpha: float = 0.25):
    """Loss and gradients of one indexer layer for a batch of B sequences (T1-T4).

    h: [B, d]; w_dq: [r, d]; w_iuq: [n_h*d_h, r]; w_w: [n_h, d] (float64 values);
    keys[b]: [N_b, d_h]; labels[b]: bool [N_b]. Returns (loss, g_dq, g_iuq, g_w)
    with the gradients in the weights' own layouts.
    """
    h = np.asarray(h, np.float64)
    w_dq, w_iuq, w_w = (np.asarray(m, np.float64) for m in (w_dq, w_iuq, w_w))
    B = h.shape[0]
    c = h @ w_dq.T                       # [B, r]
    q = (c @ w_iuq.T).reshape(B, n_h, d_h)
    w = h @ w_w.T                        # [B, n_h]
    total = sum(int(np.asarray(k).shape[0]) for k in keys)
    loss = 0.0
    dq = np.zeros((B, n_h, d_h))
    dw = np.zeros((B, n_h))
    for b in range(B):
        K = np.asarray(keys[b], np.float64)
        if K.shape[0] == 0:
            continue
        dots = K @ q[b].T                # [N, n_h]
        relu = np.maximum(dots, 0.0)
        x = relu @ w[b]                  # [N]
        y = np.asarray(labels[b], bool)
        loss += focal_terms(x, y, gamma, alpha).sum()
        g = focal_grad(x, y, gamma, alpha) / total  # d loss / d x_s
        dw[b] = relu.T @ g
        coef = (dots > 0) * g[:, None] * w[b][None, :]   # [N, n_h]: d loss / d dot
        dq[b] = coef.T @ K
    loss /= max(total, 1)
    dqf = dq.reshape(B, n_h * d_h)
    g_iuq = dqf.T @ c                    # [n_h*d_h, r]
    dc = dqf @ w_iuq                     # [B, r]
    g_dq = dc.T @ h                      # [r, d]
    g_w = dw.T @ h                       # [n_h, d]
    return loss, g_dq, g_iuq, g_w
