"""Checks that pin the training-step oracle to things other than itself.

Each `check_*` takes the oracle module (or a copy with a planted mistake) and
raises AssertionError on disagreement with: the hand-worked focal terms and
forward pass in tests/golden/train_hand.json, the reduction of the focal form
to half the plain binary cross-entropy at gamma = 0 and alpha = 1/2 (written
here with logaddexp), and central finite differences of the loss.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_hand():
    with open(os.path.join(GOLDEN, "train_hand.json")) as f:
        return json.load(f)


def check_focal_hand(T):
    fx = load_hand()
    for c in fx["focal"]:
        p = c["p"][0] / c["p"][1]
        x = np.array([math.log(p / (1 - p))])
        y = np.array([c["y"]])
        lv = c["loss"][0] + c["loss"][1] * math.log(2)
        gv = c["grad"][0] + c["grad"][1] * math.log(2)
        assert abs(T.focal_terms(x, y, fx["gamma"], fx["alpha"])[0] - lv) < 1e-12, c
        assert abs(T.focal_grad(x, y, fx["gamma"], fx["alpha"])[0] - gv) < 1e-12, c


def check_bce_special_case(T):
    """gamma = 0, alpha = 1/2: half the binary cross-entropy, gradient (sigmoid(x) - y) / 2."""
    rng = np.random.default_rng(3)
    x = rng.normal(0, 4, 200)
    y = rng.random(200) < 0.3
    bce = np.where(y, np.logaddexp(0, -x), np.logaddexp(0, x))
    assert np.allclose(T.focal_terms(x, y, 0.0, 0.5), 0.5 * bce, rtol=1e-13, atol=1e-15)
    assert np.allclose(T.focal_grad(x, y, 0.0, 0.5), 0.5 * (1 / (1 + np.exp(-x)) - y), rtol=1e-12, atol=1e-15)


def check_focal_grad_fd(T):
    rng = np.random.default_rng(4)
    x = rng.normal(0, 3, 100)
    y = rng.random(100) < 0.5
    for gamma, alpha in ((2.0, 0.25), (0.5, 0.7), (3.0, 0.5)):
        e = 1e-6
        fd = (T.focal_terms(x + e, y, gamma, alpha) - T.focal_terms(x - e, y, gamma, alpha)) / (2 * e)
        assert np.allclose(T.focal_grad(x, y, gamma, alpha), fd, rtol=1e-6, atol=1e-9), (gamma, alpha)


def check_chain_hand(T):
    c = load_hand()["chain"]
    fx = load_hand()
    loss, g_dq, g_iuq, g_w = T.train_step(np.array(c["h"], float), np.array(c["w_dq"], float),
                                          np.array(c["w_iuq"], float), np.array(c["w_w"], float),
                                          [np.array(c["keys"], float)], [np.array(c["labels"], bool)],
                                          c["n_h"], c["d_h"], fx["gamma"], fx["alpha"])
    want = T.focal_terms(np.array(c["x"], float), np.array(c["labels"], bool), fx["gamma"], fx["alpha"]).mean()
    assert abs(loss - want) < 1e-12, (loss, want)
    assert g_dq.shape == (2, 2) and g_iuq.shape == (4, 2) and g_w.shape == (2, 2)


def _tiny_problem(seed):
    """A small problem whose head dots stay away from 0 (no ReLU kink within the difference step)."""
    rng = np.random.default_rng(seed)
    B, d, r, n_h, d_h = 2, 6, 5, 3, 4
    while True:
        h = rng.normal(0, 1, (B, d))
        w_dq = rng.normal(0, 0.5, (r, d))
        w_iuq = rng.normal(0, 0.5, (n_h * d_h, r))
        w_w = rng.normal(0, 0.5, (n_h, d))
        keys = [rng.normal(0, 1, (n, d_h)) for n in (7, 5)]
        labels = [rng.random(k.shape[0]) < 0.4 for k in keys]
        q = ((h @ w_dq.T) @ w_iuq.T).reshape(B, n_h, d_h)
        if min(np.abs(keys[b] @ q[b].T).min() for b in range(B)) > 1e-2:
            return (h, w_dq, w_iuq, w_w, keys, labels, n_h, d_h)
        seed += 1000


def check_train_fd(T):
    """Every gradient entry against central differences of the loss."""
    args = _tiny_problem(7)
    h, w_dq, w_iuq, w_w, keys, labels, n_h, d_h = args
    loss, g_dq, g_iuq, g_w = T.train_step(*args, gamma=2.0, alpha=0.25)
    assert g_dq.shape == w_dq.shape and g_iuq.shape == w_iuq.shape and g_w.shape == w_w.shape
    e = 1e-6
    for name, W, G in (("w_dq", w_dq, g_dq), ("w_iuq", w_iuq, g_iuq), ("w_w", w_w, g_w)):
        for idx in np.ndindex(W.shape):
            Wp, Wm = W.copy(), W.copy()
            Wp[idx] += e
            Wm[idx] -= e
            ap = dict(w_dq=w_dq, w_iuq=w_iuq, w_w=w_w)
            ap[name] = Wp
            lp = T.train_step(h, ap["w_dq"], ap["w_iuq"], ap["w_w"], keys, labels, n_h, d_h, 2.0, 0.25)[0]
            ap[name] = Wm
            lm = T.train_step(h, ap["w_dq"], ap["w_iuq"], ap["w_w"], keys, labels, n_h, d_h, 2.0, 0.25)[0]
            fd = (lp - lm) / (2 * e)
            assert abs(fd - G[idx]) <= 1e-6 * max(1.0, abs(fd)) + 1e-9, (name, idx, fd, G[idx])


ALL = [check_focal_hand, check_bce_special_case, check_focal_grad_fd, check_chain_hand, check_train_fd]
