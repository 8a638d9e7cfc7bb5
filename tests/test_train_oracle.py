"""Pins of the training-step oracle (CPU), and plausible mistakes each caught by a pin."""
import types

import numpy as np
import pytest

from oracle import train_oracle as T
from tests import train_checks as C


@pytest.mark.parametrize("check", C.ALL, ids=lambda f: f.__name__)
def test_train_oracle_pin(check):
    check(T)


def _clone():
    m = types.ModuleType("train_mutant")
    m.__dict__.update({k: v for k, v in T.__dict__.items() if not k.startswith("__")})
    return m


def _step_with(**flags):
    """train_step with one planted change, written out so that each flag touches one line of the maths."""
    def step(h, w_dq, w_iuq, w_w, keys, labels, n_h, d_h, gamma=2.0, alpha=0.25):
        B = h.shape[0]
        c = h @ w_dq.T
        q = (c @ w_iuq.T).reshape(B, n_h, d_h)
        w = h @ w_w.T
        total = sum(k.shape[0] for k in keys)
        loss, dq, dw = 0.0, np.zeros((B, n_h, d_h)), np.zeros((B, n_h))
        for b in range(B):
            dots = keys[b] @ q[b].T
            relu = np.maximum(dots, 0.0)
            x = relu @ w[b]
            loss += T.focal_terms(x, labels[b], gamma, alpha).sum()
            g = T.focal_grad(x, labels[b], gamma, alpha) / (1 if flags.get("no_mean") else total)
            dw[b] = (dots if flags.get("dw_no_relu") else relu).T @ g
            mask = 1.0 if flags.get("no_relu_mask") else (dots > 0)
            wf = 1.0 if flags.get("no_gate") else w[b][None, :]
            dq[b] = (mask * g[:, None] * wf).T @ keys[b]
        loss /= total
        dqf = dq.reshape(B, -1)
        g_iuq = dqf.T @ c
        dc = dqf @ w_iuq
        if flags.get("skip_dc_chain"):  # the gradient of W^DQ taken as if c were the trained input
            dc = dqf[:, : c.shape[1]]
        g_dq = dc.T @ h
        return loss, g_dq, g_iuq, dw.T @ h
    return step


def _mut_neg_sign(m):
    orig = T.focal_grad
    m.focal_grad = lambda x, y, g, a: np.where(np.asarray(y, bool), orig(x, y, g, a), -orig(x, y, g, a))


def _mut_gamma_ignored(m):
    orig = T.focal_terms
    m.focal_terms = lambda x, y, g, a: orig(x, y, 0.0, a)


def _mut_alpha_swapped(m):
    orig = T.focal_terms
    m.focal_terms = lambda x, y, g, a: orig(x, y, g, 1.0 - a)


def _mut_no_relu_mask(m):
    m.train_step = _step_with(no_relu_mask=True)


def _mut_no_gate(m):
    m.train_step = _step_with(no_gate=True)


def _mut_no_mean(m):
    m.train_step = _step_with(no_mean=True)


def _mut_dw_no_relu(m):
    m.train_step = _step_with(dw_no_relu=True)


def _mut_skip_dc_chain(m):
    m.train_step = _step_with(skip_dc_chain=True)


MUTATIONS = [_mut_neg_sign, _mut_gamma_ignored, _mut_alpha_swapped, _mut_no_relu_mask, _mut_no_gate, _mut_no_mean,
             _mut_dw_no_relu, _mut_skip_dc_chain]


@pytest.mark.parametrize("mut", MUTATIONS, ids=lambda f: f.__name__)
def test_train_mutation_is_caught(mut):
    m = _clone()
    mut(m)
    failed = []
    for check in C.ALL:
        try:
            check(m)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"{mut.__name__} passed every pin"
