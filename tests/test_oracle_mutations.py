"""Each plausible mistake, planted in a copy of the oracle, is caught by at least one pin.

The mistakes are planted on the CPU in a throw-away copy of the oracle module.
The real oracle is never modified.
"""
import inspect
import types

import numpy as np
import pytest

from oracle import lsa_oracle as O
from tests import oracle_checks as C


def _clone():
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: v for k, v in O.__dict__.items() if not k.startswith("__")})
    m.E4M3FN_TABLE = O.E4M3FN_TABLE.copy()
    return m


def _mut_no_relu(m):
    m.logits = lambda q, w, K: (K @ q.T) @ w


def _mut_relu_after_gate(m):
    m.logits = lambda q, w, K: np.maximum((K @ q.T) * w, 0).sum(axis=1)


def _mut_sum_then_relu(m):
    m.logits = lambda q, w, K: np.maximum((K @ q.T) @ w, 0)


def _mut_strict_threshold(m):
    m.select = lambda x, theta=0.5: np.asarray(x) > m.logit_threshold(theta)


def _mut_threshold_sign(m):
    m.logit_threshold = lambda theta: float(np.log((1 - theta) / theta)) + (0.1 if theta == 0.5 else 0.0)


def _mut_union_and(m):
    def union(masks):
        out = np.ones_like(np.asarray(masks[0], bool))
        for x in masks:
            out &= np.asarray(x, bool)
        return out
    m.union = union


def _mut_topk_tie_high(m):
    def topk(y, idx, k):
        order = np.lexsort((-np.asarray(idx), -np.asarray(y, float)))
        return np.sort(np.asarray(idx)[order[:min(k, len(idx))]])
    m.topk = topk


def _mut_topk_score_order(m):
    def topk(y, idx, k):
        order = np.lexsort((np.asarray(idx), -np.asarray(y, float)))
        return np.asarray(idx)[order[:min(k, len(idx))]]
    m.topk = topk


def _mut_topk_smallest(m):
    def topk(y, idx, k):
        order = np.lexsort((np.asarray(idx), np.asarray(y, float)))
        return np.sort(np.asarray(idx)[order[:min(k, len(idx))]])
    m.topk = topk


def _mut_proj_no_transpose_q(m):
    def project(h, w_dq, w_iuq, w_w, n_h, d_h):
        h = np.atleast_2d(h)
        c = h @ w_dq.T
        q = (c @ w_iuq.T).reshape(h.shape[0], d_h, n_h).transpose(0, 2, 1)  # head/dim swapped
        return c, q, h @ w_w.T
    m.project = project


def _mut_proj_gate_from_c(m):
    def project(h, w_dq, w_iuq, w_w, n_h, d_h):
        h = np.atleast_2d(h)
        c = h @ w_dq.T
        q = (c @ w_iuq.T).reshape(h.shape[0], n_h, d_h)
        return c, q, -(h @ w_w.T)          # gate sign flipped
    m.project = project


def _mut_bf16_low_half(m):
    def bf16_to_f64(bits):
        b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return b.view(np.float32).astype(np.float64)
    m.bf16_to_f64 = bf16_to_f64


def _mut_e4m3_bias8(m):
    t = m.E4M3FN_TABLE.copy()
    m.E4M3FN_TABLE = t * 0.5


def _mut_e4m3_no_subnormal(m):
    t = m.E4M3FN_TABLE.copy()
    t[0x01:0x08] = 0.0
    t[0x81:0x88] = 0.0
    m.E4M3FN_TABLE = t


def _mut_sigmoid_sign(m):
    m.sigmoid = lambda x: 1.0 / (1.0 + np.exp(np.asarray(x, float)))


def _mut_compact_descending(m):
    m.compact = lambda mask: np.flatnonzero(np.asarray(mask, bool))[::-1].astype(np.int64)


def _mut_gather_offset(m):
    m.gather = lambda pool, idx: np.asarray(pool)[np.minimum(np.asarray(idx) + 1, len(pool) - 1)]


def _from_source(m, fn_name, old, new):
    """Re-define one oracle function in the copy from its source with `old` replaced by `new`."""
    src = inspect.getsource(getattr(O, fn_name))
    assert old in src, (fn_name, old)
    exec(compile(src.replace(old, new), f"<mutant {fn_name}>", "exec"), m.__dict__)


def _mut_fp8_divide_scale(m):
    _from_source(m, "decode_keys", "e4m3fn_to_f64(keys) * np.asarray(scale", "e4m3fn_to_f64(keys) / np.asarray(scale")


def _mut_fp8_scale_wrong_axis(m):
    _from_source(m, "decode_keys", "[:, None]", "[None, :]")


def _mut_fp8_scale_ignored(m):
    _from_source(m, "decode_keys", "* np.asarray(scale, np.float32).astype(np.float64)[:, None]", "")


def _mut_path_mem_query_topk(m):
    _from_source(m, "run_path", "nw = inp.nat_w[l]", "nw = inp.mem_w[l]")


def _mut_path_other_layer_keys(m):
    _from_source(m, "run_path", 'per["K"][l][idx]', 'per["K"][(l + 1) % L][idx]')


def _mut_path_topk_over_own_selection(m):
    _from_source(m, "run_path", "tk[l] = topk(y, idx, w.k)",
                 "tk[l] = topk(y[per['mask'][l][idx]], idx[per['mask'][l][idx]], w.k)")


def _mut_path_first_layer_h(m):
    _from_source(m, "run_path", "decode_act(inp.h[l][b:b + 1]", "decode_act(inp.h[0][b:b + 1]")


def _mut_step_mem_weights(m):
    _from_source(m, "step_topk", "nw = inp.nat_w[l]", "nw = inp.mem_w[l]")


def _mut_step_trigger_h(m):
    _from_source(m, "step_topk", "decode_act(h_step[l][b:b + 1]", "decode_act(inp.h[l][b:b + 1]")


def _mut_step_whole_sequence(m):  # ranks every entry instead of the resident subset
    _from_source(m, "step_topk", "idx = np.asarray(lists[b], dtype=np.int64)",
                 "idx = np.arange(s1 - s0, dtype=np.int64)")


MUTANTS = [_mut_no_relu, _mut_relu_after_gate, _mut_sum_then_relu, _mut_strict_threshold,
           _mut_threshold_sign, _mut_union_and, _mut_topk_tie_high, _mut_topk_score_order,
           _mut_topk_smallest, _mut_proj_no_transpose_q, _mut_proj_gate_from_c, _mut_bf16_low_half,
           _mut_e4m3_bias8, _mut_e4m3_no_subnormal, _mut_sigmoid_sign, _mut_compact_descending,
           _mut_gather_offset, _mut_fp8_divide_scale, _mut_fp8_scale_wrong_axis, _mut_fp8_scale_ignored,
           _mut_path_mem_query_topk, _mut_path_other_layer_keys, _mut_path_topk_over_own_selection,
           _mut_path_first_layer_h, _mut_step_mem_weights, _mut_step_trigger_h, _mut_step_whole_sequence]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutate):
    m = _clone()
    mutate(m)
    caught = []
    for check in C.ALL_CHECKS:
        try:
            check(m)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin catches {mutate.__name__}"
    print(mutate.__name__, "caught by", caught)
