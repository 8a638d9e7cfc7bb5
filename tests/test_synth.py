"""The seeded generator: determinism, layout and the planting structure.

The checks run on narrow copies of the workloads (d, r and n_h cut down): the
layout and the planting rule do not depend on the width, and the full-width
weights would dominate the CPU suite's time.
"""
import dataclasses

import numpy as np

from sparse_kv_retrieval_amd import synth


def _narrow(w, **kw):
    return dataclasses.replace(synth.scaled(w, **kw), d=512, r=256, n_h=8)


def test_deterministic_and_layout():
    w = _narrow(synth.WORKLOADS["ragged_b32"], N=(100, 0, 65, 1), name="t")
    a, b = synth.make(w), synth.make(w)
    assert a.key_offsets.tolist() == [0, 100, 100, 165, 166]
    assert a.mask_word_offsets.tolist() == [0, 2, 2, 4, 5]
    for l in range(w.L):
        assert a.keys[l].dtype == np.uint16 and a.keys[l].shape == (166, 128)
        assert np.array_equal(a.keys[l], b.keys[l])
        assert np.array_equal(a.h[l], b.h[l])
        assert np.array_equal(a.mem_w[l].w_iuq, b.mem_w[l].w_iuq)
        assert a.mem_w[l].w_dq.shape == (w.r, w.d) and a.mem_w[l].w_w.shape == (w.n_h, w.d)
    assert np.array_equal(a.pool, b.pool) and a.pool.shape == (166, 512)


def test_fp8_keys_and_scales():
    w = _narrow(synth.WORKLOADS["fp8_1m"], N=300, B=2, name="t8")
    inp = synth.make(w, with_pool=False)
    assert inp.keys[0].dtype == np.uint8 and inp.key_scale[0].shape == (600,)
    assert np.all(inp.key_scale[0] > 0)
    # every row reaches the format maximum (+-448 = 0x7E / 0xFE) by construction of its scale
    assert np.all(np.any((inp.keys[0] & 0x7F) == 0x7E, axis=1))


def test_ragged_lengths_in_range():
    n = synth.lengths(synth.WORKLOADS["ragged_b32"])
    assert n.size == 32 and n.min() >= 16384 // 4 and n.max() <= 524288 // 4


def test_tiny_is_plain_gaussian():
    w = synth.WORKLOADS["tiny_f32"]
    inp = synth.make(w)
    assert inp.keys[0].dtype == np.float32 and inp.keys[0].shape == (1024, 32)
    assert not inp.planted[0].any()
    assert inp.h[0].dtype == np.float32 and inp.h[0].shape == (1, 256)


def test_planted_fraction():
    w = _narrow(synth.WORKLOADS["three_layer_b8"], N=2000, B=2, name="tp")
    inp = synth.make(w, with_pool=False)
    for l in range(w.L):
        assert inp.planted[l].sum() == 2 * round(0.05 * 2000)
