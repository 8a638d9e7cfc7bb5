"""Per-step top-k over the resident subset (lsa_topk_step) against the oracle, through the C-ABI
(marked gpu).

After one trigger (project, score, union), each layer's union rows of keys are packed once with
lsa_gather; then every decode step projects its own native query from the step's hidden state
and ranks the resident subset with lsa_topk_step. Every step's top-k of every (layer, sequence)
is compared with the oracle's step_topk over the same union lists.
"""
import dataclasses

import numpy as np
import pytest

from sparse_kv_retrieval_amd import synth
from tests import parity as P

W = synth.WORKLOADS

CASES = {
    # (workload, decode steps)
    "three_layer_mixed": (synth.scaled(W["three_layer_b8"], N=(3000, 0, 1, 64, 65, 700), k=128), 64),
    "fp8_two_seq": (synth.scaled(W["fp8_1m"], N=(5000, 63), k=512), 64),
    "ragged_small": (synth.scaled(W["ragged_b32"], N=(2000, 1500, 127, 0, 129), k=100), 64),
    "bf16_16heads_d64": (dataclasses.replace(synth.scaled(W["three_layer_b8"], N=(2100, 333), k=64), n_h=16, d_h=64,
                                             d=512, r=256, name="h16d64"), 16),
    "f32_d32": (W["tiny_f32"], 16),
    "k_over_subset": (synth.scaled(W["three_layer_b8"], N=(600, 200), k=4096), 8),
    # the metric's workload at full size, a few steps
    "three_layer_b8_full": (W["three_layer_b8"], 4),
    "fp8_1m_full": (W["fp8_1m"], 2),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_decode_steps(case):
    import torch
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w, T = CASES[case]
    P.say(f"[steps] case={case} B={w.B} L={w.L} dtype={w.key_dtype} k={w.k} steps={T}")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", guard=True)
    p.alloc_steps()
    p.run()
    p.pack_subset_keys()
    torch.cuda.synchronize()
    counts, lists = P.gpu_union_lists(p, inp)
    # the packed keys are the union rows of each layer's keys, bit for bit
    for l in range(w.L):
        ks = p.keys_sub[l].cpu().numpy()
        off = 0
        for b in range(w.B):
            s0 = int(inp.key_offsets[b])
            want = inp.keys[l][s0 + lists[b]]
            got = ks[off:off + lists[b].size]
            assert got.tobytes() == np.ascontiguousarray(want).tobytes(), f"packed keys l={l} b={b}"
            off += lists[b].size
    hs = synth.step_hidden(inp, T)
    for t in range(T):
        p.set_step_hidden(hs[t])
        p.step()
        torch.cuda.synchronize()
        P.check_step(p, inp, hs[t], lists, f"step {t}")
    assert p.check_guards() == [], f"writes outside an output buffer: {p.check_guards()}"
    P.say(f"[steps] case={case} ok: {T} steps, union sizes {counts.tolist()[:8]}")
