"""lsa_topk_step_noalloc (the allocation-free entry point) against lsa_topk_step with a workspace,
through the C-ABI (marked gpu).

Two calls in a row on one device, the second with a smaller input than the first: the fixed
scratch keeps the first call's contents, so the second shows that each call clears what it
needs. Both entry points run the same kernels, so their outputs must be identical bit for bit.
"""
import numpy as np
import pytest

from sparse_kv_retrieval_amd import synth
from tests import parity as P

W = synth.WORKLOADS


def _compare(torch, w, steps):
    from sparse_kv_retrieval_amd import lsa
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    inp = synth.make(w)
    p = Pipeline(inp, "cuda")
    p.alloc_steps()
    p.run()
    p.pack_subset_keys()
    hs = synth.step_hidden(inp, steps)
    for t in range(steps):
        p.set_step_hidden(hs[t])
        p.step()  # lsa_topk_step with the pipeline's workspace
        torch.cuda.synchronize()
        want = [x.clone() for x in p.step_idx + p.step_score + [p.step_count]]
        for x in p.step_idx + p.step_score + [p.step_count]:
            x.fill_(-3)
        tl = [dict(q=p.q_step[l], w=p.g_step[l], keys=p.keys_sub[l], key_scale=p.scale[l],
                   topk_idx_out=p.step_idx[l], topk_score_out=p.step_score[l]) for l in range(w.L)]
        lsa.topk_step_noalloc(tl, B=w.B, key_offsets=p.key_off, key_offsets_host=p.key_off_h, idx=p.idx,
                              count=p.count, n_h=w.n_h, d_h=w.d_h, key_dtype=w.key_dtype, k=w.k,
                              topk_count_out=p.step_count)
        torch.cuda.synchronize()
        got = p.step_idx + p.step_score + [p.step_count]
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"step {t}: lsa_topk_step_noalloc differs from lsa_topk_step"
    return int(p.rows)


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    import torch
    big = synth.scaled(W["three_layer_b8"], N=(60_000, 40_000, 129), k=256)
    small = synth.scaled(W["three_layer_b8"], N=(3000, 0, 65), k=64)
    P.say("[noalloc] first call: 3 sequences, 100K entries")
    r1 = _compare(torch, big, 3)
    P.say("[noalloc] second call: a smaller input on the same scratch")
    r2 = _compare(torch, small, 3)
    assert r2 < r1
    P.say("[noalloc] ok")
