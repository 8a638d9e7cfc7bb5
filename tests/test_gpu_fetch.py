"""lsa_fetch_host: the load step from a cold pool in pinned host memory (marked gpu).

The fetched rows must be byte-identical to the pool rows that the union list
names (the oracle's gather is plain indexing of the pool), at small sizes in
full and at the full three-layer size on sampled rows. A pool in pageable
host memory is refused without leaving an error behind.
"""
import numpy as np
import pytest

from sparse_kv_retrieval_amd import synth
from tests import parity as P
from tests.test_gpu_parity import SMALL


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["ragged_small", "three_layer_mixed"])
def test_fetch_host_small(case, torch_cuda):
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = SMALL[case]
    P.say(f"[fetch] case={case}")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", guard=True, host_pool=True)
    p.run()  # the load step reads the pinned host pool
    torch_cuda.cuda.synchronize()
    assert p.check_guards() == [], f"writes outside an output buffer: {p.check_guards()}"
    _, lists = P.gpu_union_lists(p, inp)
    P.check_gather(p, inp, lists)


@pytest.mark.gpu
def test_fetch_host_full_size(torch_cuda):
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = synth.WORKLOADS["three_layer_b8"]
    P.say("[fetch] three_layer_b8: generating")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", host_pool=True)
    P.say("[fetch] three_layer_b8: running")
    p.run()
    torch_cuda.cuda.synchronize()
    _, lists = P.gpu_union_lists(p, inp)
    P.check_gather(p, inp, lists)
    # the HBM gather of the same rows writes the same bytes
    fetched = p.gathered.clone()
    p.gathered.zero_()
    p.gather()
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(fetched, p.gathered)


@pytest.mark.gpu
def test_fetch_host_refuses_pageable_memory(torch_cuda):
    from sparse_kv_retrieval_amd import lsa
    w = SMALL["ragged_small"]
    inp = synth.make(w)
    ko = inp.key_offsets.astype(np.int64)
    dev = torch_cuda.device("cuda")
    pageable = torch_cuda.from_numpy(inp.pool.view(np.int16).copy())  # not pinned
    t = lambda a: torch_cuda.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = torch_cuda.zeros((10, w.pool_dim), dtype=torch_cuda.int16, device=dev)
    with pytest.raises(lsa.LsaError) as ei:
        lsa.fetch_host(pageable, row_bytes=w.pool_dim * 2, B=w.B, pool_row_offsets=t(ko), pool_row_offsets_host=ko,
                       idx=t(np.zeros(int(ko[-1]), np.int32)), idx_offsets=t(ko[:-1]),
                       count=t(np.ones(w.B, np.int32)), out=out, out_capacity_rows=10)
    assert ei.value.status == lsa.ERR_INVALID_ARG and "pinned" in str(ei.value)
    # no error is left behind for the next HIP call
    x = torch_cuda.ones(4, device=dev) * 2
    torch_cuda.cuda.synchronize()
    assert float(x.sum()) == 8.0
