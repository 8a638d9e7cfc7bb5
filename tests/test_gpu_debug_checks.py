"""The debug build's device range checks (marked gpu).

A list entry outside [0, N_b) of its sequence is counted by lsa_debug_range_errors and its row is
not read: the gather leaves its output row untouched, and the top-k scoring of gathered rows scores
it as an all-zero key (y = 0). A clean call counts nothing. The debug copy of the library is loaded
in a child process, so that the product library of this process is untouched. The product build
itself is checked on the CPU (tests/test_capi_host.py): it has no checks and says so.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_ROOT = os.path.join(ROOT, "sparse_kv_retrieval_amd", "_debug")

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from sparse_kv_retrieval_amd import lsa
assert lsa.LIB_PATH.startswith(sys.argv[1]), lsa.LIB_PATH
dev = "cuda"
print("[debug-checks] library:", lsa.LIB_PATH, flush=True)
assert lsa.debug_range_errors() == 0

# gather: two sequences of 8 and 5 pool rows of 64 bytes; one entry past N_0, one negative in sequence 1
rng = np.random.default_rng(5)
pool_h = rng.integers(-30000, 30000, size=(13, 32), dtype=np.int16)
pool = torch.from_numpy(pool_h).to(dev)
po_h = np.array([0, 8, 13], np.int64)
po = torch.from_numpy(po_h).to(dev)
idx_h = np.array([0, 3, 8, 7, -1, 2], np.int32)
idx = torch.from_numpy(idx_h).to(dev)
io = torch.tensor([0, 4, 6], dtype=torch.int64, device=dev)
cnt = torch.tensor([4, 2], dtype=torch.int32, device=dev)
out = torch.full((6, 32), 7, dtype=torch.int16, device=dev)
lsa.gather(pool, row_bytes=64, B=2, pool_row_offsets=po, pool_row_offsets_host=po_h, idx=idx, idx_offsets=io,
           count=cnt, out=out, out_capacity_rows=6)
n = lsa.debug_range_errors()
o = out.cpu().numpy()
print("[debug-checks] gather: errors", n, flush=True)
assert n == 2, n
for r, (b, e) in enumerate([(0, 0), (0, 3), (0, 8), (0, 7), (1, -1), (1, 2)]):
    if 0 <= e < po_h[b + 1] - po_h[b]:
        assert (o[r] == pool_h[po_h[b] + e]).all(), r
    else:
        assert (o[r] == 7).all(), r  # the row was not read, and its output not written
# the same call with the bad entries replaced: nothing counted
idx2 = torch.from_numpy(np.array([0, 3, 5, 7, 4, 2], np.int32)).to(dev)
lsa.gather(pool, row_bytes=64, B=2, pool_row_offsets=po, pool_row_offsets_host=po_h, idx=idx2, idx_offsets=io,
           count=cnt, out=out, out_capacity_rows=6)
assert lsa.debug_range_errors() == 0

# top-k scoring of gathered rows: one sequence of 100 bf16 keys, a list of 40 with two bad entries
N, nh, dh, M = 100, 64, 128, 40
keys = torch.randn(N, dh, device=dev).to(torch.bfloat16).view(torch.int16)
q = torch.randn(1, nh, dh, device=dev)
w = torch.randn(1, nh, device=dev)
lst = np.arange(0, 2 * M, 2, dtype=np.int32)
lst[5], lst[7] = N, -3
ko_h = np.array([0, N], np.int64)
ko = torch.from_numpy(ko_h).to(dev)
li = torch.zeros(N, dtype=torch.int32, device=dev)
li[:M] = torch.from_numpy(lst).to(dev)
lc = torch.tensor([M], dtype=torch.int32, device=dev)
ws = torch.zeros(lsa.topk_workspace_size(1, 1, N, 1), dtype=torch.uint8, device=dev)
layer = [dict(q=q, w=w, keys=keys, key_scale=None)]
lsa.topk_score(layer, B=1, key_offsets=ko, key_offsets_host=ko_h, idx=li, count=lc, n_h=nh, d_h=dh,
               key_dtype="bf16", workspace=ws)
n = lsa.debug_range_errors()
y = ws[: 4 * N].view(torch.float32).cpu().numpy()
print("[debug-checks] topk score: errors", n, flush=True)
assert n >= 2, n
assert y[5] == 0.0 and y[7] == 0.0, (y[5], y[7])
# the valid entries against a float64 reference on the CPU
K = keys.view(torch.bfloat16).float().cpu().double().numpy()
Q, Wt = q[0].cpu().double().numpy(), w[0].cpu().double().numpy()
for i in range(M):
    if i in (5, 7):
        continue
    ref = float(np.sum(Wt * np.maximum(Q @ K[lst[i]], 0.0)))
    assert abs(y[i] - ref) <= 2e-2 + 1e-3 * abs(ref), (i, y[i], ref)
li[:M] = torch.from_numpy(np.arange(0, 2 * M, 2, dtype=np.int32)).to(dev)
lsa.topk_score(layer, B=1, key_offsets=ko, key_offsets_host=ko_h, idx=li, count=lc, n_h=nh, d_h=dh,
               key_dtype="bf16", workspace=ws)
assert lsa.debug_range_errors() == 0
print("[debug-checks] ok", flush=True)
"""


@pytest.mark.gpu
def test_debug_build_counts_and_skips_out_of_range_entries():
    lib = os.path.join(DEBUG_ROOT, "sparse_kv_retrieval_amd", "liblsa.so")
    if not os.path.exists(lib):
        pytest.skip("the debug build is missing (sparse_kv_retrieval_amd.build.build_debug)")
    r = subprocess.run([sys.executable, "-c", CHILD, DEBUG_ROOT], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "[debug-checks] ok" in r.stdout
