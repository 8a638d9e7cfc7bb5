"""OR-union and compaction (lsa_union_compact) on hand-made masks (marked gpu).

Integer work, so the result must be bit-exact: the union word of every sequence is the OR of the
layers' words with the bits at or beyond N_b cleared, the list holds the set bits' entry indices in
ascending order, and the count is their number. The masks here are random bit patterns, including
set bits past N_b (which the union must drop), dense chunks, empty sequences, sequences with more
than 2048 words before their last chunk (the carry-in takes several rounds of loads), and enough
sequences that the kernel's chunks grow from 64 words to 128, 192 and 256 (it keeps its grid at
one block per compute unit where it can: 256 on this device).
"""
import numpy as np
import pytest

from tests import parity as P

@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


CASES = {
    # name: (entries per sequence, layers, probability that a bit is set)
    "sparse_ragged": ((1000, 0, 64, 63, 65, 20_000, 1), 3, 0.05),
    "dense_chunks": ((40_000, 17_000), 2, 0.9),
    "all_set": ((16_384, 16_385, 5), 1, 1.0),
    "long_sequences": ((300_000, 150_001), 3, 0.07),
    "eight_layers": ((9_000, 70_000, 333), 8, 0.03),
    "five_layers": ((1200, 64, 130), 5, 0.2),
    "single_entry": ((1,), 4, 0.5),
    # 256 compute units: 469 words x 40 sequences needs 128-word chunks, 1600 x 20 needs 192,
    # 1024 x 64 needs 256, and 200 ragged sequences stay at the 256-word maximum
    "chunks_128": ((30_000,) * 40, 3, 0.1),
    "chunks_192": ((102_400,) * 20, 3, 0.05),
    "chunks_256": ((65_536,) * 64, 2, 0.05),
    "chunks_256_capped": ((40_000, 1, 0, 39_999) * 50, 3, 0.1),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_union_compact_exact(case, torch_cuda):
    from sparse_kv_retrieval_amd import lsa
    torch = torch_cuda
    n, L, dens = CASES[case]
    P.say(f"[union] case={case} N={n} L={L} density={dens}")
    rng = np.random.default_rng(sum(n) + 7 * L)
    n = np.asarray(n, np.int64)
    B = len(n)
    ko = np.zeros(B + 1, np.int64)
    ko[1:] = np.cumsum(n)
    words = (n + 63) // 64
    mwo = np.zeros(B + 1, np.int64)
    mwo[1:] = np.cumsum(words)
    W = int(mwo[-1])
    # every bit of every word drawn, including the bits past N_b of each sequence's last word
    bits = rng.random((L, W * 64)) < dens
    masks_h = np.packbits(bits.reshape(L, W, 64)[:, :, ::-1], axis=2).view(">u8").reshape(L, W).astype(np.uint64)
    masks = [torch.from_numpy(m.view(np.int64)).cuda() for m in masks_h]
    idx = torch.full((max(int(ko[-1]), 1),), -5, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    um = torch.zeros(max(W, 1), dtype=torch.int64, device="cuda")
    lsa.union_compact(masks, B=B, key_offsets=torch.from_numpy(ko).cuda(), key_offsets_host=ko,
                      mask_word_offsets=torch.from_numpy(mwo).cuda(), mask_word_offsets_host=mwo, idx_out=idx,
                      count_out=cnt, union_mask_out=um)
    torch.cuda.synchronize()
    idx_h, cnt_h, um_h = idx.cpu().numpy(), cnt.cpu().numpy(), um.cpu().numpy().view(np.uint64)
    orbits = bits.any(axis=0)
    for b in range(B):
        sel = orbits[mwo[b] * 64: mwo[b] * 64 + n[b]]
        want = np.flatnonzero(sel).astype(np.int32)
        assert cnt_h[b] == want.size, (b, cnt_h[b], want.size)
        assert np.array_equal(idx_h[ko[b]: ko[b] + want.size], want), b
        # the union words: the layers' OR with the bits at or beyond N_b cleared
        wbits = np.zeros(words[b] * 64, bool)
        wbits[: n[b]] = sel
        want_words = np.packbits(wbits.reshape(-1, 64)[:, ::-1], axis=1).view(">u8").reshape(-1).astype(np.uint64)
        assert np.array_equal(um_h[mwo[b]: mwo[b + 1]], want_words), b
        # nothing written past the count in the sequence's region
        assert (idx_h[ko[b] + want.size: ko[b + 1]] == -5).all(), b
