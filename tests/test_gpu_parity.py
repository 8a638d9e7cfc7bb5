"""HIP path vs the CPU oracle, through the C-ABI (marked gpu).

Small cases span several tiles, ragged tails, empty and one-entry sequences,
k above and below the subset size, and every key dtype and head shape.
The full-size cases run the workloads at their real sizes, with the launch
configuration that bench.py times, and compare every output with the oracle.
"""
import dataclasses

import numpy as np
import pytest

from sparse_kv_retrieval_amd import synth
from tests import parity as P

W = synth.WORKLOADS

SMALL = {
    "tiny_f32": W["tiny_f32"],
    "tiny_f32_k_over": dataclasses.replace(W["tiny_f32"], k=4096, name="tiny_k_over"),
    "single_bf16_tail": synth.scaled(W["single_layer_500k"], N=(4099,), k=256),
    "three_layer_mixed": synth.scaled(W["three_layer_b8"], N=(3000, 0, 1, 64, 65, 700), k=128),
    "fp8_two_seq": synth.scaled(W["fp8_1m"], N=(5000, 63), k=512),
    "ragged_small": synth.scaled(W["ragged_b32"], N=(2000, 1500, 127, 0, 129), k=100),
    "bf16_16heads_d64": dataclasses.replace(
        synth.scaled(W["three_layer_b8"], N=(2100, 333), k=64), n_h=16, d_h=64, d=512, r=256, name="h16d64"),
    "fp8_8heads_d32": dataclasses.replace(
        synth.scaled(W["fp8_1m"], N=(1000,), k=32), n_h=8, d_h=32, d=256, r=128, L=2, name="h8d32"),
    "f32_d128_48heads": dataclasses.replace(
        synth.scaled(W["three_layer_b8"], N=(777, 64), k=50), key_dtype="f32", act_dtype="f32", n_h=48, d=256,
        r=128, L=2, name="f32h48"),
    "single_k_ge_count": synth.scaled(W["three_layer_b8"], N=(600, 200), k=4096),
    # other loading thresholds: the comparison is x >= ln(theta / (1 - theta))
    "three_layer_theta03": dataclasses.replace(synth.scaled(W["three_layer_b8"], N=(4000, 129, 0, 2500), k=128),
                                               threshold=0.3, name="theta03"),
    "fp8_theta07": dataclasses.replace(synth.scaled(W["fp8_1m"], N=(3000, 700), k=200), threshold=0.7,
                                       name="fp8_theta07"),
    "bf16_d64_theta07": dataclasses.replace(
        synth.scaled(W["three_layer_b8"], N=(1500, 65), k=64), n_h=16, d_h=64, d=512, r=256, threshold=0.7,
        name="h16d64_theta07"),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    return torch


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(SMALL))
def test_small_parity(case, torch_cuda):
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = SMALL[case]
    P.say(f"[parity] case={case} B={w.B} L={w.L} N={w.N} dtype={w.key_dtype} n_h={w.n_h} d_h={w.d_h} k={w.k}")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", with_scores=True, guard=True)
    p.run()
    torch_cuda.cuda.synchronize()
    assert p.check_guards() == [], f"writes outside an output buffer: {p.check_guards()}"
    st, counts = P.full_check(p, inp)
    P.say(f"[parity] case={case} ok counts={counts.tolist()} band={st['band']} "
          f"band_mismatch={st['mismatch_in_band']} max_dI={st['max_dI']:.2e}")


# Launch variants of the score pass, passed to lsa_score_select_ex: the pair
# kernel (two waves per tile), the one-wave-per-tile kernel with other chunk
# sizes and LDS rings, and the full hi + lo pass on every tile.
SCORE_VARIANTS = {
    "pairs": {"kernel": "pairs"},
    "chunk2": {"kernel": "stream", "chunk_words": 2},
    "chunk3_ring8": {"chunk_words": 3, "ring": 8},
    "chunk5": {"chunk_words": 5},
    "guard": {"guard": 1},
    "guard_chunk2": {"guard": 1, "chunk_words": 2},
    "chunk4": {"chunk_words": 4},
    "chunk8": {"chunk_words": 8},
}


@pytest.mark.gpu
@pytest.mark.parametrize("variant", list(SCORE_VARIANTS))
@pytest.mark.parametrize("case", ["three_layer_mixed", "fp8_two_seq", "ragged_small", "bf16_16heads_d64"])
def test_score_variants(case, variant, torch_cuda):
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = SMALL[case]
    P.say(f"[variant] case={case} variant={variant}")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", with_scores=True, guard=True)
    p.score_options = SCORE_VARIANTS[variant]
    p.run()
    torch_cuda.cuda.synchronize()
    assert p.check_guards() == [], f"writes outside an output buffer: {p.check_guards()}"
    P.full_check(p, inp)


@pytest.mark.gpu
def test_repeat_is_deterministic(torch_cuda):
    """Two runs give bit-identical masks, lists, top-k and gather."""
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = SMALL["three_layer_mixed"]
    P.say("[parity] determinism")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", with_scores=True)
    snaps = []
    for _ in range(2):
        p.run()
        p.score_with_sigmoid()
        torch_cuda.cuda.synchronize()
        snaps.append([t.clone() for t in (p.masks + p.masks_scored + p.scores + [p.idx[: p.rows], p.count, p.topk_count]
                                          + p.topk_idx + p.topk_score + [p.gathered])])
    for a, b in zip(*snaps):
        assert torch_cuda.equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("rows,K", [(37, 96), (64, 4096), (16, 32)])
def test_pack_weights_layout(rows, K, torch_cuda):
    """lsa_pack_weights against the layout its header defines, written out with numpy."""
    from sparse_kv_retrieval_amd import lsa
    P.say(f"[parity] pack layout {rows}x{K}")
    rng = np.random.default_rng(rows * 7 + K)
    w = rng.integers(0, 1 << 16, (rows, K), dtype=np.uint64).astype(np.uint16)
    wd = torch_cuda.from_numpy(w.view(np.int16)).cuda()
    out = torch_cuda.empty(lsa.pack_weights_size(rows, K), dtype=torch_cuda.uint8, device="cuda")
    lsa.pack_weights(wd, rows, K, out)
    got = out.cpu().numpy().view(np.uint16)
    nrb, nch = (rows + 15) // 16, K // 32
    pad = np.zeros((nrb * 16, K), np.uint16)
    pad[:rows] = w
    # block (rb, ch), unit l = 16*kg + m: row 16rb + m, columns 32ch + 8kg .. + 7
    want = pad.reshape(nrb, 16, nch, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert np.array_equal(got, want)


@pytest.mark.gpu
def test_unpacked_projection_parity(torch_cuda):
    """The same path with plain out x in bf16 weights (lsa_project instead of lsa_project_packed)."""
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = SMALL["three_layer_mixed"]
    P.say("[parity] unpacked projection")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", with_scores=True, guard=True, packed=False)
    assert not p.packed
    p.run()
    torch_cuda.cuda.synchronize()
    assert p.check_guards() == []
    P.full_check(p, inp)


@pytest.mark.gpu
def test_graph_replay_matches_eager(torch_cuda):
    """The whole path captured in one HIP graph: every replay equals the eager run bit for bit."""
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = SMALL["three_layer_mixed"]
    P.say("[parity] graph replay")
    inp = synth.make(w)
    p = Pipeline(inp, "cuda", with_scores=True)
    p.run()
    torch_cuda.cuda.synchronize()

    def written():
        # the parts of the outputs a run writes: union lists hold count_b entries per region,
        # the gathered buffer holds sum(count) rows; everything else is written in full
        counts = p.count.cpu().numpy()
        parts = [t for t in p.outputs() if t is not p.idx and t is not getattr(p, "gathered", None)]
        parts += [p.idx[int(p.key_off_h[b]): int(p.key_off_h[b]) + int(counts[b])] for b in range(w.B)]
        parts.append(p.gathered[: int(counts.sum())])
        return [t.clone() for t in parts]

    want = written()
    g = p.capture()
    for rep in range(3):
        for t in p.outputs():  # eager work between replays: overwrite every output
            t.view(torch_cuda.uint8).fill_(0xA5 if rep % 2 else 0x3C)
        torch_cuda.cuda.synchronize()
        g.replay()
        torch_cuda.cuda.synchronize()
        for a, b in zip(written(), want):
            assert torch_cuda.equal(a, b), f"replay {rep} differs"


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["single_layer_500k", "three_layer_b8", "fp8_1m", "ragged_b32"])
def test_full_size(name, torch_cuda):
    """The workloads at their full sizes, in the launch configuration bench.py times, against the
    oracle on every output: every entry's mask bit (both score passes) and sigmoid score, every
    union list, every (layer, sequence)'s top-k, every gathered row."""
    from sparse_kv_retrieval_amd.pipeline import Pipeline
    w = W[name]
    P.say(f"[full] case={name}: generating")
    inp = synth.make(w)
    P.say(f"[full] case={name}: rows={int(inp.key_offsets[-1])} running")
    p = Pipeline(inp, "cuda", with_scores=True, guard=True)
    p.run()
    torch_cuda.cuda.synchronize()
    assert p.check_guards() == [], f"writes outside an output buffer: {p.check_guards()}"
    P.say(f"[full] case={name}: checking against the oracle")
    st, counts = P.full_check(p, inp)
    frac = counts.sum() / max(1, int(inp.key_offsets[-1]))
    P.say(f"[full] case={name}: ok, union fraction {frac:.4f}, band={st['band']} "
          f"band_mismatch={st['mismatch_in_band']} run_vs_scored={st['run_vs_scored']} max_dI={st['max_dI']:.2e}")
