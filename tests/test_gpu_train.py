"""lsa_train_step against the training-step oracle (marked gpu).

The oracle (oracle/train_oracle.train_step) works in float64 on the same bf16
inputs, decoded exactly. Tolerances, from the kernel's arithmetic:
  * the projections keep about 16 significant bits of q (c enters the second
    product as bf16 hi + lo), and the key scan keeps about 16 bits of q and of
    each gradient coefficient g_s w_j (hi + lo pairs), with fp32 accumulation;
    a head dot q_j . K_s is then within about 1e-5 of sum_i |q_ji| |K_si|;
  * the loss is a mean of smooth functions of x_s: relative error LOSS_RTOL;
  * a gradient element is a sum over ~10^5 to 10^6 terms of mixed signs, so
    its rounding error is judged against the matrix's largest element
    (ELEM_RTOL), plus the ReLU kink: a head dot within KINK_BAND of
    sum_i |q_ji| |K_si| may fall on either side of 0, which adds or drops the
    whole term g_s w_j K_s of dq. kink_allowance() sums the magnitudes of all
    such terms (from the oracle's own dots) and carries them through the later
    products, element by element. A transposed operand, a wrong head or a
    dropped term still gives errors far beyond both allowances.
"""
import dataclasses

import numpy as np
import pytest

from oracle import lsa_oracle as O
from oracle import train_oracle as TO
from sparse_kv_retrieval_amd import synth as S
from tests.parity import say

LOSS_RTOL = 1e-4
ELEM_RTOL = 1e-4
KINK_BAND = 1e-4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _workload(N, d=256, r=128, name="train_small", seed=21):
    base = S.WORKLOADS["train_b8"]
    return dataclasses.replace(S.scaled(base, N=N, name=name), d=d, r=r, L=1, seed=seed)


def run_gpu(torch, inp, words, gamma, alpha, layer=0, ws_fill=0x7F, labels_dev=None):
    from sparse_kv_retrieval_amd import lsa
    w = inp.workload
    dev = torch.device("cuda")

    def u16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    mw = inp.mem_w[layer]
    ko = torch.from_numpy(inp.key_offsets).to(dev)
    mo = torch.from_numpy(inp.mask_word_offsets).to(dev)
    if labels_dev is not None:
        labels = labels_dev
    elif words.size:
        labels = torch.from_numpy(words.view(np.int64)).to(dev)
    else:
        labels = torch.zeros(1, dtype=torch.int64, device=dev)
    keys = u16(inp.keys[layer]) if inp.keys[layer].size else torch.zeros(8, dtype=torch.int16, device=dev)
    # outputs start as garbage so that an unwritten element shows
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    g_dq = torch.full((w.r, w.d), float("nan"), dtype=torch.float32, device=dev)
    g_iuq = torch.full((w.n_h * w.d_h, w.r), float("nan"), dtype=torch.float32, device=dev)
    g_w = torch.full((w.n_h, w.d), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.full((lsa.train_workspace_size(w.B, inp.key_offsets, w.r),), ws_fill, dtype=torch.uint8, device=dev)
    lsa.train_step(h=u16(inp.h[layer]), w_dq=u16(mw.w_dq), w_iuq=u16(mw.w_iuq), w_w=u16(mw.w_w), keys=keys,
                   key_offsets=ko, key_offsets_host=inp.key_offsets, labels=labels, mask_word_offsets=mo,
                   mask_word_offsets_host=inp.mask_word_offsets, B=w.B, d=w.d, r=w.r, n_h=w.n_h, d_h=w.d_h,
                   gamma=gamma, alpha=alpha, loss=loss, g_dq=g_dq, g_iuq=g_iuq, g_w=g_w, workspace=ws)
    torch.cuda.synchronize()
    return (float(loss.item()), g_dq.cpu().numpy().astype(np.float64), g_iuq.cpu().numpy().astype(np.float64),
            g_w.cpu().numpy().astype(np.float64))


def run_oracle(inp, lab, gamma, alpha, layer=0):
    w = inp.workload
    mw = inp.mem_w[layer]
    keys, labels = [], []
    for b in range(w.B):
        s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
        keys.append(O.decode_keys(inp.keys[layer][s0:s1], "bf16"))
        labels.append(lab[s0:s1])
    return TO.train_step(O.decode_act(inp.h[layer], "bf16"), O.decode_act(mw.w_dq, "bf16"),
                         O.decode_act(mw.w_iuq, "bf16"), O.decode_act(mw.w_w, "bf16"), keys, labels,
                         w.n_h, w.d_h, gamma=gamma, alpha=alpha)


def kink_allowance(inp, lab, gamma, alpha, layer=0):
    """Element-wise bounds on what ReLU-kink decisions near 0 can move: (g_dq, g_iuq, g_w) arrays.

    A pair (entry s, head j) whose oracle dot lies within the band may flip; it
    then adds or drops t = g_s w_j K_s in row j of dq, t W^IUQ_j in dc (W^IUQ_j:
    the head's 128 rows of the w_iuq buffer), and their outer products with c
    and h in the gradients. The bound sums |t| and |t W^IUQ_j| over every
    such pair, so it holds whichever of them flip."""
    w = inp.workload
    mw = inp.mem_w[layer]
    H = O.decode_act(inp.h[layer], "bf16")
    Wdq, Wiuq, Ww = (O.decode_act(m, "bf16") for m in (mw.w_dq, mw.w_iuq, mw.w_w))
    c, q, gate = O.project(H, Wdq, Wiuq, Ww, w.n_h, w.d_h)
    total = max(int(inp.key_offsets[-1] - inp.key_offsets[0]), 1)
    a_dq = np.zeros((w.B, w.n_h, w.d_h))
    a_dc = np.zeros((w.B, w.r))
    for b in range(w.B):
        s0, s1 = int(inp.key_offsets[b]), int(inp.key_offsets[b + 1])
        if s1 == s0:
            continue
        K = O.decode_keys(inp.keys[layer][s0:s1], "bf16")
        dots = K @ q[b].T
        band = np.abs(dots) <= KINK_BAND * (np.abs(K) @ np.abs(q[b]).T)
        g = TO.focal_grad(np.maximum(dots, 0.0) @ gate[b], lab[s0:s1], gamma, alpha) / total
        for j in np.flatnonzero(band.any(axis=0)):
            rows = np.flatnonzero(band[:, j])
            t = np.abs(g[rows] * gate[b][j])[:, None] * K[rows]              # [pairs, d_h] flipped terms
            a_dq[b, j] = np.abs(t).sum(axis=0)
            a_dc[b] += np.abs(t @ Wiuq[j * w.d_h:(j + 1) * w.d_h]).sum(axis=0)
    a_iuq = a_dq.reshape(w.B, -1).T @ np.abs(c)
    return a_dc.T @ np.abs(H), a_iuq, np.zeros((w.n_h, w.d))


def compare(got, ref, allow, tag):
    loss, *gg = got
    rloss, *rg = ref
    assert np.isfinite(loss), f"{tag}: loss not finite"
    assert abs(loss - rloss) <= LOSS_RTOL * abs(rloss) + 1e-12, f"{tag}: loss {loss} vs {rloss}"
    errs = {}
    for name, g, r, a in zip(("g_dq", "g_iuq", "g_w"), gg, rg, allow):
        assert np.isfinite(g).all(), f"{tag}: {name} has unwritten or non-finite elements"
        scale = np.abs(r).max()
        if scale == 0.0:
            assert not g.any(), f"{tag}: {name} should be 0"
            errs[name] = 0.0
            continue
        err = np.abs(g - r)
        bad = err > ELEM_RTOL * scale + a
        errs[name] = (float(np.linalg.norm(g - r) / np.linalg.norm(r)), float(err.max() / scale),
                      float(a.max() / scale))
        assert not bad.any(), (f"{tag}: {name} differs at {np.argwhere(bad)[:5].tolist()}: "
                               f"max error {err.max() / scale} of the largest element")
    say(f"{tag}: loss {loss:.6g} (oracle {rloss:.6g}) [fro, max elem, max kink allowance]: {errs}")
    return errs


SMALL = {
    # several tiles and scan blocks, a 1-entry tail block, an empty and a 1-entry sequence
    "ragged": dict(N=(1000, 33, 0, 2049, 1), flip=0.05),
    "one_block_exact": dict(N=(1024,), flip=0.02),
    "many_seq": dict(N=tuple(int(x) for x in np.random.default_rng(5).integers(0, 3000, size=32)), flip=0.03),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_train_small(torch_cuda, case):
    cfg = SMALL[case]
    w = _workload(cfg["N"], name="train_" + case)
    say(f"train_small {case}: B={w.B} N={w.N}")
    inp = S.make(w, with_pool=False)
    lab, words = S.train_labels(inp, 0, cfg["flip"])
    compare(run_gpu(torch_cuda, inp, words, 2.0, 0.25), run_oracle(inp, lab, 2.0, 0.25),
            kink_allowance(inp, lab, 2.0, 0.25), case)


@pytest.mark.parametrize("gamma,alpha", [(0.0, 0.5), (0.0, 0.25), (1.5, 0.25), (2.0, 1.0), (3.0, 0.0)])
def test_train_parameters(torch_cuda, gamma, alpha):
    w = _workload((700, 1500), name="train_params", seed=22)
    say(f"train_parameters gamma={gamma} alpha={alpha}")
    inp = S.make(w, with_pool=False)
    lab, words = S.train_labels(inp, 0, 0.1)
    compare(run_gpu(torch_cuda, inp, words, gamma, alpha), run_oracle(inp, lab, gamma, alpha),
            kink_allowance(inp, lab, gamma, alpha), f"gamma={gamma} alpha={alpha}")


def test_train_no_entries(torch_cuda):
    w = _workload((0, 0), name="train_empty")
    say("train_no_entries")
    inp = S.make(w, with_pool=False)
    lab, words = S.train_labels(inp, 0, 0.1)
    loss, g_dq, g_iuq, g_w = run_gpu(torch_cuda, inp, words, 2.0, 0.25)
    assert loss == 0.0 and not g_dq.any() and not g_iuq.any() and not g_w.any()


def test_train_wide_shape(torch_cuda):
    """d and r not multiples of the outer-product tiles (256 columns, 32 rows)."""
    w = _workload((3000, 77), d=32 * 23, r=32 * 9, name="train_wide", seed=23)
    say(f"train_wide_shape d={w.d} r={w.r}")
    inp = S.make(w, with_pool=False)
    lab, words = S.train_labels(inp, 0, 0.05)
    compare(run_gpu(torch_cuda, inp, words, 2.0, 0.25), run_oracle(inp, lab, 2.0, 0.25),
            kink_allowance(inp, lab, 2.0, 0.25), "wide")


def test_train_full_size(torch_cuda):
    """The 8 x 125K-entry batch, d = 4096, r = 2048: every gradient element checked."""
    w = S.WORKLOADS["train_b8"]
    say(f"train_full_size {w.name} B={w.B} N={w.N[0]}")
    inp = S.make(w, with_pool=False)
    lab, words = S.train_labels(inp, 0, 0.02)
    got = run_gpu(torch_cuda, inp, words, 2.0, 0.25)
    say("  gpu done")
    compare(got, run_oracle(inp, lab, 2.0, 0.25), kink_allowance(inp, lab, 2.0, 0.25), "full")


def test_train_deterministic_and_workspace_independent(torch_cuda):
    """Two calls give the same bits, whatever the workspace held before (the split projection adds two
    partial sums into zeroed outputs, which rounds the same in either order)."""
    from sparse_kv_retrieval_amd import lsa
    w = _workload((5000, 1234), name="train_det", seed=24)
    say("train_deterministic")
    inp = S.make(w, with_pool=False)
    lab, words = S.train_labels(inp, 0, 0.05)
    first = run_gpu(torch_cuda, inp, words, 2.0, 0.25)
    second = run_gpu(torch_cuda, inp, words, 2.0, 0.25, ws_fill=0xFF)  # NaN patterns instead of 0x7F bytes
    assert first[0] == second[0]
    for a, b in zip(first[1:], second[1:]):
        assert np.array_equal(a, b)
    assert lsa.train_workspace_size(w.B, inp.key_offsets, w.r) > 0


@pytest.mark.parametrize("kind", ["all_golden", "no_golden", "saturated"])
def test_train_label_and_logit_extremes(torch_cuda, kind):
    """Every entry golden, none golden, and logits in the hundreds (h scaled by 8: the sigmoid
    saturates, the focal weights vanish for the easy entries)."""
    w = _workload((2100, 300), name="train_" + kind, seed=25)
    say(f"train_extremes {kind}")
    inp = S.make(w, with_pool=False)
    lab, _ = S.train_labels(inp, 0, 0.05)
    if kind == "all_golden":
        lab = np.ones_like(lab)
    elif kind == "no_golden":
        lab = np.zeros_like(lab)
    else:
        inp.h[0] = S.f32_to_bf16_bits(S.bf16_bits_to_f32(inp.h[0]) * np.float32(8.0))
    words = S.pack_mask_words(lab, inp.key_offsets, inp.mask_word_offsets)
    compare(run_gpu(torch_cuda, inp, words, 2.0, 0.25), run_oracle(inp, lab, 2.0, 0.25),
            kink_allowance(inp, lab, 2.0, 0.25), kind)


def test_train_on_mined_labels(torch_cuda):
    """Labels straight from golden-label mining: lsa_golden_labels writes the window's label set in the
    same bit layout that lsa_train_step reads, so the mined words feed the training step on the device.
    The mined set is judged as the mining tests judge it (the golden-label oracle's bounds: entries whose
    nucleus mass lies within rounding of p may fall either way), and the training oracle then trains on
    the GPU's mined labels, so the training comparison does not depend on how those entries fell."""
    from oracle import golden_oracle as G
    from sparse_kv_retrieval_amd import lsa
    from sparse_kv_retrieval_amd import synth_golden as SG
    dev = torch_cuda.device("cuda")
    gw = SG.WORKLOADS["golden_small"]
    gi = SG.make(gw)
    W = gw.words
    golden = torch_cuda.full((W,), -1, dtype=torch_cuda.int64, device=dev)
    lsa.golden_labels(torch_cuda.from_numpy(gi.logits).to(dev), row_stride=gw.row_stride, T=gw.T, L=gw.L,
                      n_valid=torch_cuda.from_numpy(gi.n_valid).to(dev), top_p=gw.p, theta=gw.theta,
                      row_mask=torch_cuda.empty((gw.T * gw.L, W), dtype=torch_cuda.int64, device=dev), golden=golden,
                      workspace=torch_cuda.empty(lsa.golden_workspace_size(gw.T, gw.L, gw.row_stride),
                                                 dtype=torch_cuda.uint8, device=dev))
    torch_cuda.cuda.synchronize()
    sure, never = G.golden_bounds(gi.logits, gi.n_valid, gw.p, gw.theta, 1e-5)
    N = sure.size
    bits = np.unpackbits(golden.cpu().numpy().view(np.uint8), bitorder="little").astype(bool)
    mined = bits[:N]
    assert not (sure & ~mined).any() and not (never & mined).any() and not bits[N:W * 64].any(), \
        "mined label set outside the oracle's bounds"
    lab = mined  # the GPU's labels feed both sides of the training comparison
    w = _workload((N,), name="train_mined", seed=26)
    say(f"train_on_mined_labels: N={N}, {int(lab.sum())} golden")
    inp = S.make(w, with_pool=False)
    assert int(inp.mask_word_offsets[-1]) == (N + 63) // 64 <= W
    got = run_gpu(torch_cuda, inp, np.zeros(0, np.uint64), 2.0, 0.25, labels_dev=golden[:(N + 63) // 64])
    compare(got, run_oracle(inp, lab, 2.0, 0.25), kink_allowance(inp, lab, 2.0, 0.25), "mined")
