"""Host-side C-ABI checks. They need no GPU: every call here is rejected by
argument validation before anything touches the device."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")


@pytest.fixture(scope="module")
def lsa():
    from sparse_kv_retrieval_amd import lsa as mod
    return mod


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for f in ("lsa_project", "lsa_score_select", "lsa_union_compact", "lsa_topk", "lsa_gather",
              "lsa_topk_workspace_size", "lsa_pack_weights_size", "lsa_pack_weights", "lsa_project_packed",
              "lsa_topk_score", "lsa_topk_select", "lsa_score_select_ex", "lsa_topk_step",
              "lsa_topk_step_noalloc", "lsa_debug_range_errors",
              "lsa_last_error", "lsa_version"):
        assert f in fns


def test_library_exports_every_declared_symbol(lsa):
    lib = ctypes.CDLL(lsa.LIB_PATH)
    for f in declared_functions():
        assert hasattr(lib, f), f
    out = subprocess.run(["nm", "-D", "--defined-only", lsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (lsa_\w+)", out))
    assert set(declared_functions()) == exported, exported ^ set(declared_functions())
    assert set(lsa.EXPORTED) == exported


def test_version(lsa):
    assert lsa.version() == 2


def test_release_build_has_no_range_checks(lsa):
    # the product library compiles no device range checks, and the query says so before any HIP call
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.debug_range_errors, stream=0, match="range checks")


def test_debug_build_exports_every_declared_symbol():
    lib = os.path.join(ROOT, "sparse_kv_retrieval_amd", "_debug", "sparse_kv_retrieval_amd", "liblsa.so")
    if not os.path.exists(lib):
        subprocess.run([sys.executable, "-c", "from sparse_kv_retrieval_amd import build; build.build_debug()"],
                       cwd=ROOT, check=True)
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True).stdout
    assert set(re.findall(r"\bT (lsa_\w+)", out)) == set(declared_functions())


def _offs(n):
    ko = np.zeros(len(n) + 1, np.int64)
    ko[1:] = np.cumsum(n)
    mw = np.zeros(len(n) + 1, np.int64)
    mw[1:] = np.cumsum((np.asarray(n) + 63) // 64)
    return ko, mw


FAKE = 1 << 20  # non-null, 16-byte aligned stand-in address (never dereferenced: validation fails first)


def _score_layer(**kw):
    d = dict(q=FAKE, w=FAKE, keys=FAKE, key_scale=None, mask_out=FAKE, score_out=None)
    d.update(kw)
    return d


def _expect(lsa, status, fn, *a, match=None, **kw):
    with pytest.raises(lsa.LsaError) as ei:
        fn(*a, **kw)
    assert ei.value.status == status, str(ei.value)
    if match:
        assert re.search(match, str(ei.value)), str(ei.value)


def test_score_select_validation(lsa):
    ko, mw = _offs([100, 0, 65])
    base = dict(B=3, key_offsets=FAKE, key_offsets_host=ko, mask_word_offsets=FAKE, mask_word_offsets_host=mw,
                n_h=64, d_h=128, key_dtype="bf16", threshold=0.5, stream=0)
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer(q=None)], **base, match="must be set")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.score_select, [_score_layer()], **{**base, "d_h": 96}, match="d_h")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.score_select, [_score_layer()], **{**base, "n_h": 65}, match="n_h")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.score_select, [_score_layer()], **{**base, "key_dtype": 7})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()], **{**base, "threshold": 1.0})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()], **{**base, "threshold": 0.0})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()] * 9, **base, match="L must")
    bad = ko.copy(); bad[2] = 50
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()], **{**base, "key_offsets_host": bad},
            match="decreasing")
    badw = mw.copy(); badw[1] += 1; badw[2] += 1; badw[3] += 1
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()], **{**base, "mask_word_offsets_host": badw},
            match="ceil")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()], **{**base, "key_dtype": "fp8"},
            match="key_scale")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer(key_scale=FAKE)], **base, match="only for fp8")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer(keys=FAKE + 4)], **base, match="aligned")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()], **{**base, "B": 0})
    assert "B must" in lsa.last_error()
    # lsa_score_select_ex: the same checks, then the options
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer(q=None)], **base, options={}, match="must be set")
    for bad_opt, what in (({"kernel": 3}, "kernel"), ({"chunk_words": 1}, "chunk_words"),
                          ({"chunk_words": 65}, "chunk_words"), ({"ring": 6}, "ring"), ({"guard": 2}, "guard")):
        _expect(lsa, lsa.ERR_INVALID_ARG, lsa.score_select, [_score_layer()], **base, options=bad_opt, match=what)
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.score_select, [_score_layer()], **{**base, "key_dtype": "f32"},
            options={"kernel": "stream"}, match="one-wave-per-tile")


def test_project_validation(lsa):
    lay = dict(h=FAKE, w_dq=FAKE, w_iuq=FAKE, w_w=FAKE, c_out=FAKE + 4096, q_out=FAKE + 8192, w_out=FAKE + 16384)
    base = dict(B=8, d=4096, r=2048, n_h=64, d_h=128, dtype="bf16", stream=0)
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.project, [{**lay, "h": None}], **base)
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.project, [lay], **{**base, "d": 4001}, match="multiples")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.project, [lay], **{**base, "B": 129})
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.project, [lay], **{**base, "dtype": "fp8"})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.project, [{**lay, "q_out": lay["c_out"]}], **base, match="alias")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.project, [lay], **{**base, "n_h": 3, "d_h": 5})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.project, [{**lay, "w_w": FAKE + 8}], **base, match="aligned")


def test_packed_projection_validation(lsa):
    assert lsa.pack_weights_size(2048, 4096) == 128 * 128 * 1024
    assert lsa.pack_weights_size(64, 4096) == 4 * 128 * 1024
    assert lsa.pack_weights_size(65, 4096) == 5 * 128 * 1024   # rows padded to a multiple of 16
    assert lsa.pack_weights_size(64, 4010) == 0                 # K not a multiple of 32
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.pack_weights, FAKE, 64, 4010, FAKE, out_bytes=1 << 30, stream=0)
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.pack_weights, FAKE, 64, 4096, FAKE, out_bytes=1000, stream=0,
            match="needs")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.pack_weights, FAKE + 2, 64, 4096, FAKE, out_bytes=1 << 30, stream=0,
            match="aligned")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.pack_weights, None, 64, 4096, FAKE, out_bytes=1 << 30, stream=0)
    lay = dict(h=FAKE, w_dq=FAKE, w_iuq=FAKE, w_w=FAKE, c_out=FAKE + 4096, q_out=FAKE + 8192, w_out=FAKE + 16384)
    base = dict(B=8, d=4096, r=2048, n_h=64, d_h=128, stream=0)
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.project_packed, [lay], **{**base, "B": 33}, match="B must")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.project_packed, [lay], **{**base, "r": 2016}, match="multiple")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.project_packed, [lay], **{**base, "n_h": 3, "d_h": 5})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.project_packed, [{**lay, "w_w": FAKE + 8}], **base, match="aligned")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.project_packed, [{**lay, "w_out": lay["c_out"]}], **base, match="alias")


def test_union_topk_gather_validation(lsa):
    ko, mw = _offs([10, 20])
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.union_compact, [FAKE, None], B=2, key_offsets=FAKE, key_offsets_host=ko,
            mask_word_offsets=FAKE, mask_word_offsets_host=mw, idx_out=FAKE, count_out=FAKE, stream=0)
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.union_compact, [FAKE], B=2, key_offsets=FAKE, key_offsets_host=ko,
            mask_word_offsets=FAKE, mask_word_offsets_host=mw, idx_out=None, count_out=FAKE, stream=0)
    tl = dict(q=FAKE, w=FAKE, keys=FAKE, key_scale=None, topk_idx_out=FAKE, topk_score_out=None)
    tb = dict(B=2, key_offsets=FAKE, key_offsets_host=ko, idx=FAKE, count=FAKE, n_h=64, d_h=128, key_dtype="bf16",
              k=2048, topk_count_out=FAKE, stream=0)

    class _WS:  # a workspace tensor stand-in that is too small
        def numel(self):
            return 4

        def element_size(self):
            return 1

        def data_ptr(self):
            return FAKE
    _expect(lsa, lsa.ERR_WORKSPACE, lsa.topk, [tl], **tb, workspace=_WS(), match="workspace")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.topk, [tl], **{**tb, "k": 0}, workspace=_WS())
    # scores [L][rows] fp32, then (256-byte aligned) 2048-bin histograms per (layer, sequence)
    assert lsa.topk_workspace_size(3, 2, 30, 2048) == 512 + 3 * 2 * 2048 * 4
    assert lsa.topk_workspace_size(3, 0, 30, 2048) == 0
    # the allocation-free variant refuses a call whose scratch exceeds its fixed array, before any HIP call
    big = np.array([0, 5_000_000, 10_000_000], np.int64)
    nb = {k_: v for k_, v in tb.items() if k_ not in ("key_offsets_host",)}
    assert lsa.topk_workspace_size(1, 2, 10_000_000, 2048) > lsa.NOALLOC_SCRATCH_BYTES
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.topk_step_noalloc, [tl], **nb, key_offsets_host=big, match="scratch")
    # the per-step top-k over packed subset keys: the same checks, and at most 1024 sequences
    _expect(lsa, lsa.ERR_WORKSPACE, lsa.topk_step, [tl], **tb, workspace=_WS(), match="workspace")
    ko1025 = np.arange(1026, dtype=np.int64)
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.topk_step, [tl], **{**tb, "B": 1025, "key_offsets_host": ko1025},
            workspace=_WS(), match="B must")
    # the two stages of the top-k check what each reads
    class _WSBig(_WS):  # a workspace stand-in that is large enough
        def numel(self):
            return 1 << 20
    sb = {k_: v for k_, v in tb.items() if k_ not in ("k", "topk_count_out")}
    _expect(lsa, lsa.ERR_WORKSPACE, lsa.topk_score, [tl], **sb, workspace=_WS(), match="workspace")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.topk_score, [tl], **{**sb, "d_h": 96}, workspace=_WS(), match="d_h")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.topk_score, [{**tl, "keys": None}], **sb, workspace=_WSBig(),
            match="must be set")
    xb = {k_: v for k_, v in tb.items() if k_ not in ("n_h", "d_h", "key_dtype")}
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.topk_select, [tl], **{**xb, "k": 0}, workspace=_WS())
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.topk_select, [{**tl, "topk_idx_out": None}], **xb, workspace=_WSBig(),
            match="topk_idx_out")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.topk_select, [tl], **{**xb, "topk_count_out": None}, workspace=_WS())
    _expect(lsa, lsa.ERR_WORKSPACE, lsa.topk_select, [tl], **xb, workspace=_WS(), match="workspace")
    gb = dict(row_bytes=1024, B=2, pool_row_offsets=FAKE, pool_row_offsets_host=ko, idx=FAKE, idx_offsets=FAKE,
              count=FAKE, out=FAKE, out_capacity_rows=30, stream=0)
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.gather, FAKE, **{**gb, "row_bytes": 1000}, match="multiple of 16")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.gather, None, **gb)
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.gather, FAKE + 8, **gb, match="aligned")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.gather, FAKE, **{**gb, "out_capacity_rows": -1})
    # the host-pool fetch checks its pool before asking the runtime about it
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.fetch_host, None, **gb, match="NULL")


class _Buf:
    """A device-buffer stand-in of a given size (never dereferenced: validation fails first)."""
    def __init__(self, nbytes, ptr=FAKE):
        self.n, self.ptr = nbytes, ptr

    def numel(self):
        return self.n

    def element_size(self):
        return 1

    def data_ptr(self):
        return self.ptr


def test_golden_labels_validation(lsa):
    need = lsa.golden_workspace_size(4, 21, 1000)
    assert need > 0 and lsa.golden_workspace_size(4, 21, 70000) > need
    assert lsa.golden_workspace_size(0, 21, 1000) == 0
    ws = _Buf(need)
    gb = dict(row_stride=1000, T=4, L=21, n_valid=FAKE, top_p=0.6, theta=3, row_mask=FAKE, golden=FAKE,
              workspace=ws, stream=0)
    _expect(lsa, lsa.ERR_WORKSPACE, lsa.golden_labels, FAKE, **{**gb, "workspace": _Buf(need - 1)},
            match="workspace")
    _expect(lsa, lsa.ERR_WORKSPACE, lsa.golden_labels, FAKE, **{**gb, "workspace": None}, match="workspace")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "workspace": _Buf(need, FAKE + 8)},
            match="aligned")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, None, **gb, match="must be set")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "golden": None}, match="must be set")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "n_valid": None}, match="must be set")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "L": 65}, match="L <= 64")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "T": 0})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "top_p": 0.0}, match="top_p")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "top_p": 1.5}, match="top_p")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "top_p": float("nan")}, match="top_p")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "theta": 0}, match="theta")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.golden_labels, FAKE, **{**gb, "row_stride": 0}, match="row_stride")
    _expect(lsa, lsa.ERR_UNSUPPORTED, lsa.golden_labels, FAKE, **{**gb, "row_stride": (1 << 28) + 1,
                                                                     "workspace": _Buf(1 << 40)})
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE + 2, **gb, match="aligned")
    _expect(lsa, lsa.ERR_INVALID_ARG, lsa.golden_labels, FAKE, **{**gb, "row_mask": FAKE + 4}, match="aligned")


def test_train_step_validation(lsa):
    ko = np.array([0, 1000, 1000, 3049], np.int64)
    mo = np.array([0, 16, 16, 49], np.int64)
    need = lsa.train_workspace_size(3, ko, 128)
    assert need > 0 and lsa.train_workspace_size(3, np.array([0, 1000, 1000, 300000]), 128) > need
    assert lsa.train_workspace_size(0, ko, 128) == 0
    tb = dict(h=FAKE, w_dq=FAKE, w_iuq=FAKE, w_w=FAKE, keys=FAKE, key_offsets=FAKE, key_offsets_host=ko,
              labels=FAKE, mask_word_offsets=FAKE, mask_word_offsets_host=mo, B=3, d=256, r=128, n_h=64, d_h=128,
              gamma=2.0, alpha=0.25, loss=FAKE, g_dq=FAKE, g_iuq=FAKE, g_w=FAKE, workspace=_Buf(need), stream=0)

    def bad(st, match=None, **kw):
        _expect(lsa, st, lsa.train_step, **{**tb, **kw}, match=match)

    bad(lsa.ERR_WORKSPACE, "workspace", workspace=_Buf(need - 1))
    bad(lsa.ERR_WORKSPACE, "workspace", workspace=None)
    bad(lsa.ERR_INVALID_ARG, "aligned", workspace=_Buf(need, FAKE + 8))
    for name in ("h", "w_dq", "w_iuq", "w_w", "keys", "labels", "loss", "g_dq", "g_iuq", "g_w"):
        bad(lsa.ERR_INVALID_ARG, "must be set", **{name: None})
    bad(lsa.ERR_INVALID_ARG, "aligned", h=FAKE + 2)
    bad(lsa.ERR_INVALID_ARG, "aligned", keys=FAKE + 8)
    bad(lsa.ERR_INVALID_ARG, "aligned", w_w=FAKE + 8)
    bad(lsa.ERR_INVALID_ARG, "aligned", labels=FAKE + 4)
    bad(lsa.ERR_INVALID_ARG, "aligned", g_iuq=FAKE + 4)
    bad(lsa.ERR_UNSUPPORTED, "B must be", B=0)
    bad(lsa.ERR_UNSUPPORTED, "B must be", B=33)
    bad(lsa.ERR_UNSUPPORTED, "n_h = 64", n_h=32)
    bad(lsa.ERR_UNSUPPORTED, "n_h = 64", d_h=64)
    bad(lsa.ERR_UNSUPPORTED, "multiples of 32", d=250)
    bad(lsa.ERR_UNSUPPORTED, "multiples of 32", r=0)
    bad(lsa.ERR_INVALID_ARG, "gamma", gamma=-1.0)
    bad(lsa.ERR_INVALID_ARG, "gamma", gamma=float("nan"))
    bad(lsa.ERR_INVALID_ARG, "alpha", alpha=1.5)
    bad(lsa.ERR_INVALID_ARG, "ceil", mask_word_offsets_host=np.array([0, 15, 15, 48], np.int64))
    bad(lsa.ERR_INVALID_ARG, "decreasing", key_offsets_host=np.array([0, 1000, 999, 3049], np.int64))
    long_ko = np.array([0, 1 << 23, 1 << 23, 1 << 23], np.int64)
    long_mo = np.array([0, (1 << 23) // 64] * 1 + [(1 << 23) // 64] * 2, np.int64)
    bad(lsa.ERR_UNSUPPORTED, "longer", key_offsets_host=long_ko, mask_word_offsets_host=long_mo,
        workspace=_Buf(1 << 40))


def test_binding_has_no_oracle_import():
    """The product path (binding, pipeline, library sources) never refers to the oracle."""
    pkg = os.path.join(ROOT, "sparse_kv_retrieval_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", txt, re.M), f
                assert "lsa_oracle" not in txt and "golden_oracle" not in txt and "train_oracle" not in txt, f
