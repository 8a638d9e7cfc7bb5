"""Python binding for `liblsa.so` (the C-ABI declared in include/lsa.h).

This module only marshals arguments. Every step of the selection path runs in
the library's HIP kernels. Tensors are passed by `data_ptr()`, `*_host` offset
arrays are int64 numpy arrays (or CPU tensors), and the stream defaults to
torch's current stream. If the library has not been built, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsa.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
MAX_LAYERS = 8
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4


class LsaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first (__graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class ProjLayer(ctypes.Structure):
    _fields_ = [("h", _vp), ("w_dq", _vp), ("w_iuq", _vp), ("w_w", _vp),
                ("c_out", _vp), ("q_out", _vp), ("w_out", _vp)]


class ScoreLayer(ctypes.Structure):
    _fields_ = [("q", _vp), ("w", _vp), ("keys", _vp), ("key_scale", _vp),
                ("mask_out", _vp), ("score_out", _vp)]


class ScoreOptions(ctypes.Structure):
    _fields_ = [("kernel", _i32), ("chunk_words", _i32), ("ring", _i32), ("guard", _i32)]


SCORE_KERNELS = {"auto": 0, "stream": 1, "pairs": 2}


class TopkLayer(ctypes.Structure):
    _fields_ = [("q", _vp), ("w", _vp), ("keys", _vp), ("key_scale", _vp),
                ("topk_idx_out", _vp), ("topk_score_out", _vp)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_project = _sig("lsa_project", _i32, [ctypes.POINTER(ProjLayer), _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp])
_pack_size = _sig("lsa_pack_weights_size", _sz, [_i32, _i32])
_pack = _sig("lsa_pack_weights", _i32, [_vp, _i32, _i32, _vp, _sz, _vp])
_project_packed = _sig("lsa_project_packed", _i32, [ctypes.POINTER(ProjLayer), _i32, _i32, _i32, _i32, _i32, _i32,
                                                     _vp])
_score_select = _sig("lsa_score_select", _i32, [ctypes.POINTER(ScoreLayer), _i32, _i32, _vp, _vp, _vp, _vp,
                                                 _i32, _i32, _i32, _f32, _vp])
_score_select_ex = _sig("lsa_score_select_ex", _i32, [ctypes.POINTER(ScoreLayer), _i32, _i32, _vp, _vp, _vp, _vp,
                                                       _i32, _i32, _i32, _f32, ctypes.POINTER(ScoreOptions), _vp])
_union_compact = _sig("lsa_union_compact", _i32, [ctypes.POINTER(_vp), _i32, _i32, _vp, _vp, _vp, _vp,
                                                   _vp, _vp, _vp, _vp])
_topk_ws = _sig("lsa_topk_workspace_size", _sz, [_i32, _i32, _i64, _i32])
_topk = _sig("lsa_topk", _i32, [ctypes.POINTER(TopkLayer), _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _vp, _vp, _sz, _vp])
_topk_score = _sig("lsa_topk_score", _i32, [ctypes.POINTER(TopkLayer), _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                             _i32, _vp, _sz, _vp])
_topk_step = _sig("lsa_topk_step", _i32, [ctypes.POINTER(TopkLayer), _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                           _i32, _i32, _vp, _vp, _sz, _vp])
_topk_step_noalloc = _sig("lsa_topk_step_noalloc", _i32, [ctypes.POINTER(TopkLayer), _i32, _i32, _vp, _vp, _vp, _vp,
                                                           _i32, _i32, _i32, _i32, _vp, _vp])
_topk_select = _sig("lsa_topk_select", _i32, [ctypes.POINTER(TopkLayer), _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp,
                                               _vp, _sz, _vp])
_gather = _sig("lsa_gather", _i32, [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp])
_fetch_host = _sig("lsa_fetch_host", _i32, [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp])
_golden_ws = _sig("lsa_golden_workspace_size", _sz, [_i32, _i32, _i64])
_golden = _sig("lsa_golden_labels", _i32, [_vp, _i64, _i32, _i32, _vp, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _sz,
                                           _vp])
_train_ws = _sig("lsa_train_workspace_size", _sz, [_i32, _vp, _i32])
_train = _sig("lsa_train_step", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                       _i32, _f32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_debug_range_errors = _sig("lsa_debug_range_errors", _i32, [_vp, ctypes.POINTER(_i64)])
_last_error = _sig("lsa_last_error", ctypes.c_char_p, [])
_version = _sig("lsa_version", _i32, [])

EXPORTED = ("lsa_project", "lsa_pack_weights_size", "lsa_pack_weights", "lsa_project_packed", "lsa_score_select",
            "lsa_score_select_ex", "lsa_topk_step", "lsa_topk_step_noalloc",
            "lsa_topk_score", "lsa_topk_select", "lsa_union_compact", "lsa_topk_workspace_size", "lsa_topk",
            "lsa_gather", "lsa_fetch_host", "lsa_golden_workspace_size", "lsa_golden_labels", "lsa_train_workspace_size",
            "lsa_train_step", "lsa_debug_range_errors", "lsa_last_error",
            "lsa_version")


def last_error() -> str:
    return _last_error().decode()


def version() -> int:
    return int(_version())


def debug_range_errors(stream=None) -> int:
    """lsa_debug_range_errors: out-of-range list entries met since the last call (debug builds only;
    waits for the stream)."""
    n = _i64(0)
    _check("lsa_debug_range_errors", _debug_range_errors(_stream(stream), ctypes.byref(n)))
    return int(n.value)


def _p(t):
    """Device pointer of a tensor (or None/int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _host64(a):
    """Host int64 array -> (keep-alive object, pointer)."""
    if a is None:
        return None, None
    if hasattr(a, "numpy"):
        a = a.detach().cpu().numpy()
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return arr, arr.ctypes.data


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    """Size in bytes of a tensor (0 for None)."""
    return 0 if t is None else t.numel() * t.element_size()


def _check(fn, st):
    if st != OK:
        raise LsaError(fn, st, last_error())


def project(layers, *, B, d, r, n_h, d_h, dtype, stream=None):
    """lsa_project. `layers`: list of dicts with h, w_dq, w_iuq, w_w, c_out, q_out, w_out tensors."""
    arr = (ProjLayer * len(layers))(*[ProjLayer(*[_p(x[k]) for k in ("h", "w_dq", "w_iuq", "w_w", "c_out",
                                                                      "q_out", "w_out")]) for x in layers])
    _check("lsa_project", _project(arr, len(layers), B, d, r, n_h, d_h, DTYPES.get(dtype, dtype), _stream(stream)))


def pack_weights_size(rows, K) -> int:
    """lsa_pack_weights_size: bytes of the packed operand layout of a rows x K bf16 matrix."""
    return int(_pack_size(rows, K))


def pack_weights(w, rows, K, out, out_bytes=None, stream=None):
    """lsa_pack_weights: `w` a [rows, K] bf16 (int16 bits) tensor, `out` a byte tensor of pack_weights_size bytes."""
    if out_bytes is None:
        out_bytes = out.numel() * out.element_size()
    _check("lsa_pack_weights", _pack(_p(w), rows, K, _p(out), int(out_bytes), _stream(stream)))


def project_packed(layers, *, B, d, r, n_h, d_h, stream=None):
    """lsa_project_packed: as project(), with w_dq, w_iuq, w_w packed by pack_weights (bf16)."""
    arr = (ProjLayer * len(layers))(*[ProjLayer(*[_p(x[k]) for k in ("h", "w_dq", "w_iuq", "w_w", "c_out",
                                                                      "q_out", "w_out")]) for x in layers])
    _check("lsa_project_packed", _project_packed(arr, len(layers), B, d, r, n_h, d_h, _stream(stream)))


def score_select(layers, *, B, key_offsets, key_offsets_host, mask_word_offsets, mask_word_offsets_host,
                 n_h, d_h, key_dtype, threshold=0.5, options=None, stream=None):
    """lsa_score_select. `layers`: dicts with q, w, keys, key_scale (fp8), mask_out, score_out (optional).

    With `options` (a dict with any of kernel ("auto", "stream", "pairs"), chunk_words, ring, guard),
    lsa_score_select_ex with those launch options instead."""
    arr = (ScoreLayer * len(layers))(*[ScoreLayer(_p(x["q"]), _p(x["w"]), _p(x["keys"]), _p(x.get("key_scale")),
                                                  _p(x["mask_out"]), _p(x.get("score_out"))) for x in layers])
    ko, kop = _host64(key_offsets_host)
    mo, mop = _host64(mask_word_offsets_host)
    args = (arr, len(layers), B, _p(key_offsets), kop, _p(mask_word_offsets), mop, n_h, d_h,
            DTYPES.get(key_dtype, key_dtype), float(threshold))
    if options is None:
        _check("lsa_score_select", _score_select(*args, _stream(stream)))
        return
    o = ScoreOptions(SCORE_KERNELS.get(options.get("kernel", 0), options.get("kernel", 0)),
                     int(options.get("chunk_words", 0)), int(options.get("ring", 0)), int(options.get("guard", 0)))
    _check("lsa_score_select_ex", _score_select_ex(*args, ctypes.byref(o), _stream(stream)))


def union_compact(masks, *, B, key_offsets, key_offsets_host, mask_word_offsets, mask_word_offsets_host,
                  idx_out, count_out, union_mask_out=None, stream=None):
    """lsa_union_compact over a list of per-layer mask tensors."""
    marr = (_vp * len(masks))(*[_p(m) for m in masks])
    ko, kop = _host64(key_offsets_host)
    mo, mop = _host64(mask_word_offsets_host)
    _check("lsa_union_compact", _union_compact(marr, len(masks), B, _p(key_offsets), kop, _p(mask_word_offsets),
                                               mop, _p(idx_out), _p(count_out), _p(union_mask_out),
                                               _stream(stream)))


def topk_workspace_size(L, B, total_rows, k) -> int:
    return int(_topk_ws(L, B, total_rows, k))


def topk(layers, *, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, key_dtype, k, topk_count_out,
         workspace, stream=None):
    """lsa_topk. `layers`: dicts with q, w, keys, key_scale (fp8), topk_idx_out, topk_score_out (optional)."""
    arr = (TopkLayer * len(layers))(*[TopkLayer(_p(x["q"]), _p(x["w"]), _p(x["keys"]), _p(x.get("key_scale")),
                                                _p(x["topk_idx_out"]), _p(x.get("topk_score_out"))) for x in layers])
    ko, kop = _host64(key_offsets_host)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("lsa_topk", _topk(arr, len(layers), B, _p(key_offsets), kop, _p(idx), _p(count), n_h, d_h,
                             DTYPES.get(key_dtype, key_dtype), k, _p(topk_count_out), _p(workspace), nbytes,
                             _stream(stream)))


def topk_step(layers, *, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, key_dtype, k, topk_count_out,
              workspace, stream=None):
    """lsa_topk_step: as topk, with each layer's `keys` the packed subset keys (one decode step)."""
    arr = (TopkLayer * len(layers))(*[TopkLayer(_p(x["q"]), _p(x["w"]), _p(x["keys"]), _p(x.get("key_scale")),
                                                _p(x["topk_idx_out"]), _p(x.get("topk_score_out"))) for x in layers])
    ko, kop = _host64(key_offsets_host)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("lsa_topk_step", _topk_step(arr, len(layers), B, _p(key_offsets), kop, _p(idx), _p(count), n_h, d_h,
                                       DTYPES.get(key_dtype, key_dtype), k, _p(topk_count_out), _p(workspace),
                                       nbytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def topk_step_noalloc(layers, *, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, key_dtype, k,
                      topk_count_out, stream=None):
    """lsa_topk_step_noalloc: as topk_step, with the library's own fixed scratch instead of a workspace."""
    arr = (TopkLayer * len(layers))(*[TopkLayer(_p(x["q"]), _p(x["w"]), _p(x["keys"]), _p(x.get("key_scale")),
                                                _p(x["topk_idx_out"]), _p(x.get("topk_score_out"))) for x in layers])
    ko, kop = _host64(key_offsets_host)
    _check("lsa_topk_step_noalloc", _topk_step_noalloc(arr, len(layers), B, _p(key_offsets), kop, _p(idx), _p(count),
                                                       n_h, d_h, DTYPES.get(key_dtype, key_dtype), k,
                                                       _p(topk_count_out), _stream(stream)))


def _topk_layers(layers):
    return (TopkLayer * len(layers))(*[TopkLayer(_p(x.get("q")), _p(x.get("w")), _p(x.get("keys")),
                                                 _p(x.get("key_scale")), _p(x.get("topk_idx_out")),
                                                 _p(x.get("topk_score_out"))) for x in layers])


def topk_score(layers, *, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, key_dtype, workspace,
               stream=None):
    """lsa_topk_score: the subset scores into the workspace. `layers`: dicts with q, w, keys, key_scale."""
    ko, kop = _host64(key_offsets_host)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("lsa_topk_score", _topk_score(_topk_layers(layers), len(layers), B, _p(key_offsets), kop, _p(idx),
                                         _p(count), n_h, d_h, DTYPES.get(key_dtype, key_dtype), _p(workspace),
                                         nbytes, _stream(stream)))


def topk_select(layers, *, B, key_offsets, key_offsets_host, idx, count, k, topk_count_out, workspace,
                stream=None):
    """lsa_topk_select: the top-k from the scores in the workspace. `layers`: dicts with topk_idx_out
    and topk_score_out (optional)."""
    ko, kop = _host64(key_offsets_host)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("lsa_topk_select", _topk_select(_topk_layers(layers), len(layers), B, _p(key_offsets), kop, _p(idx),
                                           _p(count), k, _p(topk_count_out), _p(workspace), nbytes,
                                           _stream(stream)))


def gather(pool, *, row_bytes, B, pool_row_offsets, pool_row_offsets_host, idx, idx_offsets, count, out,
           out_row_offsets=None, out_capacity_rows, stream=None):
    """lsa_gather (packed mode when out_row_offsets is None)."""
    po, pop = _host64(pool_row_offsets_host)
    _check("lsa_gather", _gather(_p(pool), int(row_bytes), B, _p(pool_row_offsets), pop, _p(idx), _p(idx_offsets),
                                 _p(count), _p(out), _p(out_row_offsets), int(out_capacity_rows), _stream(stream)))


def fetch_host(pool_host, *, row_bytes, B, pool_row_offsets, pool_row_offsets_host, idx, idx_offsets, count, out,
               out_row_offsets=None, out_capacity_rows, stream=None):
    """lsa_fetch_host: pool_host is a pinned CPU tensor (pin_memory=True); out is on the device."""
    po, pop = _host64(pool_row_offsets_host)
    _check("lsa_fetch_host", _fetch_host(_p(pool_host), int(row_bytes), B, _p(pool_row_offsets), pop, _p(idx),
                                         _p(idx_offsets), _p(count), _p(out), _p(out_row_offsets),
                                         int(out_capacity_rows), _stream(stream)))


def golden_workspace_size(T, L, row_stride) -> int:
    return int(_golden_ws(int(T), int(L), int(row_stride)))


def golden_labels(logits, *, row_stride, T, L, n_valid, top_p, theta, row_mask, golden, workspace,
                  nucleus_size=None, token_golden=None, stream=None):
    """lsa_golden_labels: logits [T, L, row_stride] fp32 and n_valid [T] int32 on the device; the mask
    outputs are int64 tensors of ceil(row_stride / 64) words per row; workspace is a device tensor of at
    least golden_workspace_size(T, L, row_stride) bytes."""
    _check("lsa_golden_labels", _golden(_p(logits), int(row_stride), int(T), int(L), _p(n_valid), float(top_p),
                                        int(theta), _p(row_mask), _p(nucleus_size), _p(token_golden), _p(golden),
                                        _p(workspace), _nbytes(workspace), _stream(stream)))


def train_workspace_size(B, key_offsets_host, r) -> int:
    ko, kop = _host64(key_offsets_host)
    return int(_train_ws(int(B), kop, int(r)))


def train_step(*, h, w_dq, w_iuq, w_w, keys, key_offsets, key_offsets_host, labels, mask_word_offsets,
               mask_word_offsets_host, B, d, r, n_h, d_h, gamma, alpha, loss, g_dq, g_iuq, g_w, workspace,
               stream=None):
    """lsa_train_step: h [B, d], w_dq [r, d], w_iuq [n_h*d_h, r], w_w [n_h, d] and keys [rows, d_h] as bf16
    bits on the device; labels are the selection path's bit masks; loss [1] and the gradients (the
    weights' shapes) are fp32 device tensors; workspace holds train_workspace_size(...) bytes."""
    ko, kop = _host64(key_offsets_host)
    mo, mop = _host64(mask_word_offsets_host)
    _check("lsa_train_step", _train(_p(h), _p(w_dq), _p(w_iuq), _p(w_w), _p(keys), _p(key_offsets), kop, _p(labels),
                                    _p(mask_word_offsets), mop, int(B), int(d), int(r), int(n_h), int(d_h),
                                    float(gamma), float(alpha), _p(loss), _p(g_dq), _p(g_iuq), _p(g_w),
                                    _p(workspace), _nbytes(workspace), _stream(stream)))
