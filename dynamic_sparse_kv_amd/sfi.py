"""ctypes binding of libsfi (include/sfi.h): argument marshalling only.

Every function carries the C entry point's name and argument order; torch
tensors are passed as raw pointers, ``None`` as NULL.  Statuses other than
SFI_OK raise :class:`SfiError`.  Nothing here computes: every step runs in the
HIP kernels of libsfi.so, and the library must have been built
(``python -m dynamic_sparse_kv_amd.build``) -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional
import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsfi.so")

SFI_OK = 0
SFI_ERR_NULL = -1
SFI_ERR_SHAPE = -2
SFI_ERR_RANGE = -3
SFI_ERR_WORKSPACE = -4
SFI_ERR_UNSUPPORTED = -5
SFI_ERR_HIP = -6

SFI_SCORE_FUSED = 0
SFI_SCORE_RAW = 1

_c_int = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class SfiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sfi_status_string(status)} ({status})")


class sfi_kv(ctypes.Structure):
    _fields_ = [
        ("k", _vp), ("v", _vp), ("page_table", _vp),
        ("page_size", _c_int), ("max_pages", _c_int), ("num_pages", _c_int),
        ("seq_len", _vp),
        ("B", _c_int), ("Hq", _c_int), ("Hkv", _c_int), ("d", _c_int),
        ("cap", _c_int), ("max_seq_len", _c_int),
        ("k_new", _vp), ("v_new", _vp),
        ("norm_stats", _vp), ("norm_stats_valid", _c_int),
        ("slow_len_host", _vp), ("fast_len_host", _vp),
    ]


class sfi_select_params(ctypes.Structure):
    _fields_ = [
        ("mode", _c_int), ("lambda_", ctypes.c_float), ("norm_coef", ctypes.c_float),
        ("pos_tau", ctypes.c_float), ("n_sink", _c_int), ("window", _c_int), ("k", _c_int),
        ("k_per_seq", _vp), ("nms_radius", _c_int), ("nms_alpha", ctypes.c_float),
        ("excl_beta", ctypes.c_float),
    ]


class sfi_deferred(ctypes.Structure):
    """A postponed selection (filled by sfi_decode_layer_step, passed on as is)."""
    _fields_ = [
        ("active", _c_int), ("params", sfi_select_params), ("batch_ids", _vp), ("batch_n", _c_int),
        ("seq_len", _vp), ("B", _c_int), ("H", _c_int), ("max_seq_len", _c_int),
        ("evidence", _vp), ("key_norm", _vp), ("ld", _c_int), ("sel_idx", _vp), ("sel_count", _vp),
        ("fused_out", _vp), ("ws", _vp), ("ws_bytes", _sz),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m dynamic_sparse_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.sfi_slow_workspace_bytes.argtypes = [P(sfi_kv)]
        L.sfi_slow_workspace_bytes.restype = _sz
        L.sfi_select_workspace_bytes.argtypes = [_c_int, _c_int, _c_int]
        L.sfi_select_workspace_bytes.restype = _sz
        L.sfi_fast_workspace_bytes.argtypes = [P(sfi_kv), _c_int, _c_int, _c_int]
        L.sfi_fast_workspace_bytes.restype = _sz
        L.sfi_verify_workspace_bytes.argtypes = [P(sfi_kv), _c_int]
        L.sfi_verify_workspace_bytes.restype = _sz
        L.sfi_slow_step.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp, _sz, _vp]
        L.sfi_slow_step.restype = _c_int
        L.sfi_select.argtypes = [P(sfi_select_params), _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                 _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _sz, _vp]
        L.sfi_select.restype = _c_int
        L.sfi_fast_step.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                    _c_int, _vp, _vp, _sz, _vp]
        L.sfi_fast_step.restype = _c_int
        L.sfi_verify_raw_logits.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _c_int, ctypes.c_uint32, _vp, _vp,
                                            _c_int, _vp, _c_int, _vp, _sz, _vp]
        L.sfi_verify_raw_logits.restype = _c_int
        L.sfi_append_kv.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _vp, _c_int, _vp]
        L.sfi_append_kv.restype = _c_int
        L.sfi_fast_step_noalloc.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                            _c_int, _vp, _vp]
        L.sfi_fast_step_noalloc.restype = _c_int
        L.sfi_slow_window_workspace_bytes.argtypes = [P(sfi_kv), _c_int]
        L.sfi_slow_window_workspace_bytes.restype = _sz
        L.sfi_slow_step_window.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _c_int, _vp, _vp, _vp, _c_int, _vp,
                                           _sz, _vp]
        L.sfi_slow_step_window.restype = _c_int
        L.sfi_compact_selected.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp]
        L.sfi_compact_selected.restype = _c_int
        L.sfi_fast_step_compact.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                            _c_int, _vp, _vp, _vp, _vp, _sz, _vp]
        L.sfi_fast_step_compact.restype = _c_int
        L.sfi_decode_step_workspace_bytes.argtypes = [P(sfi_kv), _c_int, _c_int, _c_int]
        L.sfi_decode_step_workspace_bytes.restype = _sz
        L.sfi_decode_step.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int,
                                      _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _sz, _vp]
        L.sfi_decode_step.restype = _c_int
        L.sfi_decode_step_select_workspace_bytes.argtypes = [P(sfi_kv), _c_int, _c_int, _c_int]
        L.sfi_decode_step_select_workspace_bytes.restype = _sz
        L.sfi_decode_step_select.argtypes = [P(sfi_kv), P(sfi_select_params), _vp, _c_int, _vp, _c_int,
                                             _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _sz, _vp]
        L.sfi_decode_step_select.restype = _c_int
        L.sfi_decode_layer_step.argtypes = [P(sfi_kv), P(sfi_select_params), _vp, _c_int, _vp, _c_int,
                                            _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _sz,
                                            P(sfi_deferred), P(sfi_deferred), _vp]
        L.sfi_decode_layer_step.restype = _c_int
        L.sfi_run_deferred.argtypes = [P(sfi_deferred), _vp]
        L.sfi_run_deferred.restype = _c_int
        L.sfi_verify_aggregate.argtypes = [P(sfi_kv), _vp, _c_int, _vp, _c_int, ctypes.c_uint32, _vp,
                                           _vp, _c_int, _vp, _sz, _vp]
        L.sfi_verify_aggregate.restype = _c_int
        L.sfi_schedule.argtypes = [_vp, _c_int, _c_int, _c_int, _vp]
        L.sfi_schedule.restype = _c_int
        L.sfi_status_string.argtypes = [_c_int]
        L.sfi_status_string.restype = ctypes.c_char_p
        L.sfi_version.argtypes = []
        L.sfi_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != SFI_OK:
        raise SfiError(status, where)


def sfi_status_string(status: int) -> str:
    return lib().sfi_status_string(status).decode()


def sfi_version() -> str:
    return lib().sfi_version().decode()


def make_kv(k, v, seq_len, Hq: int, max_seq_len: int, page_table=None, page_size: int = 0) -> sfi_kv:
    """Describe a cache held in torch tensors.

    Contiguous: k, v are [B][Hkv][cap][d] bf16.  Paged: k, v are a pool
    [P][Hkv][page][d] and page_table is int32 [B][max_pages]."""
    kv = sfi_kv()
    kv.k, kv.v = _ptr(k), _ptr(v)
    kv.seq_len = _ptr(seq_len)
    kv.Hq = Hq
    kv.max_seq_len = int(max_seq_len)
    if page_table is None:
        kv.B, kv.Hkv, kv.cap, kv.d = (int(x) for x in k.shape)
        kv.page_table = None
        kv.page_size = 0
        kv.max_pages = 0
        kv.num_pages = 0
    else:
        kv.Hkv, kv.d = int(k.shape[1]), int(k.shape[3])
        kv.B, kv.max_pages = (int(x) for x in page_table.shape)
        kv.page_table = _ptr(page_table)
        kv.page_size = int(page_size or k.shape[2])
        kv.num_pages = int(k.shape[0])
        kv.cap = 0
    return kv


def with_new_rows(kv: sfi_kv, k_new, v_new) -> sfi_kv:
    """A copy of kv whose step calls also append each listed sequence's new
    row (k_new, v_new: [B][Hkv][d] bf16) at cache row seq_len - 1."""
    x = sfi_kv()
    ctypes.pointer(x)[0] = kv
    x.k_new, x.v_new = _ptr(k_new), _ptr(v_new)
    return x


def with_norm_stats(kv: sfi_kv, norm_stats, valid: bool) -> sfi_kv:
    """A copy of kv that keeps the key-norm statistics norm_stats ([B][Hkv][2]
    float64: sum and sum of squares of the cached rows' key norms) current;
    valid = True vouches that they are current for the call's slow sequences,
    so a combined step-and-select call forms the prior from them."""
    x = sfi_kv()
    ctypes.pointer(x)[0] = kv
    x.norm_stats = _ptr(norm_stats)
    x.norm_stats_valid = 1 if valid else 0
    return x


def _host_i32(a) -> Optional[int]:
    if a is None:
        return None
    if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous and a.ndim == 1):
        raise TypeError("row-count hints are 1-D C-contiguous int32 numpy arrays")
    return a.ctypes.data


def with_len_hints(kv: sfi_kv, slow_lens=None, fast_lens=None) -> sfi_kv:
    """A copy of kv carrying host row-count hints for the call's lists, in
    list order: slow_lens the slow entries' seq_len, fast_lens bounds on the
    fast entries' row lists (min(seq_len, n_sink + window) plus the entry's
    selection count).  The launchers then plan each entry's workgroups from
    its own rows.  The copy keeps the arrays referenced."""
    x = sfi_kv()
    ctypes.pointer(x)[0] = kv
    x.slow_len_host = _host_i32(slow_lens)
    x.fast_len_host = _host_i32(fast_lens)
    x._hold = (slow_lens, fast_lens)
    return x


def select_params(mode: int, lam: float, k: int, n_sink: int, window: int,
                  norm_coef: float = 0.5, pos_tau: float = 1024.0,
                  k_per_seq=None, nms_radius: int = 0, nms_alpha: float = 0.0,
                  excl_beta: float = 0.0) -> sfi_select_params:
    p = sfi_select_params()
    p.mode, p.lambda_, p.norm_coef, p.pos_tau = mode, lam, norm_coef, pos_tau
    p.n_sink, p.window, p.k = n_sink, window, k
    p.k_per_seq = _ptr(k_per_seq)
    p.nms_radius, p.nms_alpha, p.excl_beta = nms_radius, nms_alpha, excl_beta
    return p


def sfi_slow_workspace_bytes(kv: sfi_kv) -> int:
    return int(lib().sfi_slow_workspace_bytes(ctypes.byref(kv)))


def sfi_select_workspace_bytes(B: int, H: int, max_seq_len: int) -> int:
    return int(lib().sfi_select_workspace_bytes(B, H, max_seq_len))


def sfi_fast_workspace_bytes(kv: sfi_kv, sel_k: int, n_sink: int, window: int) -> int:
    return int(lib().sfi_fast_workspace_bytes(ctypes.byref(kv), sel_k, n_sink, window))


def sfi_verify_workspace_bytes(kv: sfi_kv, T: int) -> int:
    return int(lib().sfi_verify_workspace_bytes(ctypes.byref(kv), T))


def sfi_slow_step(kv: sfi_kv, batch_ids, batch_n: int, q, out, evidence, key_norm, ld: int,
                  ws, ws_bytes: int, stream=None):
    _check(lib().sfi_slow_step(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(q), _ptr(out),
                               _ptr(evidence), _ptr(key_norm), ld, _ptr(ws), ws_bytes,
                               _stream(stream)), "sfi_slow_step")


def sfi_select(p: sfi_select_params, batch_ids, batch_n: int, seq_len, B: int, H: int,
               max_seq_len: int, score, key_norm, ld: int, sel_idx, sel_count, fused_out,
               ws, ws_bytes: int, stream=None):
    _check(lib().sfi_select(ctypes.byref(p), _ptr(batch_ids), batch_n, _ptr(seq_len), B, H,
                            max_seq_len, _ptr(score), _ptr(key_norm), ld, _ptr(sel_idx),
                            _ptr(sel_count), _ptr(fused_out), _ptr(ws), ws_bytes,
                            _stream(stream)), "sfi_select")


def sfi_fast_step(kv: sfi_kv, batch_ids, batch_n: int, q, sel_idx, sel_count, sel_heads: int,
                  sel_k: int, n_sink: int, window: int, out, ws, ws_bytes: int, stream=None):
    _check(lib().sfi_fast_step(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(q), _ptr(sel_idx),
                               _ptr(sel_count), sel_heads, sel_k, n_sink, window, _ptr(out),
                               _ptr(ws), ws_bytes, _stream(stream)), "sfi_fast_step")


def sfi_verify_raw_logits(kv: sfi_kv, batch_ids, batch_n: int, q, T: int, row_mask: int, out, agg, ld: int,
                          logits, logits_ld: int, ws, ws_bytes: int, stream=None):
    _check(lib().sfi_verify_raw_logits(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(q), T, row_mask,
                                       _ptr(out), _ptr(agg), ld, _ptr(logits), logits_ld, _ptr(ws), ws_bytes,
                                       _stream(stream)), "sfi_verify_raw_logits")


def sfi_append_kv(kv: sfi_kv, batch_ids, batch_n: int, k_new, v_new, T: int, stream=None):
    _check(lib().sfi_append_kv(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(k_new), _ptr(v_new), T,
                               _stream(stream)), "sfi_append_kv")


def sfi_fast_step_noalloc(kv: sfi_kv, batch_ids, batch_n: int, q, sel_idx, sel_count, sel_heads: int,
                          sel_k: int, n_sink: int, window: int, out, stream=None):
    _check(lib().sfi_fast_step_noalloc(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(q), _ptr(sel_idx),
                                       _ptr(sel_count), sel_heads, sel_k, n_sink, window, _ptr(out),
                                       _stream(stream)), "sfi_fast_step_noalloc")


def sfi_slow_window_workspace_bytes(kv: sfi_kv, w: int) -> int:
    return int(lib().sfi_slow_window_workspace_bytes(ctypes.byref(kv), w))


def sfi_slow_step_window(kv: sfi_kv, batch_ids, batch_n: int, q_win, w: int, out, evidence, key_norm,
                         ld: int, ws, ws_bytes: int, stream=None):
    _check(lib().sfi_slow_step_window(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(q_win), w, _ptr(out),
                                      _ptr(evidence), _ptr(key_norm), ld, _ptr(ws), ws_bytes, _stream(stream)),
           "sfi_slow_step_window")


def sfi_compact_selected(kv: sfi_kv, batch_ids, batch_n: int, sel_idx, sel_count, sel_heads: int,
                         sel_k: int, ck, cv, stream=None):
    _check(lib().sfi_compact_selected(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(sel_idx),
                                      _ptr(sel_count), sel_heads, sel_k, _ptr(ck), _ptr(cv), _stream(stream)),
           "sfi_compact_selected")


def sfi_fast_step_compact(kv: sfi_kv, batch_ids, batch_n: int, q, sel_idx, sel_count, sel_heads: int,
                          sel_k: int, n_sink: int, window: int, ck, cv, out, ws, ws_bytes: int, stream=None):
    _check(lib().sfi_fast_step_compact(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(q), _ptr(sel_idx),
                                       _ptr(sel_count), sel_heads, sel_k, n_sink, window, _ptr(ck), _ptr(cv),
                                       _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "sfi_fast_step_compact")


def sfi_decode_step_workspace_bytes(kv: sfi_kv, sel_k: int, n_sink: int, window: int) -> int:
    return int(lib().sfi_decode_step_workspace_bytes(ctypes.byref(kv), sel_k, n_sink, window))


def sfi_decode_step(kv: sfi_kv, slow_ids, n_slow: int, fast_ids, n_fast: int, q, out, evidence,
                    key_norm, ld: int, sel_idx, sel_count, sel_heads: int, sel_k: int, n_sink: int,
                    window: int, ws, ws_bytes: int, stream=None):
    _check(lib().sfi_decode_step(ctypes.byref(kv), _ptr(slow_ids), n_slow, _ptr(fast_ids), n_fast,
                                 _ptr(q), _ptr(out), _ptr(evidence), _ptr(key_norm), ld, _ptr(sel_idx),
                                 _ptr(sel_count), sel_heads, sel_k, n_sink, window, _ptr(ws), ws_bytes,
                                 _stream(stream)), "sfi_decode_step")


def sfi_decode_step_select_workspace_bytes(kv: sfi_kv, sel_k: int, n_sink: int, window: int) -> int:
    return lib().sfi_decode_step_select_workspace_bytes(ctypes.byref(kv), sel_k, n_sink, window)


def sfi_decode_step_select(kv: sfi_kv, p: sfi_select_params, slow_ids, n_slow: int, fast_ids,
                           n_fast: int, q, out, evidence, key_norm, ld: int, sel_idx, sel_count,
                           fused_out, ws, ws_bytes: int, stream=None):
    _check(lib().sfi_decode_step_select(ctypes.byref(kv), ctypes.byref(p), _ptr(slow_ids), n_slow,
                                        _ptr(fast_ids), n_fast, _ptr(q), _ptr(out), _ptr(evidence),
                                        _ptr(key_norm), ld, _ptr(sel_idx), _ptr(sel_count),
                                        _ptr(fused_out), _ptr(ws), ws_bytes, _stream(stream)),
           "sfi_decode_step_select")


def sfi_decode_layer_step(kv: sfi_kv, p: sfi_select_params, slow_ids, n_slow: int, fast_ids,
                          n_fast: int, q, out, evidence, key_norm, ld: int, sel_idx, sel_count,
                          fused_out, ws, ws_bytes: int, pending: Optional[sfi_deferred],
                          defer: Optional[sfi_deferred], stream=None):
    _check(lib().sfi_decode_layer_step(ctypes.byref(kv), ctypes.byref(p), _ptr(slow_ids), n_slow,
                                       _ptr(fast_ids), n_fast, _ptr(q), _ptr(out), _ptr(evidence),
                                       _ptr(key_norm), ld, _ptr(sel_idx), _ptr(sel_count),
                                       _ptr(fused_out), _ptr(ws), ws_bytes,
                                       None if pending is None else ctypes.byref(pending),
                                       None if defer is None else ctypes.byref(defer),
                                       _stream(stream)), "sfi_decode_layer_step")


def sfi_run_deferred(d: Optional[sfi_deferred], stream=None):
    _check(lib().sfi_run_deferred(None if d is None else ctypes.byref(d), _stream(stream)),
           "sfi_run_deferred")


def sfi_verify_aggregate(kv: sfi_kv, batch_ids, batch_n: int, q, T: int, row_mask: int, out, agg,
                         ld: int, ws, ws_bytes: int, stream=None):
    _check(lib().sfi_verify_aggregate(ctypes.byref(kv), _ptr(batch_ids), batch_n, _ptr(q), T,
                                      row_mask, _ptr(out), _ptr(agg), ld, _ptr(ws), ws_bytes,
                                      _stream(stream)), "sfi_verify_aggregate")


def sfi_schedule(events, budget: int):
    """events: host uint8/bool numpy [steps][B] -> slow uint8 numpy [steps][B]."""
    import numpy as np
    ev = np.ascontiguousarray(events, dtype=np.uint8)
    steps, B = ev.shape
    slow = np.zeros_like(ev)
    _check(lib().sfi_schedule(ev.ctypes.data, steps, B, budget, slow.ctypes.data), "sfi_schedule")
    return slow
