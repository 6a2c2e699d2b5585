"""The C ABI without a GPU: exports, host-only calls, argument validation.

Every compute call made here fails validation before anything is enqueued
(or has batch_n == 0), so no kernel is ever launched from these tests.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from dynamic_sparse_kv_amd import sfi
from oracle import sfi_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # never dereferenced: each call below is rejected first


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "sfi.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sfi_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 10
    L = ctypes.CDLL(sfi.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert sfi.sfi_status_string(sfi.SFI_OK) == "ok"
    for s in range(-6, 0):
        assert sfi.sfi_status_string(s) not in ("", "unknown status")
    assert "gfx950" in sfi.sfi_version()


@pytest.mark.parametrize("seed", range(12))
def test_schedule_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    steps, B = int(rng.integers(1, 60)), int(rng.integers(1, 5))
    ev = rng.random((steps, B)) < rng.uniform(0.0, 0.3)
    budget = int(rng.integers(-1, 20))
    got = sfi.sfi_schedule(ev, budget).astype(bool)
    want = O.schedule(ev, None if budget < 0 else budget)
    np.testing.assert_array_equal(got, want)


def _kv(**over):
    kv = sfi.sfi_kv()
    kv.k = kv.v = kv.seq_len = FAKE
    kv.page_table = None
    kv.page_size = kv.max_pages = kv.num_pages = 0
    kv.B, kv.Hq, kv.Hkv, kv.d, kv.cap, kv.max_seq_len = 2, 8, 2, 128, 1000, 900
    for k, v in over.items():
        setattr(kv, k, v)
    return kv


def _slow(kv, ws_bytes=1 << 40, ld=1000, **kw):
    L = sfi.lib()
    args = dict(batch_ids=None, batch_n=1, q=FAKE, out=FAKE, evidence=None, key_norm=None)
    args.update(kw)
    return L.sfi_slow_step(ctypes.byref(kv), args["batch_ids"], args["batch_n"], args["q"],
                           args["out"], args["evidence"], args["key_norm"], ld, FAKE, ws_bytes, None)


def test_workspace_sizes():
    kv = _kv()
    assert sfi.sfi_slow_workspace_bytes(kv) > 0
    assert sfi.sfi_fast_workspace_bytes(kv, 64, 4, 256) > 0
    assert sfi.sfi_verify_workspace_bytes(kv, 8) > 0
    assert sfi.sfi_select_workspace_bytes(2, 2, 900) >= 2 * 2 * 900 * 4
    assert sfi.sfi_slow_workspace_bytes(_kv(d=96)) == 0
    assert sfi.sfi_select_workspace_bytes(0, 2, 900) == 0
    assert sfi.sfi_verify_workspace_bytes(kv, 0) == 0


def test_slow_step_validation():
    assert sfi.lib().sfi_slow_step(None, None, 1, FAKE, FAKE, None, None, 0, FAKE, 1, None) == sfi.SFI_ERR_NULL
    assert _slow(_kv(k=None)) == sfi.SFI_ERR_NULL
    assert _slow(_kv(Hq=6, Hkv=4)) == sfi.SFI_ERR_SHAPE
    assert _slow(_kv(d=96)) == sfi.SFI_ERR_UNSUPPORTED
    assert _slow(_kv(Hq=6, Hkv=2)) == sfi.SFI_ERR_UNSUPPORTED       # G = 3
    assert _slow(_kv(max_seq_len=1001)) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(max_seq_len=0)) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(), batch_n=3) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(), q=None) == sfi.SFI_ERR_NULL
    assert _slow(_kv(), evidence=FAKE, ld=899) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(), ws_bytes=16) == sfi.SFI_ERR_WORKSPACE
    assert _slow(_kv(), batch_n=0) == sfi.SFI_OK                      # nothing to do
    # paged descriptions
    assert _slow(_kv(page_table=FAKE, page_size=24, max_pages=100, num_pages=200)) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(page_table=FAKE, page_size=16, max_pages=10, num_pages=200)) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(page_table=FAKE, page_size=16, max_pages=100, num_pages=0)) == sfi.SFI_ERR_SHAPE
    # fused-append rows: both or neither, 16-byte aligned
    assert _slow(_kv(k_new=FAKE)) == sfi.SFI_ERR_NULL
    assert _slow(_kv(k_new=FAKE, v_new=FAKE + 4)) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(k_new=FAKE, v_new=FAKE), batch_n=0) == sfi.SFI_OK
    # key-norm statistics: 8-byte aligned
    assert _slow(_kv(norm_stats=FAKE + 4)) == sfi.SFI_ERR_RANGE
    assert _slow(_kv(norm_stats=FAKE, norm_stats_valid=1), batch_n=0) == sfi.SFI_OK


def test_fused_rows_refused_where_unsupported():
    """sfi_append_kv (its rows come as arguments) and the verify and window
    calls reject a cache description that carries fused-append rows."""
    L = sfi.lib()
    kv = _kv(k_new=FAKE, v_new=FAKE)
    assert L.sfi_append_kv(ctypes.byref(kv), None, 1, FAKE, FAKE, 1, None) == sfi.SFI_ERR_RANGE
    assert L.sfi_verify_aggregate(ctypes.byref(kv), None, 1, FAKE, 8, 0xFF, FAKE, FAKE, 1000, FAKE,
                                  1 << 40, None) == sfi.SFI_ERR_RANGE
    assert L.sfi_slow_step_window(ctypes.byref(kv), None, 1, FAKE, 4, FAKE, FAKE, None, 1000, FAKE,
                                  1 << 40, None) == sfi.SFI_ERR_RANGE
    kv2 = sfi.with_new_rows(_kv(), FAKE, FAKE)
    assert (kv2.k_new, kv2.v_new, kv2.B, kv2.max_seq_len) == (FAKE, FAKE, 2, 900)
    kv3 = sfi.with_norm_stats(kv2, FAKE, True)
    assert (kv3.norm_stats, kv3.norm_stats_valid, kv3.k_new, kv3.B) == (FAKE, 1, FAKE, 2)
    assert kv2.norm_stats is None and kv2.norm_stats_valid == 0


def _select(p, B=2, H=2, max_len=900, ld=900, ws_bytes=1 << 40, **kw):
    args = dict(seq_len=FAKE, score=FAKE, key_norm=FAKE, sel_idx=FAKE, sel_count=FAKE, batch_n=1)
    args.update(kw)
    return sfi.lib().sfi_select(ctypes.byref(p), None, args["batch_n"], args["seq_len"], B, H, max_len,
                                args["score"], args["key_norm"], ld, args["sel_idx"], args["sel_count"],
                                None, FAKE, ws_bytes, None)


def test_select_validation():
    P = sfi.select_params
    ok = P(sfi.SFI_SCORE_FUSED, 0.3, 64, 4, 256)
    assert _select(P(sfi.SFI_SCORE_FUSED, 1.5, 64, 4, 256)) == sfi.SFI_ERR_RANGE
    assert _select(P(sfi.SFI_SCORE_FUSED, -0.1, 64, 4, 256)) == sfi.SFI_ERR_RANGE
    assert _select(P(sfi.SFI_SCORE_FUSED, 0.3, 0, 4, 256)) == sfi.SFI_ERR_RANGE
    assert _select(P(sfi.SFI_SCORE_FUSED, 0.3, 64, -1, 256)) == sfi.SFI_ERR_RANGE
    assert _select(P(sfi.SFI_SCORE_FUSED, 0.3, 64, 4, 256, pos_tau=0.0)) == sfi.SFI_ERR_RANGE
    assert _select(P(7, 0.3, 64, 4, 256)) == sfi.SFI_ERR_RANGE
    assert _select(ok, key_norm=None) == sfi.SFI_ERR_NULL
    assert _select(ok, ld=899) == sfi.SFI_ERR_RANGE
    assert _select(ok, ws_bytes=8) == sfi.SFI_ERR_WORKSPACE
    assert _select(ok, batch_n=3) == sfi.SFI_ERR_RANGE
    assert _select(ok, batch_n=0) == sfi.SFI_OK
    raw = P(sfi.SFI_SCORE_RAW, 0.0, 64, 4, 256)
    assert _select(raw, key_norm=None, batch_n=0) == sfi.SFI_OK          # RAW needs no norms
    # score refinements: radius in [0, 8], alpha and beta in [0, 1)
    for kw in (dict(nms_radius=9), dict(nms_radius=-1), dict(nms_radius=2, nms_alpha=1.0),
               dict(nms_radius=2, nms_alpha=-0.1), dict(excl_beta=1.0), dict(excl_beta=-0.5),
               dict(excl_beta=float("nan"))):
        assert _select(P(sfi.SFI_SCORE_FUSED, 0.3, 64, 4, 256, **kw)) == sfi.SFI_ERR_RANGE, kw
    ref = P(sfi.SFI_SCORE_FUSED, 0.3, 64, 4, 256, nms_radius=8, nms_alpha=0.9, excl_beta=0.5)
    assert _select(ref, batch_n=0) == sfi.SFI_OK


def test_fast_step_validation():
    L = sfi.lib()

    def call(kv, sel_heads=2, sel_k=64, ws_bytes=1 << 40, sel_idx=FAKE, n_sink=4, window=256, batch_n=1):
        return L.sfi_fast_step(ctypes.byref(kv), None, batch_n, FAKE, sel_idx, FAKE, sel_heads, sel_k,
                               n_sink, window, FAKE, FAKE, ws_bytes, None)

    assert call(_kv(), sel_heads=3) == sfi.SFI_ERR_SHAPE
    assert call(_kv(), sel_k=-1) == sfi.SFI_ERR_RANGE
    assert call(_kv(), window=-1) == sfi.SFI_ERR_RANGE
    assert call(_kv(), sel_idx=None) == sfi.SFI_ERR_NULL
    assert call(_kv(), ws_bytes=8) == sfi.SFI_ERR_WORKSPACE
    assert call(_kv(d=256)) == sfi.SFI_ERR_UNSUPPORTED
    assert call(_kv(), batch_n=0) == sfi.SFI_OK


def test_fast_step_noalloc_validation():
    """Argument errors of the no-workspace fast step are reported before the
    library's scratch array is touched (no device call is made)."""
    L = sfi.lib()

    def call(kv, sel_heads=2, sel_k=64, sel_idx=FAKE, q=FAKE, n_sink=4, window=256, batch_n=1):
        return L.sfi_fast_step_noalloc(ctypes.byref(kv), None, batch_n, q, sel_idx, FAKE, sel_heads, sel_k,
                                       n_sink, window, FAKE, None)

    assert call(_kv(), sel_heads=3) == sfi.SFI_ERR_SHAPE
    assert call(_kv(), sel_k=-1) == sfi.SFI_ERR_RANGE
    assert call(_kv(), n_sink=-1) == sfi.SFI_ERR_RANGE
    assert call(_kv(), sel_idx=None) == sfi.SFI_ERR_NULL
    assert call(_kv(), q=None) == sfi.SFI_ERR_NULL
    assert call(_kv(), q=FAKE + 4) == sfi.SFI_ERR_RANGE
    assert call(_kv(d=256)) == sfi.SFI_ERR_UNSUPPORTED
    assert call(_kv(), batch_n=-1) == sfi.SFI_ERR_RANGE
    assert call(_kv(), batch_n=0) == sfi.SFI_OK


def test_decode_step_validation():
    L = sfi.lib()

    def call(kv, n_slow=1, n_fast=1, evidence=FAKE, ld=1000, sel_count=FAKE, sel_heads=2,
             sel_k=64, ws_bytes=1 << 40):
        return L.sfi_decode_step(ctypes.byref(kv), FAKE, n_slow, FAKE, n_fast, FAKE, FAKE, evidence,
                                 None, ld, FAKE, sel_count, sel_heads, sel_k, 4, 256, FAKE, ws_bytes,
                                 None)

    kv = _kv()
    B = kv.B
    assert call(kv, n_slow=B, n_fast=1) == sfi.SFI_ERR_RANGE            # more ids than sequences
    assert call(kv, n_slow=-1) == sfi.SFI_ERR_RANGE
    assert call(kv, evidence=None) == sfi.SFI_ERR_NULL                  # slow part needs evidence
    assert call(kv, ld=10) == sfi.SFI_ERR_RANGE
    assert call(kv, sel_count=None) == sfi.SFI_ERR_NULL
    assert call(kv, sel_heads=3) == sfi.SFI_ERR_SHAPE
    assert call(kv, ws_bytes=8) == sfi.SFI_ERR_WORKSPACE
    assert call(_kv(d=256)) == sfi.SFI_ERR_UNSUPPORTED
    assert call(kv, n_slow=0, n_fast=0) == sfi.SFI_OK
    need = sfi.sfi_decode_step_workspace_bytes(kv, 64, 4, 256)
    assert need == sfi.sfi_slow_workspace_bytes(kv) + sfi.sfi_fast_workspace_bytes(kv, 64, 4, 256)
    assert call(kv, n_slow=0, n_fast=0, ws_bytes=need) == sfi.SFI_OK


def test_len_hints_validation():
    """Host row-count hints: each listed entry's hint is checked against its
    range (slow: 0..max_seq_len; fast: 0..n_sink + window + sel_k) before
    anything is enqueued; entries past the list are not read."""
    L = sfi.lib()
    ok_s = np.array([900, 0, -5], dtype=np.int32)      # third entry never listed below
    bad_s = np.array([901], dtype=np.int32)
    neg = np.array([-1], dtype=np.int32)
    fmax = np.array([4 + 256 + 64], dtype=np.int32)
    fbad = np.array([4 + 256 + 65], dtype=np.int32)

    def slow(kv, batch_n=1):
        return L.sfi_slow_step(ctypes.byref(kv), None, batch_n, FAKE, FAKE, None, None, 900, FAKE, 1 << 40, None)

    def fast(kv, batch_n=1):
        return L.sfi_fast_step(ctypes.byref(kv), None, batch_n, FAKE, FAKE, FAKE, 2, 64, 4, 256, FAKE, FAKE,
                               1 << 40, None)

    def step(kv, n_slow=1, n_fast=1):
        return L.sfi_decode_step(ctypes.byref(kv), FAKE, n_slow, FAKE, n_fast, FAKE, FAKE, FAKE, None, 1000,
                                 FAKE, FAKE, 2, 64, 4, 256, FAKE, 1 << 40, None)

    H = sfi.with_len_hints
    assert slow(H(_kv(max_seq_len=900), bad_s)) == sfi.SFI_ERR_RANGE
    assert slow(H(_kv(max_seq_len=900), neg)) == sfi.SFI_ERR_RANGE
    assert slow(H(_kv(max_seq_len=900), ok_s), batch_n=0) == sfi.SFI_OK
    assert fast(H(_kv(), None, fbad)) == sfi.SFI_ERR_RANGE
    assert fast(H(_kv(), None, neg)) == sfi.SFI_ERR_RANGE
    assert fast(H(_kv(), None, fmax), batch_n=0) == sfi.SFI_OK
    assert fast(H(_kv(), bad_s, None), batch_n=0) == sfi.SFI_OK       # a fast step reads no slow hint
    assert step(H(_kv(), None, fbad)) == sfi.SFI_ERR_RANGE
    assert step(H(_kv(max_seq_len=900), bad_s, fmax)) == sfi.SFI_ERR_RANGE
    assert step(H(_kv(max_seq_len=900), ok_s[:2], fmax), n_slow=0, n_fast=0) == sfi.SFI_OK
    kv = H(_kv(), ok_s, fmax)
    assert kv.slow_len_host == ok_s.ctypes.data and kv.fast_len_host == fmax.ctypes.data
    assert kv.B == 2 and _kv().slow_len_host is None
    with pytest.raises(TypeError):
        H(_kv(), np.array([1, 2], dtype=np.int64))
    with pytest.raises(TypeError):
        H(_kv(), None, [5])


def test_layer_step_validation():
    """sfi_decode_layer_step / sfi_run_deferred: argument checks and the
    cases with nothing to launch (no kernel runs here)."""
    L = sfi.lib()
    p = sfi.select_params(sfi.SFI_SCORE_FUSED, 0.3, 64, 4, 256)

    def deferred(**over):
        d = sfi.sfi_deferred()
        d.active = 1
        d.params = sfi.select_params(sfi.SFI_SCORE_FUSED, 0.3, 64, 4, 256)
        d.batch_ids, d.batch_n, d.seq_len = FAKE + 64, 1, FAKE + 128
        d.B, d.H, d.max_seq_len = 2, 2, 900
        d.evidence, d.key_norm, d.ld = FAKE + 192, FAKE + 256, 1000
        d.sel_idx, d.sel_count, d.fused_out = FAKE + 320, FAKE + 384, None
        d.ws, d.ws_bytes = FAKE + 512, 1 << 40
        for k, v in over.items():
            setattr(d, k, v)
        return d

    def call(kv, pending=None, defer=None, n_slow=0, n_fast=0):
        return L.sfi_decode_layer_step(ctypes.byref(kv), ctypes.byref(p), FAKE, n_slow, FAKE, n_fast, FAKE,
                                       FAKE, FAKE, FAKE, 1000, FAKE, FAKE, None, FAKE, 1 << 40,
                                       None if pending is None else ctypes.byref(pending),
                                       None if defer is None else ctypes.byref(defer), None)

    kv = _kv()
    assert L.sfi_run_deferred(None, None) == sfi.SFI_ERR_NULL
    assert L.sfi_run_deferred(ctypes.byref(deferred(active=0)), None) == sfi.SFI_OK
    assert L.sfi_run_deferred(ctypes.byref(deferred(batch_n=0)), None) == sfi.SFI_OK
    out = sfi.sfi_deferred()
    out.active = 7
    assert call(kv, deferred(batch_n=0), out) == sfi.SFI_OK                   # nothing to run
    assert out.active == 0                                                      # no slow sequences
    assert call(kv, deferred(sel_idx=FAKE), out) == sfi.SFI_ERR_RANGE          # aliases this call
    assert call(kv, deferred(evidence=FAKE), out) == sfi.SFI_ERR_RANGE
    raw = deferred()
    raw.params.mode = sfi.SFI_SCORE_RAW
    assert call(kv, raw, out) == sfi.SFI_ERR_RANGE                             # FUSED only
    assert call(kv, deferred(B=0), out) == sfi.SFI_ERR_SHAPE
    assert call(kv, deferred(ld=10), out) == sfi.SFI_ERR_RANGE
    assert call(kv, deferred(ws_bytes=8), out) == sfi.SFI_ERR_WORKSPACE
    assert call(kv, deferred(ws=FAKE + 520), out) == sfi.SFI_ERR_RANGE          # workspaces 256-byte aligned
    assert call(kv, deferred(key_norm=None), out) == sfi.SFI_ERR_NULL
    assert call(kv, None, out, n_slow=kv.B, n_fast=1) == sfi.SFI_ERR_RANGE    # this call's own checks
    assert call(_kv(d=256), None, out) == sfi.SFI_ERR_UNSUPPORTED
    # a deferred selection has one key and one pick pass: no exclusivity
    ex = deferred()
    ex.params.excl_beta = 0.5
    assert call(kv, ex, out) == sfi.SFI_ERR_UNSUPPORTED
    p.excl_beta = 0.5
    assert call(kv, None, out) == sfi.SFI_ERR_UNSUPPORTED
    p.excl_beta = 0.0


def test_verify_validation():
    L = sfi.lib()

    def call(kv, T=8, mask=0xFF, ld=1000, ws_bytes=1 << 40, agg=FAKE, batch_n=1):
        return L.sfi_verify_aggregate(ctypes.byref(kv), None, batch_n, FAKE, T, mask, FAKE, agg, ld,
                                      FAKE, ws_bytes, None)

    kv = _kv(Hq=32, Hkv=8)
    assert call(kv, T=9, mask=0x1FF) == sfi.SFI_ERR_UNSUPPORTED          # 4 * 9 > 32 rows
    assert call(kv, T=0, mask=0) == sfi.SFI_ERR_UNSUPPORTED
    assert call(kv, mask=0) == sfi.SFI_ERR_RANGE
    assert call(kv, mask=0x100) == sfi.SFI_ERR_RANGE
    assert call(kv, ld=10) == sfi.SFI_ERR_RANGE
    assert call(kv, agg=None) == sfi.SFI_ERR_NULL
    assert call(kv, ws_bytes=8) == sfi.SFI_ERR_WORKSPACE
    assert call(_kv(Hq=40, Hkv=8), T=4, mask=0xF) == sfi.SFI_ERR_UNSUPPORTED  # G = 5 has no MFMA tile
    assert call(kv, batch_n=0) == sfi.SFI_OK


def test_compact_validation():
    """sfi_compact_selected / sfi_fast_step_compact: argument checks and the
    cases with nothing to launch (no kernel runs here)."""
    L = sfi.lib()

    def compact(kv, ck=FAKE, cv=FAKE, sel_heads=2, sel_k=64, batch_n=1, sel_count=FAKE):
        return L.sfi_compact_selected(ctypes.byref(kv), None, batch_n, FAKE, sel_count, sel_heads, sel_k,
                                      ck, cv, None)

    def fast(kv, ck=FAKE, cv=FAKE, ws_bytes=1 << 40, batch_n=1, q=FAKE):
        return L.sfi_fast_step_compact(ctypes.byref(kv), None, batch_n, q, FAKE, FAKE, 2, 64, 4, 256,
                                       ck, cv, FAKE, FAKE, ws_bytes, None)

    kv = _kv()
    assert compact(kv, ck=None) == sfi.SFI_ERR_NULL
    assert compact(kv, cv=FAKE + 8) == sfi.SFI_ERR_RANGE                  # copies are 16-byte aligned
    assert compact(kv, sel_heads=3) == sfi.SFI_ERR_SHAPE
    assert compact(kv, sel_count=None) == sfi.SFI_ERR_NULL
    assert compact(kv, batch_n=3) == sfi.SFI_ERR_RANGE
    assert compact(_kv(d=96)) == sfi.SFI_ERR_UNSUPPORTED
    assert compact(kv, batch_n=0) == sfi.SFI_OK
    assert compact(kv, sel_k=0) == sfi.SFI_OK
    assert fast(kv, ck=None) == sfi.SFI_ERR_NULL
    assert fast(kv, ck=FAKE + 4) == sfi.SFI_ERR_RANGE
    assert fast(kv, q=None) == sfi.SFI_ERR_NULL
    assert fast(kv, ws_bytes=8) == sfi.SFI_ERR_WORKSPACE
    assert fast(kv, batch_n=0) == sfi.SFI_OK


def test_paged_length_limit():
    """A paged cache longer than 4,194,304 rows is rejected (its decode chunks
    stage their page ids in LDS)."""
    L = sfi.lib()
    kv = _kv(page_table=FAKE, page_size=16, max_pages=300000, num_pages=10, cap=0, max_seq_len=4194305)
    assert L.sfi_fast_step(ctypes.byref(kv), None, 1, FAKE, FAKE, FAKE, 2, 64, 4, 256, FAKE, FAKE, 1 << 40,
                           None) == sfi.SFI_ERR_UNSUPPORTED
    kv.max_seq_len = 4194304
    assert L.sfi_fast_step(ctypes.byref(kv), None, 0, FAKE, FAKE, FAKE, 2, 64, 4, 256, FAKE, FAKE, 1 << 40,
                           None) == sfi.SFI_OK


def test_slow_window_validation():
    L = sfi.lib()

    def call(kv, w=8, ld=1000, ws_bytes=1 << 40, ev=FAKE, batch_n=1):
        return L.sfi_slow_step_window(ctypes.byref(kv), None, batch_n, FAKE, w, FAKE, ev, None, ld, FAKE,
                                      ws_bytes, None)

    kv = _kv(Hq=32, Hkv=8)
    assert call(kv, w=9) == sfi.SFI_ERR_UNSUPPORTED                 # 4 x 9 rows > one 32-column tile
    assert call(kv, w=0) == sfi.SFI_ERR_UNSUPPORTED
    assert call(_kv(Hq=40, Hkv=8), w=4) == sfi.SFI_ERR_UNSUPPORTED  # G = 5
    assert call(kv, ld=899) == sfi.SFI_ERR_RANGE
    assert call(kv, ev=None) == sfi.SFI_ERR_NULL
    assert call(kv, ws_bytes=8) == sfi.SFI_ERR_WORKSPACE
    assert call(kv, batch_n=0) == sfi.SFI_OK
    assert L.sfi_slow_window_workspace_bytes(ctypes.byref(kv), 8) > 0
    assert L.sfi_slow_window_workspace_bytes(ctypes.byref(kv), 0) == 0


def test_alignment_requirements():
    """K/V, queries and outputs are 16-byte aligned, workspaces 256-byte
    aligned: misaligned pointers are rejected before any launch."""
    L = sfi.lib()

    def fast(kv, q=FAKE, out=FAKE, ws=FAKE):
        return L.sfi_fast_step(ctypes.byref(kv), None, 1, q, FAKE, FAKE, 2, 64, 4, 256, out, ws, 1 << 40, None)

    assert fast(_kv(k=FAKE + 8)) == sfi.SFI_ERR_RANGE
    assert fast(_kv(v=FAKE + 2)) == sfi.SFI_ERR_RANGE
    assert fast(_kv(), q=FAKE + 4) == sfi.SFI_ERR_RANGE
    assert fast(_kv(), out=FAKE + 12) == sfi.SFI_ERR_RANGE
    assert fast(_kv(), ws=FAKE + 128) == sfi.SFI_ERR_RANGE
    assert L.sfi_slow_step(ctypes.byref(_kv()), None, 1, FAKE, FAKE, None, None, 1000, FAKE + 64, 1 << 40,
                           None) == sfi.SFI_ERR_RANGE
