"""GPU parity: every libsfi entry point against the CPU oracle.

Inputs come from the seeded generator (drawn on the GPU, copied to the host
for the oracle); expected values come only from oracle/.  Tolerances are in
tests/parity_util.py.  Cases span several tiles/splits and ragged tails, GQA
groups 1/4/5/8, d = 64 and 128, batch subsets, paged caches, the degenerate
selections (empty candidate set, fewer candidates than k, exact ties) and a
sampled check at the full 32K-context, 8-sequence shape.
"""
import math
import sys

import numpy as np
import pytest
import torch

from dynamic_sparse_kv_amd import sfi
from dynamic_sparse_kv_amd import workload as W
from dynamic_sparse_kv_amd.runner import DecodePlan, SFIDecoder, VegasDecoder
from oracle import sfi_oracle as O

from parity_util import (EVID_TOL, NORM_TOL, OUT_TOL, check_selection, nms_ambiguous, row_rel_err,
                         tie_band_keys)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(t):
    return W.bf16_bits(t)


def _rand_kv(B, Hkv, cap, d, seed, hh=0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    K = torch.randn((B, Hkv, cap, d), generator=g, device=DEV)
    if hh:
        idx = torch.randint(0, cap, (hh,), generator=g, device=DEV)
        K[:, :, idx] *= 3.0
    V = torch.randn((B, Hkv, cap, d), generator=g, device=DEV)
    return K.to(torch.bfloat16).contiguous(), V.to(torch.bfloat16).contiguous()


def _rand_q(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16).contiguous()


# ----------------------------------------------------------------- slow step

SLOW_CASES = [
    # B, Hq, Hkv, d, lens
    (1, 8, 2, 64, [4097]),
    (3, 32, 8, 128, [3000, 517, 9000]),
    (2, 8, 8, 128, [1300, 257]),          # G = 1
    (2, 40, 8, 128, [5000, 2049]),        # G = 5
    (1, 16, 2, 64, [700]),                # G = 8
    (2, 8, 2, 128, [1, 33]),              # tiny contexts
]


@pytest.mark.parametrize("case", SLOW_CASES, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-d{c[3]}")
def test_slow_step_matches_oracle(case):
    B, Hq, Hkv, d, lens = case
    _say(f"slow step case {case}")
    cap = max(lens) + 5
    K, V = _rand_kv(B, Hkv, cap, d, seed=B * 1000 + Hq + d, hh=7)
    q = _rand_q((B, Hq, d), seed=11 + Hq)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dec = SFIDecoder(K, V, Hq, max(lens), n_sink=4, window=256, k=64, lam=0.3)
    dec.slow(q, seq, None, B, select=False)
    torch.cuda.synchronize()
    out = dec.out.cpu().numpy()
    ev = dec.evidence.cpu().numpy()
    nrm = dec.key_norm.cpu().numpy()
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for b in range(B):
        n = lens[b]
        o_ref, p = O.dense_step(qb[b], Kb[b], Vb[b], n)
        f_ref = O.evidence(p, Hkv)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL
        assert row_rel_err(ev[b, :, :n], f_ref) <= EVID_TOL
        np.testing.assert_allclose(ev[b, :, :n].sum(axis=1), 1.0, rtol=1e-4)
        np.testing.assert_allclose(nrm[b, :, :n], O.key_norms(Kb[b], n), rtol=NORM_TOL)


def test_slow_batch_subset_and_plain_dense():
    B, Hq, Hkv, d = 4, 32, 8, 128
    lens = [2000, 3000, 1000, 2500]
    K, V = _rand_kv(B, Hkv, 3100, d, seed=5)
    q = _rand_q((B, Hq, d), seed=6)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dec = SFIDecoder(K, V, Hq, 3000, n_sink=4, window=256, k=64, lam=0.3)
    dec.out.fill_(7.0)
    ids = torch.tensor([2, 0], dtype=torch.int32, device=DEV)
    dec.dense(q, seq, ids, 2)
    torch.cuda.synchronize()
    out = dec.out.cpu().numpy()
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for b in (0, 2):
        o_ref, _ = O.dense_step(qb[b], Kb[b], Vb[b], lens[b])
        assert row_rel_err(out[b], o_ref) <= OUT_TOL
    assert np.all(out[1] == 7.0) and np.all(out[3] == 7.0)     # untouched slots


# ------------------------------------------------------------------- select

def _select_gpu(mode, score, key_norm, lens, k, n_sink, window, lam=0.3, H=None, fused=False, **refine):
    B = score.shape[0]
    H = score.shape[1] if H is None else H
    ld = score.shape[2]
    max_len = max(lens)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    p = sfi.select_params(mode, lam, k, n_sink, window, **refine)
    sel = torch.full((B, H, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
    fo = torch.zeros((B, H, ld), dtype=torch.float32, device=DEV) if fused else None
    wsb = sfi.sfi_select_workspace_bytes(B, H, max_len)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    sfi.sfi_select(p, None, B, seq, B, H, max_len, score, key_norm, ld, sel, cnt, fo, ws, wsb)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy(), (fo.cpu().numpy() if fused else None)


def test_select_raw_exact_ties_and_degenerate():
    _say("select raw ties")
    rng = np.random.default_rng(3)
    B, H, ld = 4, 3, 6000
    lens = [6000, 5000, 300, 200]     # 300: |C| = 40 < k; 200: C empty
    sc = rng.integers(-50, 50, size=(B, H, ld)).astype(np.float32)   # many exact ties
    sc[0, 1] = 1.0                                                  # all equal
    sc[1, 2] = rng.standard_normal(ld).astype(np.float32) * 1e-30   # tiny / denormal-ish values
    sc[0, 2, 100:140] = np.inf                                      # infinities rank first / last
    sc[0, 2, 200:240] = -np.inf
    k, ns, win = 257, 4, 256
    sel, cnt, _ = _select_gpu(sfi.SFI_SCORE_RAW, torch.from_numpy(sc).to(DEV), None, lens, k, ns, win)
    for b in range(B):
        lo, hi = O.candidate_range(lens[b], ns, win)
        for h in range(H):
            want = O.topk_indices(sc[b, h].astype(np.float64), lo, hi, k)
            assert cnt[b, h] == len(want)
            np.testing.assert_array_equal(sel[b, h, : len(want)], want)
            assert np.all(sel[b, h, len(want):] == -1)


def test_select_raw_large_k_and_multi_tile():
    rng = np.random.default_rng(4)
    B, H, ld = 2, 1, 70000
    lens = [70000, 65536]
    sc = rng.standard_normal((B, H, ld)).astype(np.float32)
    k = 4096
    sel, cnt, _ = _select_gpu(sfi.SFI_SCORE_RAW, torch.from_numpy(sc).to(DEV), None, lens, k, 4, 256)
    for b in range(B):
        lo, hi = O.candidate_range(lens[b], 4, 256)
        want = O.topk_indices(sc[b, 0].astype(np.float64), lo, hi, k)
        np.testing.assert_array_equal(sel[b, 0, :k], want)


def test_select_per_sequence_k():
    """k_per_seq caps each sequence's list (row stride stays k); values above
    k clamp to k and negative ones to 0."""
    _say("select per-sequence k")
    rng = np.random.default_rng(5)
    B, H, ld, kcap = 5, 2, 9000, 300
    lens = [9000, 8000, 7000, 600, 5000]
    sc = rng.standard_normal((B, H, ld)).astype(np.float32)
    kseq = np.array([300, 50, 0, 1000, -3], dtype=np.int32)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ks = torch.from_numpy(kseq).to(DEV)
    p = sfi.select_params(sfi.SFI_SCORE_RAW, 0.0, kcap, 4, 256, k_per_seq=ks)
    sel = torch.full((B, H, kcap), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
    wsb = sfi.sfi_select_workspace_bytes(B, H, max(lens))
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    sfi.sfi_select(p, None, B, seq, B, H, max(lens), torch.from_numpy(sc).to(DEV), None, ld, sel, cnt,
                   None, ws, wsb)
    torch.cuda.synchronize()
    sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        kb = int(min(max(kseq[b], 0), kcap))
        lo, hi = O.candidate_range(lens[b], 4, 256)
        for h in range(H):
            want = O.topk_indices(sc[b, h].astype(np.float64), lo, hi, kb)
            assert cnt[b, h] == len(want)
            np.testing.assert_array_equal(sel[b, h, : len(want)], want)
            assert np.all(sel[b, h, len(want):] == -1)


def test_select_fused_from_oracle_evidence():
    """Selector alone: oracle f and norms in, oracle s and Top-K out."""
    _say("select fused")
    B, Hq, Hkv, d = 2, 8, 2, 64
    lens = [4100, 3000]
    cap = 4200
    K, V = _rand_kv(B, Hkv, cap, d, seed=21, hh=20)
    q = _rand_q((B, Hq, d), seed=22)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    f = np.zeros((B, Hkv, cap), dtype=np.float32)
    nu = np.zeros((B, Hkv, cap), dtype=np.float32)
    s_ref = []
    for b in range(B):
        n = lens[b]
        _, p = O.dense_step(qb[b], Kb[b], Vb[b], n)
        fb = O.evidence(p, Hkv)
        f[b, :, :n] = fb
        nu[b, :, :n] = O.key_norms(Kb[b], n)
        s_ref.append(O.fuse(fb, O.prior(Kb[b], n), 0.3))
    k = 256
    sel, cnt, fo = _select_gpu(sfi.SFI_SCORE_FUSED, torch.from_numpy(f).to(DEV), torch.from_numpy(nu).to(DEV),
                               lens, k, 4, 256, lam=0.3, fused=True)
    ties = 0
    for b in range(B):
        n = lens[b]
        lo, hi = O.candidate_range(n, 4, 256)
        assert row_rel_err(fo[b, :, :n], s_ref[b]) <= EVID_TOL
        for g in range(Hkv):
            ties += check_selection(sel[b, g], cnt[b, g], s_ref[b][g], lo, hi, k)
    _say(f"  near-tie differences: {ties}")


def test_select_fused_long_row_many_chunks():
    """A 50,001-key row: 25 selector chunks of 2048 keys (the last one
    ragged), the fused scores and the Top-3000 against the oracle."""
    _say("select fused long row")
    B, Hq, Hkv, d = 1, 4, 2, 64
    n = 50001
    K, V = _rand_kv(B, Hkv, n, d, seed=23, hh=40)
    q = _rand_q((B, Hq, d), seed=24)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    _, p = O.dense_step(qb[0], Kb[0], Vb[0], n)
    fb = O.evidence(p, Hkv)
    s_ref = O.fuse(fb, O.prior(Kb[0], n), 0.2)
    f = torch.from_numpy(fb.astype(np.float32)[None]).to(DEV).contiguous()
    nu = torch.from_numpy(O.key_norms(Kb[0], n).astype(np.float32)[None]).to(DEV).contiguous()
    k = 3000
    sel, cnt, fo = _select_gpu(sfi.SFI_SCORE_FUSED, f, nu, [n], k, 4, 256, lam=0.2, fused=True)
    lo, hi = O.candidate_range(n, 4, 256)
    assert row_rel_err(fo[0], s_ref) <= EVID_TOL
    ties = sum(check_selection(sel[0, g], cnt[0, g], s_ref[g], lo, hi, k) for g in range(Hkv))
    _say(f"  near-tie differences: {ties}")


# ------------------------------------------- Soft-NMS and cross-head exclusivity
# The pages name both refinements without a formula; the oracle's reading
# (soft_nms, exclusive_topk) is the one the key kernel implements.  Where a
# refined score hangs on an earlier near-tie (a neighbour comparison, a
# first-round membership) the difference is allowed and counted.

def _oracle_fused_inputs(B, Hq, Hkv, d, lens, seed, lam=0.3):
    cap = max(lens) + 7
    K, V = _rand_kv(B, Hkv, cap, d, seed=seed, hh=20)
    q = _rand_q((B, Hq, d), seed=seed + 1)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    f = np.zeros((B, Hkv, cap), dtype=np.float32)
    nu = np.zeros((B, Hkv, cap), dtype=np.float32)
    s_ref = []
    for b in range(B):
        n = lens[b]
        _, p = O.dense_step(qb[b], Kb[b], Vb[b], n)
        fb = O.evidence(p, Hkv)
        f[b, :, :n] = fb
        nu[b, :, :n] = O.key_norms(Kb[b], n)
        s_ref.append(O.fuse(fb, O.prior(Kb[b], n), lam))
    return torch.from_numpy(f).to(DEV), torch.from_numpy(nu).to(DEV), s_ref


def _check_refined(sel, cnt, s_rows, lo, hi, k, radius, alpha, beta, log_scores=False):
    """Oracle Soft-NMS then exclusivity on one sequence's head rows; returns
    the number of differing keys (near-tie or ambiguous).  log_scores: RAW
    scores, whose penalties are subtracted."""
    H = len(s_rows)
    s_n = [O.soft_nms(s_rows[g], lo, hi, radius, alpha, log_scores=log_scores) for g in range(H)]
    rows, _ = O.exclusive_topk(s_n, lo, hi, k, beta, log_scores=log_scores)
    amb = np.zeros(len(s_rows[0]), dtype=bool)
    for g in range(H):
        amb |= nms_ambiguous(s_rows[g], lo, hi, radius)
        if beta > 0 and H > 1:
            amb |= tie_band_keys(s_n[g], lo, hi, k)
    return sum(check_selection(sel[g], cnt[g], rows[g], lo, hi, k, ambiguous=amb) for g in range(H))


@pytest.mark.parametrize("radius,alpha", [(1, 0.5), (3, 0.3), (8, 0.9)])
def test_select_soft_nms_raw(radius, alpha):
    _say(f"select soft-nms raw radius={radius} alpha={alpha}")
    rng = np.random.default_rng(40 + radius)
    B, H, ld = 3, 2, 9000
    lens = [9000, 5000, 600]                      # 600: 340 candidates for k = 300
    # RAW scores are summed logits, i.e. log scores of either sign: the
    # penalties are subtracted
    sc = (3.0 * rng.standard_normal((B, H, ld))).astype(np.float32)
    sc[2, 1] = rng.integers(-4, 5, size=ld).astype(np.float32)    # exact ties between neighbours
    k = 300
    sel, cnt, _ = _select_gpu(sfi.SFI_SCORE_RAW, torch.from_numpy(sc).to(DEV), None, lens, k, 4, 256,
                              nms_radius=radius, nms_alpha=alpha)
    diff = 0
    for b in range(B):
        lo, hi = O.candidate_range(lens[b], 4, 256)
        for h in range(H):
            ref = O.soft_nms(sc[b, h], lo, hi, radius, alpha, log_scores=True)
            assert np.all(ref[lo:hi] <= sc[b, h, lo:hi])          # no score rises, negative or not
            diff += check_selection(sel[b, h], cnt[b, h], ref, lo, hi, k)
    _say(f"  near-tie differences: {diff}")


def test_select_soft_nms_raw_negative_neighbour_is_not_promoted():
    """Negative RAW scores s = [-1, -2, -1.5, -3] (after 4 sinks), radius 1,
    alpha 0.5, k = 2: key 1 is penalised (two stronger neighbours), so the
    Top-2 stays {0, 2} + 4 -- scaling by 0.5 would have lifted it to -1."""
    _say("select soft-nms raw, negative scores")
    ld = 4 + 4 + 256
    sc = np.full((1, 1, ld), -50.0, dtype=np.float32)
    sc[0, 0, 4:8] = [-1.0, -2.0, -1.5, -3.0]
    sel, cnt, _ = _select_gpu(sfi.SFI_SCORE_RAW, torch.from_numpy(sc).to(DEV), None, [ld], 2, 4, 256,
                              nms_radius=1, nms_alpha=0.5)
    assert int(cnt[0, 0]) == 2
    assert list(sel[0, 0, :2]) == [4, 6]


@pytest.mark.parametrize("beta", [0.5, 0.95])
def test_select_exclusivity_raw(beta):
    _say(f"select exclusivity raw beta={beta}")
    rng = np.random.default_rng(50)
    B, H, ld = 3, 4, 7000
    lens = [7000, 4000, 700]                      # 700: every candidate fits k
    common = rng.standard_normal((B, 1, ld))
    # log scores of either sign whose heads overlap
    sc = (common + 0.6 * rng.standard_normal((B, H, ld))).astype(np.float32)
    k = 500
    sel, cnt, _ = _select_gpu(sfi.SFI_SCORE_RAW, torch.from_numpy(sc).to(DEV), None, lens, k, 4, 256,
                              excl_beta=beta)
    diff = 0
    for b in range(B):
        lo, hi = O.candidate_range(lens[b], 4, 256)
        rows, lists = O.exclusive_topk([sc[b, h] for h in range(H)], lo, hi, k, beta, log_scores=True)
        first = [O.topk_indices(sc[b, h].astype(np.float64), lo, hi, k) for h in range(H)]
        if b == 0:   # the penalty changes the lists (the test exercises the second round)
            assert any(len(np.setxor1d(lists[h], first[h])) > 0 for h in range(H))
        for h in range(H):
            diff += check_selection(sel[b, h], cnt[b, h], rows[h], lo, hi, k)
    _say(f"  near-tie differences: {diff}")


def test_select_exclusivity_reuses_workspace():
    """Two exclusivity calls in a row on one workspace, the second on
    shorter rows with a per-sequence k: the first key pass of each call
    clears the counts and histograms the previous call left."""
    _say("select exclusivity, workspace reuse")
    rng = np.random.default_rng(52)
    B, H, ld, k = 3, 4, 9000, 400
    wsb = sfi.sfi_select_workspace_bytes(B, H, ld)
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device=DEV)     # not zeroed
    diff = 0
    for lens, kseq in (([9000, 8000, 6000], None), ([5000, 2000, 4100], [400, 150, 0])):
        common = rng.standard_normal((B, 1, ld))
        sc = (common + 0.7 * rng.standard_normal((B, H, ld))).astype(np.float32)
        seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
        ks = None if kseq is None else torch.tensor(kseq, dtype=torch.int32, device=DEV)
        p = sfi.select_params(sfi.SFI_SCORE_RAW, 0.0, k, 4, 256, k_per_seq=ks, nms_radius=2, nms_alpha=0.5,
                              excl_beta=0.7)
        sel = torch.full((B, H, k), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((B, H), -7, dtype=torch.int32, device=DEV)
        sfi.sfi_select(p, None, B, seq, B, H, ld, torch.from_numpy(sc).to(DEV), None, ld, sel, cnt, None,
                       ws, wsb)
        torch.cuda.synchronize()
        sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
        for b in range(B):
            kb = k if kseq is None else min(max(kseq[b], 0), k)
            lo, hi = O.candidate_range(lens[b], 4, 256)
            diff += _check_refined(sel[b], cnt[b], [sc[b, h] for h in range(H)], lo, hi, kb, 2, 0.5, 0.7,
                                   log_scores=True)
            assert np.all(sel[b, :, kb:] == -1)
    _say(f"  differing keys: {diff}")


def test_select_refinements_fused_from_oracle_evidence():
    """FUSED scores with Soft-NMS, exclusivity and both; fused_out keeps the
    score before the refinements."""
    _say("select fused + refinements")
    B, Hq, Hkv, d = 2, 16, 4, 64
    lens = [4100, 3000]
    f, nu, s_ref = _oracle_fused_inputs(B, Hq, Hkv, d, lens, seed=31)
    k = 256
    for radius, alpha, beta in ((4, 0.5, 0.0), (0, 0.0, 0.6), (2, 0.3, 0.5)):
        sel, cnt, fo = _select_gpu(sfi.SFI_SCORE_FUSED, f, nu, lens, k, 4, 256, lam=0.3, fused=True,
                                   nms_radius=radius, nms_alpha=alpha, excl_beta=beta)
        diff = 0
        for b in range(B):
            n = lens[b]
            lo, hi = O.candidate_range(n, 4, 256)
            assert row_rel_err(fo[b, :, :n], s_ref[b]) <= EVID_TOL
            diff += _check_refined(sel[b], cnt[b], list(s_ref[b]), lo, hi, k, radius, alpha, beta)
        _say(f"  radius={radius} alpha={alpha} beta={beta}: differing keys {diff}")


@pytest.mark.parametrize("paged", [False, True])
def test_step_select_with_refinements(paged):
    """The combined step + selection call with Soft-NMS and exclusivity
    against the oracle's slow step, fused score and refinements."""
    _say(f"step_select + refinements, paged={paged}")
    B, Hq, Hkv, d = 3, 32, 8, 128
    lens = [5000, 3500, 6100]
    cap = 6200
    K, V = _rand_kv(B, Hkv, cap, d, seed=71, hh=30)
    q = _rand_q((B, Hq, d), seed=72)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kw = dict(n_sink=4, window=256, k=200, lam=0.3, nms_radius=3, nms_alpha=0.4, excl_beta=0.5)
    if paged:
        cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=B, Hq=Hq, Hkv=Hkv, d=d)
        table, npages = W.page_table(cfg, np.full(B, cap))
        Kp, Vp = W.to_paged(K, table, npages, 16), W.to_paged(V, table, npages, 16)
        tab = torch.from_numpy(table).to(DEV)
        dec = SFIDecoder(Kp, Vp, Hq, cap, page_table=tab, page_size=16, **kw)
    else:
        dec = SFIDecoder(K, V, Hq, cap, **kw)
    ids = torch.tensor([2, 0], dtype=torch.int32, device=DEV)
    dec.step_select(q, seq, ids, 2, None, 0)
    torch.cuda.synchronize()
    sel, cnt = dec.sel_idx.cpu().numpy(), dec.sel_count.cpu().numpy()
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    diff = 0
    for b in (0, 2):
        r = O.slow_select(qb[b], Kb[b], Vb[b], lens[b], lam=0.3, k=200, n_sink=4, window=256)
        diff += _check_refined(sel[b], cnt[b], list(r["s"]), r["lo"], r["hi"], 200, 3, 0.4, 0.5)
    assert np.all(cnt[1] == 0) and np.all(sel[1] == -1)     # sequence 1 not selected
    _say(f"  differing keys: {diff}")


# ----------------------------------------------------------------- fast step

def _fast_gpu(K, V, Hq, q, lens, sel_np, cnt_np, n_sink, window, sel_heads):
    B = K.shape[0]
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kv = sfi.make_kv(K, V, seq, Hq, max(lens))
    sel = torch.from_numpy(np.ascontiguousarray(sel_np, dtype=np.int32)).to(DEV)
    cnt = torch.from_numpy(np.ascontiguousarray(cnt_np, dtype=np.int32)).to(DEV)
    sel_k = sel.shape[2]
    out = torch.full((B, Hq, K.shape[3]), 9.0, device=DEV)
    wsb = sfi.sfi_fast_workspace_bytes(kv, sel_k, n_sink, window)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    sfi.sfi_fast_step(kv, None, B, q, sel, cnt, sel_heads, sel_k, n_sink, window, out, ws, wsb)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 2, 64), (32, 8, 128), (40, 8, 128)])
def test_fast_step_matches_oracle(Hq, Hkv, d):
    _say(f"fast step Hq={Hq} Hkv={Hkv} d={d}")
    B = 3
    lens = [5000, 2000, 700]
    K, V = _rand_kv(B, Hkv, 5100, d, seed=Hq + d)
    q = _rand_q((B, Hq, d), seed=Hq * 3)
    rng = np.random.default_rng(Hq)
    k = 300
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            # a slow-step selection from an earlier, shorter cache: some entries
            # now fall inside the window and must be skipped; sinks too
            pool = np.arange(0, lens[b])
            c = min(k - 3, len(pool))
            pick = np.sort(rng.choice(pool, c, replace=False))
            sel[b, g, :c] = pick
            cnt[b, g] = c
    out = _fast_gpu(K, V, Hq, q, lens, sel, cnt, 4, 256, Hkv)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for b in range(B):
        lists = [sel[b, g, : cnt[b, g]] for g in range(Hkv)]
        o_ref = O.fast_step(qb[b], Kb[b], Vb[b], lens[b], lists, 4, 256)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL


def test_fast_full_selection_equals_dense_and_shared_list():
    B, Hq, Hkv, d = 2, 32, 8, 128
    lens = [3000, 1500]
    K, V = _rand_kv(B, Hkv, 3000, d, seed=77)
    q = _rand_q((B, Hq, d), seed=78)
    ns, win = 4, 256
    k = 3000
    sel = np.full((B, 1, k), -1, dtype=np.int32)
    cnt = np.zeros((B, 1), dtype=np.int32)
    for b in range(B):
        c = np.arange(ns, lens[b] - win)
        sel[b, 0, : len(c)] = c
        cnt[b, 0] = len(c)
    out = _fast_gpu(K, V, Hq, q, lens, sel, cnt, ns, win, 1)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for b in range(B):
        o_ref, _ = O.dense_step(qb[b], Kb[b], Vb[b], lens[b])
        assert row_rel_err(out[b], o_ref) <= OUT_TOL


def test_fast_without_selection_list():
    """sel_k = 0 with no index buffer (the boundary allows it): the fast set
    is sinks + window only, including a sequence shorter than both."""
    _say("fast step, sel_k = 0")
    B, Hq, Hkv, d = 3, 32, 8, 128
    lens = [3000, 700, 150]
    K, V = _rand_kv(B, Hkv, 3000, d, seed=79)
    q = _rand_q((B, Hq, d), seed=80)
    ns, win = 4, 256
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kv = sfi.make_kv(K, V, seq, Hq, max(lens))
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device=DEV)
    out = torch.full((B, Hq, d), 9.0, device=DEV)
    wsb = sfi.sfi_fast_workspace_bytes(kv, 0, ns, win)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    sfi.sfi_fast_step(kv, None, B, q, None, cnt, Hkv, 0, ns, win, out, ws, wsb)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for b in range(B):
        o_ref = O.fast_step(qb[b], Kb[b], Vb[b], lens[b], [[]] * Hkv, ns, win)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL


# ------------------------------------------------------------ whole decode run

def test_decode_run_tiny_config_every_step():
    """Config: tiny 4K single layer, all 64 steps, slow/fast schedule."""
    cfg = W.CONFIGS["tiny-4k"]
    _say("decode run c1")
    K, V = W.make_kv(cfg, device=DEV)
    starts = W.sentence_starts(cfg)
    slow = sfi.sfi_schedule(starts, cfg.budget).astype(bool)
    np.testing.assert_array_equal(slow, O.schedule(starts, cfg.budget))
    qh = W.make_queries(cfg, starts)
    q = qh.to(DEV)
    ctx = W.context_lengths(cfg)
    plan = DecodePlan(slow, ctx, DEV)
    dec = SFIDecoder(K, V, cfg.Hq, int(ctx.max()) + cfg.steps, n_sink=cfg.n_sink, window=cfg.window,
                     k=cfg.k, lam=cfg.lam, keep_fused=True)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(qh)
    ref = O.decode_run(qb[:, 0], Kb[0], Vb[0], int(ctx[0]), slow[:, 0], lam=cfg.lam, k=cfg.k,
                       n_sink=cfg.n_sink, window=cfg.window)
    ties = 0
    for s in range(cfg.steps):
        dec.step(plan, s, q)
        torch.cuda.synchronize()
        r = ref[s]
        assert row_rel_err(dec.out[0].cpu().numpy(), r["o"]) <= OUT_TOL, s
        if r["kind"] == "slow":
            sel = dec.sel_idx[0].cpu().numpy()
            cnt = dec.sel_count[0].cpu().numpy()
            for g in range(cfg.Hkv):
                ties += check_selection(sel[g], cnt[g], r["s"][g], r["lo"], r["hi"], cfg.k)
            assert row_rel_err(dec.fused[0, :, : r["n"]].cpu().numpy(), r["s"]) <= EVID_TOL
    _say(f"  near-tie differences over the run: {ties}")
    assert ties == 0   # fast outputs above were compared against the oracle's own selection


def test_bitwise_repeatable():
    cfg = W.CONFIGS["tiny-4k"].replace(B=2, steps=24)
    K, V = W.make_kv(cfg, device=DEV)
    starts = W.sentence_starts(cfg)
    slow = O.schedule(starts, cfg.budget)
    q = W.make_queries(cfg, starts).to(DEV)
    plan = DecodePlan(slow, W.context_lengths(cfg), DEV)
    outs = []
    for rep in range(2):
        dec = SFIDecoder(K, V, cfg.Hq, cfg.ctx + cfg.steps, n_sink=4, window=256, k=cfg.k, lam=cfg.lam)
        hist = []
        for s in range(cfg.steps):
            dec.step(plan, s, q)
            hist.append(dec.out.clone())
        torch.cuda.synchronize()
        outs.append((torch.stack(hist), dec.sel_idx.clone(), dec.evidence.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)


def test_stream_pipelines_match_single_stream():
    """Two- and three-stream schedules, run eagerly, give the same bits per
    step as the same calls on one stream (slow step, selector, fast step).
    Their graph capture is refused (checked on the CPU)."""
    _say("multi-stream schedules, eager")
    cfg = W.CONFIGS["tiny-4k"].replace(B=3, steps=40, k=128)
    K, V = W.make_kv(cfg, device=DEV)
    starts = W.sentence_starts(cfg)
    slow = O.schedule(starts, cfg.budget)
    q = W.make_queries(cfg, starts).to(DEV)
    plan = DecodePlan(slow, W.context_lengths(cfg), DEV)
    res = []
    for mode in ("one", "two", "three"):
        _say(f"  mode {mode}")
        dec = SFIDecoder(K, V, cfg.Hq, cfg.ctx + cfg.steps, n_sink=4, window=256, k=cfg.k, lam=cfg.lam)
        outs = torch.zeros((cfg.steps, cfg.B, cfg.Hq, cfg.d), device=DEV)
        sa = torch.cuda.current_stream()
        if mode == "one":
            for s in range(cfg.steps):
                dec.step(plan, s, q, sa, out=outs[s], co=False)
        elif mode == "two":
            dec.run_two_streams(plan, q, 0, cfg.steps, sa, torch.cuda.Stream(), out_steps=outs)
        else:
            dec.run_pipelined(plan, q, 0, cfg.steps, sa, torch.cuda.Stream(), torch.cuda.Stream(), outs)
        torch.cuda.synchronize()
        res.append((outs.clone(), dec.sel_idx.clone(), dec.sel_count.clone()))
    for r in res[1:]:
        assert torch.equal(res[0][0].view(torch.int32), r[0].view(torch.int32))
        assert torch.equal(res[0][1], r[1]) and torch.equal(res[0][2], r[2])
    # the slow steps agree with the oracle's decode run of sequence 0 (the
    # fast steps' selections are the one-stream calls', checked elsewhere)
    Kb, Vb = _bits(K[0]), _bits(V[0])
    ref = O.decode_run(_bits(q[:, 0]), Kb, Vb, cfg.ctx, slow[:, 0], lam=cfg.lam, k=cfg.k, n_sink=4, window=256)
    got = res[1][0][:, 0].cpu().numpy()
    for s, r in enumerate(ref):
        if s == 0 or r["kind"] == "slow":
            assert row_rel_err(got[s], r["o"]) <= OUT_TOL, s


# ------------------------------------------------------------ cache append

@pytest.mark.parametrize("paged,T", [(False, 1), (True, 1), (False, 8), (True, 8)])
def test_append_kv_writes_the_new_rows(paged, T):
    """sfi_append_kv writes row t of each listed sequence at cache row
    seq_len - T + t (rows below 0 skipped) of every kv head, bit for bit,
    and leaves everything else untouched."""
    _say(f"append paged={paged} T={T}")
    B, Hq, Hkv, d, ps = 4, 8, 2, 128, 16
    lens = [37, 5, 300, 129]          # sequence 1 has fewer than T = 8 rows
    cap = 320
    g = torch.Generator(device=DEV).manual_seed(90 + T)
    Kc = torch.randn((B, Hkv, cap, d), generator=g, device=DEV).to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, cap, d), generator=g, device=DEV).to(torch.bfloat16)
    kn = torch.randn((B, T, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, T, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ids = torch.tensor([3, 1, 0], dtype=torch.int32, device=DEV)      # sequence 2 not listed
    want_k, want_v = Kc.clone(), Vc.clone()
    for b in (3, 1, 0):
        for t in range(T):
            j = lens[b] - T + t
            if j >= 0:
                want_k[b, :, j] = kn[b, t]
                want_v[b, :, j] = vn[b, t]
    if not paged:
        K, V = Kc.clone(), Vc.clone()
        kv = sfi.make_kv(K, V, seq, Hq, cap)
    else:
        npg = cap // ps
        table = np.random.default_rng(5).permutation(B * npg).astype(np.int32).reshape(B, npg)
        K = W.to_paged(Kc, table, B * npg, ps)
        V = W.to_paged(Vc, table, B * npg, ps)
        tab = torch.from_numpy(table).to(DEV)
        kv = sfi.make_kv(K, V, seq, Hq, cap, tab, ps)
    sfi.sfi_append_kv(kv, ids, 3, kn, vn, T)
    torch.cuda.synchronize()
    if paged:
        got_k = torch.stack([W.gather_paged(K, table, b, cap) for b in range(B)])
        got_v = torch.stack([W.gather_paged(V, table, b, cap) for b in range(B)])
    else:
        got_k, got_v = K, V
    assert torch.equal(got_k.view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(got_v.view(torch.int16), want_v.view(torch.int16))


def test_decode_run_with_append_equals_predrawn_cache():
    """A decode run whose steps append their own K/V row (the cache holds
    only the prefill at the start) gives the same bits, outputs and
    selections, as the run over the cache drawn up front."""
    _say("decode run with per-step append")
    cfg = W.CONFIGS["tiny-4k"].replace(B=3, steps=30, k=128)
    starts = W.sentence_starts(cfg)
    slow = O.schedule(starts, cfg.budget)
    q = W.make_queries(cfg, starts).to(DEV)
    ctx = W.context_lengths(cfg)
    plan = DecodePlan(slow, ctx, DEV)
    res = []
    for with_append in (False, True):
        K, V = W.make_kv(cfg, device=DEV)
        new_kv = W.take_decode_rows(K, V, ctx, cfg.steps) if with_append else None
        if with_append:
            assert torch.all(K[:, :, int(ctx[0]):] == 0)
        dec = SFIDecoder(K, V, cfg.Hq, cfg.ctx + cfg.steps, n_sink=4, window=256, k=cfg.k, lam=cfg.lam)
        outs = torch.zeros((cfg.steps, cfg.B, cfg.Hq, cfg.d), device=DEV)
        for s in range(cfg.steps):
            dec.step(plan, s, q, out=outs[s], new_kv=new_kv)
        torch.cuda.synchronize()
        res.append((outs.clone(), dec.sel_idx.clone(), K.clone(), V.clone()))
    assert torch.equal(res[0][0].view(torch.int32), res[1][0].view(torch.int32))
    assert torch.equal(res[0][1], res[1][1])
    n_end = int(ctx[0]) + cfg.steps
    assert torch.equal(res[0][2][:, :, :n_end].view(torch.int16), res[1][2][:, :, :n_end].view(torch.int16))
    assert torch.equal(res[0][3][:, :, :n_end].view(torch.int16), res[1][3][:, :, :n_end].view(torch.int16))


@pytest.mark.parametrize("mode,paged", [("select", False), ("select", True), ("co", False),
                                        ("split", True), ("two", False), ("layer", False),
                                        ("compact", False)])
def test_fused_append_equals_predrawn_cache(mode, paged):
    """Step calls given the step's new rows in the cache description (fused
    append) give the same bits -- outputs, selections and cache contents --
    as the same calls over the cache drawn up front, in every call path."""
    _say(f"fused append, mode={mode} paged={paged}")
    cfg = W.CONFIGS["tiny-4k"].replace(B=3, steps=28, k=128)
    starts = W.sentence_starts(cfg)
    slow = O.schedule(starts, cfg.budget)
    slow[1] = [True, False, True]     # a step with slow and fast sequences
    q = W.make_queries(cfg, starts).to(DEV)
    ctx = W.context_lengths(cfg)
    plan = DecodePlan(slow, ctx, DEV)
    cap = cfg.ctx + cfg.steps
    ps = 16
    table = None
    if paged:
        npg = (cap + ps - 1) // ps
        table = np.random.default_rng(7).permutation(cfg.B * npg).astype(np.int32).reshape(cfg.B, npg)
    res = []
    for fused in (False, True):
        Kc, Vc = W.make_kv(cfg, device=DEV, cap=cap)
        if paged:
            K = W.to_paged(Kc, table, table.size, ps)
            V = W.to_paged(Vc, table, table.size, ps)
            kw = dict(page_table=torch.from_numpy(table).to(DEV), page_size=ps)
        else:
            K, V, kw = Kc, Vc, {}
        new_kv = W.take_decode_rows(K, V, ctx, cfg.steps, table=table) if fused else None
        dec = SFIDecoder(K, V, cfg.Hq, cap, n_sink=4, window=256, k=cfg.k, lam=cfg.lam, **kw)
        outs = torch.zeros((cfg.steps, cfg.B, cfg.Hq, cfg.d), device=DEV)
        sa = torch.cuda.current_stream()
        if mode == "two":
            dec.run_two_streams(plan, q, 0, cfg.steps, sa, torch.cuda.Stream(), out_steps=outs, new_kv=new_kv)
        for s in range(cfg.steps if mode != "two" else 0):
            nr = None if new_kv is None else (new_kv[0][s], new_kv[1][s])
            if mode == "select":
                dec.step(plan, s, q, out=outs[s], new_kv=new_kv)
            elif mode == "co":
                dec.step(plan, s, q, out=outs[s], new_kv=new_kv, fused_select=False)
            elif mode == "split":
                dec.step(plan, s, q, out=outs[s], new_kv=new_kv, co=False)
            elif mode == "layer":
                own = dec.layer_step(plan, s, q, out=outs[s], new_kv=new_kv)
                sfi.sfi_run_deferred(own)
            else:  # compact: slow steps refresh the compact copy, fast steps read it
                sl, ns, nf = plan.seq_len[s], int(plan.n_slow[s]), int(plan.n_fast[s])
                if ns:
                    dec.slow(q[s], sl, plan.slow_list(s), ns, out=outs[s], new_rows=nr)
                    dec.compact(sl, plan.slow_list(s), ns)
                if nf:
                    dec.fast_compact(q[s], sl, plan.fast_list(s), nf, out=outs[s], new_rows=nr)
        torch.cuda.synchronize()
        if paged:
            n = cap
            Kg = torch.stack([W.gather_paged(K, table, b, n) for b in range(cfg.B)])
            Vg = torch.stack([W.gather_paged(V, table, b, n) for b in range(cfg.B)])
        else:
            Kg, Vg = K, V
        res.append((outs.clone(), dec.sel_idx.clone(), dec.sel_count.clone(), Kg.clone(), Vg.clone()))
    a, b = res
    assert torch.equal(a[0].view(torch.int32), b[0].view(torch.int32))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    n_end = int(ctx[0]) + cfg.steps
    for x, y in ((a[3], b[3]), (a[4], b[4])):
        assert torch.equal(x[:, :, :n_end].view(torch.int16), y[:, :, :n_end].view(torch.int16))


def test_fused_append_short_lists_and_rejections():
    """Fused append where the row sits in the sinks (seq_len <= n_sink) or in
    no list position (window 0: the first split stores it), and the calls
    that take no fused rows refuse them."""
    _say("fused append edge cases")
    B, Hq, Hkv, d, cap = 3, 8, 2, 64, 600
    g = torch.Generator(device=DEV).manual_seed(11)
    Kc = torch.randn((B, Hkv, cap, d), generator=g, device=DEV).to(torch.bfloat16)
    Vc = torch.randn((B, Hkv, cap, d), generator=g, device=DEV).to(torch.bfloat16)
    kn = torch.randn((B, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    seq = torch.tensor([3, 1, 500], dtype=torch.int32, device=DEV)
    sel = torch.full((B, Hkv, 16), -1, dtype=torch.int32, device=DEV)
    sel[2, :, :3] = torch.tensor([10, 200, 498], dtype=torch.int32, device=DEV)
    cnt = torch.tensor([[0, 0], [0, 0], [3, 3]], dtype=torch.int32, device=DEV)
    outs = []
    for fused in (False, True):
        K, V = Kc.clone(), Vc.clone()
        kv = sfi.make_kv(K, V, seq, Hq, cap)
        if fused:
            kvx = sfi.with_new_rows(kv, kn, vn)
        else:
            for b in range(B):
                n = int(seq[b])
                K[b, :, n - 1], V[b, :, n - 1] = kn[b], vn[b]
            kvx = kv
        out = torch.zeros((B, Hq, d), device=DEV)
        ws = torch.zeros(sfi.sfi_fast_workspace_bytes(kv, 16, 4, 0), dtype=torch.uint8, device=DEV)
        sfi.sfi_fast_step(kvx, None, B, q, sel, cnt, Hkv, 16, 4, 0, out, ws, ws.numel())
        torch.cuda.synchronize()
        outs.append((out.clone(), K.clone(), V.clone()))
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
    kv = sfi.with_new_rows(sfi.make_kv(Kc, Vc, seq, Hq, cap), kn, vn)
    with pytest.raises(sfi.SfiError):
        sfi.sfi_append_kv(kv, None, B, kn, vn, 1)


# ------------------------------------------------- co-launched decode step

@pytest.mark.parametrize("Hq,Hkv,d,paged", [(8, 2, 64, False), (40, 8, 128, True)])
def test_decode_step_co_launch_matches_oracle(Hq, Hkv, d, paged):
    """sfi_decode_step: slow steps (with evidence) of some sequences and fast
    steps of the others in one pass, against the oracle."""
    _say(f"co-launched step Hq={Hq} Hkv={Hkv} d={d} paged={paged}")
    B = 5
    lens = [4100, 2500, 5000, 700, 3300]
    cap = 5100
    K, V = _rand_kv(B, Hkv, cap, d, seed=300 + Hq, hh=9)
    q = _rand_q((B, Hq, d), seed=301 + Hq)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    k = 200
    rng = np.random.default_rng(Hq + d)
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            c = min(k - 5, lens[b])
            sel[b, g, :c] = np.sort(rng.choice(lens[b], c, replace=False))
            cnt[b, g] = c
    if paged:
        cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=B, Hq=Hq, Hkv=Hkv, d=d)
        table, npages = W.page_table(cfg, np.full(B, cap))
        Kd, Vd = W.to_paged(K, table, npages, 16), W.to_paged(V, table, npages, 16)
        tab = torch.from_numpy(table).to(DEV)
        dec = SFIDecoder(Kd, Vd, Hq, max(lens), n_sink=4, window=256, k=k, lam=0.3,
                         page_table=tab, page_size=16)
    else:
        dec = SFIDecoder(K, V, Hq, max(lens), n_sink=4, window=256, k=k, lam=0.3)
    dec.sel_idx.copy_(torch.from_numpy(sel))
    dec.sel_count.copy_(torch.from_numpy(cnt))
    dec.out.fill_(5.0)
    slow_b, fast_b = [3, 0], [4, 1, 2]
    sids = torch.tensor(slow_b, dtype=torch.int32, device=DEV)
    fids = torch.tensor(fast_b, dtype=torch.int32, device=DEV)
    dec.co_step(q, seq, sids, len(slow_b), fids, len(fast_b), select=False)
    torch.cuda.synchronize()
    out = dec.out.cpu().numpy()
    ev = dec.evidence.cpu().numpy()
    nrm = dec.key_norm.cpu().numpy()
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for b in slow_b:
        n = lens[b]
        o_ref, p = O.dense_step(qb[b], Kb[b], Vb[b], n)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL
        assert row_rel_err(ev[b, :, :n], O.evidence(p, Hkv)) <= EVID_TOL
        np.testing.assert_allclose(nrm[b, :, :n], O.key_norms(Kb[b], n), rtol=NORM_TOL)
    for b in fast_b:
        lists = [sel[b, g, : cnt[b, g]] for g in range(Hkv)]
        o_ref = O.fast_step(qb[b], Kb[b], Vb[b], lens[b], lists, 4, 256)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL


def test_decode_run_mixed_batch_co_launch():
    """Three sequences with their own schedules, 40 steps: every step that
    mixes slow and fast sequences is co-launched; each sequence's outputs and
    selections follow the oracle's decode run, and the separate-call path
    agrees within tolerance."""
    cfg = W.CONFIGS["tiny-4k"].replace(B=3, steps=40)
    _say("mixed-batch decode run")
    K, V = W.make_kv(cfg, device=DEV)
    starts = W.sentence_starts(cfg)
    slow = sfi.sfi_schedule(starts, cfg.budget).astype(bool)
    assert any(slow[s].any() and (~slow[s]).any() for s in range(cfg.steps))
    qh = W.make_queries(cfg, starts)
    q = qh.to(DEV)
    ctx = W.context_lengths(cfg)
    plan = DecodePlan(slow, ctx, DEV)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(qh)
    refs = [O.decode_run(qb[:, b], Kb[b], Vb[b], int(ctx[b]), slow[:, b], lam=cfg.lam, k=cfg.k,
                         n_sink=cfg.n_sink, window=cfg.window) for b in range(cfg.B)]
    decs = [SFIDecoder(K, V, cfg.Hq, int(ctx.max()) + cfg.steps, n_sink=cfg.n_sink,
                       window=cfg.window, k=cfg.k, lam=cfg.lam, keep_fused=True) for _ in range(2)]
    ties = 0
    for s in range(cfg.steps):
        for co, dec in zip((True, False), decs):
            dec.step(plan, s, q, co=co)
        torch.cuda.synchronize()
        o_co, o_sep = decs[0].out.cpu().numpy(), decs[1].out.cpu().numpy()
        for b in range(cfg.B):
            r = refs[b][s]
            assert row_rel_err(o_co[b], r["o"]) <= OUT_TOL, (s, b)
            assert row_rel_err(o_sep[b], o_co[b]) <= OUT_TOL, (s, b)
            if r["kind"] == "slow":
                sel = decs[0].sel_idx[b].cpu().numpy()
                cnt = decs[0].sel_count[b].cpu().numpy()
                for g in range(cfg.Hkv):
                    ties += check_selection(sel[g], cnt[g], r["s"][g], r["lo"], r["hi"], cfg.k)
    _say(f"  near-tie differences over the run: {ties}")
    assert ties == 0


@pytest.mark.parametrize("Hq,Hkv,d,paged", [(32, 8, 128, False), (32, 8, 128, True), (8, 2, 64, True)],
                         ids=["hkv8-d128", "hkv8-d128-paged", "hkv2-d64-paged"])
def test_ragged_run_with_len_hints(Hq, Hkv, d, paged):
    """A ragged batch (six sequences of 60 to 9000 keys, each with its own
    slow/fast schedule, rows appended by the steps): with the host row-count
    hints every launch plans each sequence's workgroups from its own length
    (a work table).  Outputs, fused scores and selections follow the
    oracle's decode run of every sequence; a run without hints agrees within
    tolerance and selects the same keys; a step given over-stated hints
    agrees with the exact ones within tolerance."""
    _say(f"ragged run with length hints, Hq={Hq} Hkv={Hkv} d={d} paged={paged}")
    B, k = 6, 200
    ctx = np.array([9000, 60, 2500, 300, 6000, 1200])
    steps = 10
    rng = np.random.default_rng(11)
    slow = rng.random((steps, B)) < 0.35
    slow[0] = True
    assert any(slow[s].any() and (~slow[s]).any() for s in range(steps))
    cap = int(ctx.max()) + steps + 8
    K, V = _rand_kv(B, Hkv, cap, d, seed=710, hh=9)
    q = _rand_q((steps, B, Hq, d), seed=711)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    refs = [O.decode_run(qb[:, b], Kb[b], Vb[b], int(ctx[b]), slow[:, b], lam=0.3, k=k, n_sink=4,
                         window=256) for b in range(B)]
    plan = DecodePlan(slow, ctx, DEV)
    max_len = int(ctx.max()) + steps
    kw = dict(n_sink=4, window=256, k=k, lam=0.3, keep_fused=True)
    decs, news = [], []
    for _ in range(2):
        if paged:
            cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=B, Hq=Hq, Hkv=Hkv, d=d)
            table, npages = W.page_table(cfg, np.full(B, cap))
            Kd, Vd = W.to_paged(K, table, npages, 16), W.to_paged(V, table, npages, 16)
            news.append(W.take_decode_rows(Kd, Vd, ctx, steps, table=table))
            decs.append(SFIDecoder(Kd, Vd, Hq, max_len, page_table=torch.from_numpy(table).to(DEV),
                                   page_size=16, **kw))
        else:
            Kd, Vd = K.clone(), V.clone()
            news.append(W.take_decode_rows(Kd, Vd, ctx, steps))
            decs.append(SFIDecoder(Kd, Vd, Hq, max_len, **kw))
    ties = 0
    for s in range(steps):
        decs[0].step(plan, s, q, new_kv=news[0])
        decs[1].step(plan, s, q, new_kv=news[1], hints=False)
        torch.cuda.synchronize()
        o_h, o_n = decs[0].out.cpu().numpy(), decs[1].out.cpu().numpy()
        for b in range(B):
            r = refs[b][s]
            assert row_rel_err(o_h[b], r["o"]) <= OUT_TOL, (s, b)
            assert row_rel_err(o_n[b], o_h[b]) <= OUT_TOL, (s, b)
            if r["kind"] == "slow":
                sel = decs[0].sel_idx[b].cpu().numpy()
                cnt = decs[0].sel_count[b].cpu().numpy()
                for g in range(Hkv):
                    ties += check_selection(sel[g], cnt[g], r["s"][g], r["lo"], r["hi"], k)
                assert row_rel_err(decs[0].fused[b, :, : r["n"]].cpu().numpy(), r["s"]) <= EVID_TOL
        assert torch.equal(decs[0].sel_idx, decs[1].sel_idx), s
        assert torch.equal(decs[0].sel_count, decs[1].sel_count), s
    _say(f"  near-tie differences over the run: {ties}")
    assert ties == 0
    # one co-launched step over the final cache: exact against over-stated hints
    dec = decs[0]
    lens = plan.seq_len_host[steps - 1].astype(np.int64)
    sb, fb = [0, 3], [1, 2, 4, 5]
    bound = np.minimum(lens, 260) + np.minimum(k, np.maximum(lens - 260, 0))
    exact = (lens[sb].astype(np.int32), bound[fb].astype(np.int32))
    over = (np.full(len(sb), max_len, dtype=np.int32), np.full(len(fb), 4 + 256 + k, dtype=np.int32))
    sids = torch.tensor(sb, dtype=torch.int32, device=DEV)
    fids = torch.tensor(fb, dtype=torch.int32, device=DEV)
    res = []
    for h in (exact, over):
        dec.co_step(q[steps - 1], plan.seq_len[steps - 1], sids, len(sb), fids, len(fb), select=False,
                    len_hints=h)
        torch.cuda.synchronize()
        res.append((dec.out.cpu().numpy(), dec.evidence.cpu().numpy()))
    for b in sb + fb:
        assert row_rel_err(res[1][0][b], res[0][0][b]) <= OUT_TOL, b
    for b in sb:
        n = int(lens[b])
        assert row_rel_err(res[1][1][b, :, :n], res[0][1][b, :, :n]) <= EVID_TOL, b


def test_len_hints_long_list_keeps_plain_plan():
    """More listed entries than a work table holds (300 > 256): with hints
    the co-launched step keeps the plain grid, sized from the longest hint.
    Outputs against the call without hints and, for sampled sequences,
    against the oracle; evidence of the slow ones likewise."""
    _say("length hints, 300 listed entries")
    B, Hq, Hkv, d, k = 300, 8, 2, 64, 16
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 400, size=B)
    lens[7] = 1
    cap = 416
    K, V = _rand_kv(B, Hkv, cap, d, seed=730, hh=3)
    q = _rand_q((B, Hq, d), seed=731)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        mid = np.arange(4, max(4, lens[b] - 32))
        for g in range(Hkv):
            c = min(k, len(mid))
            if c:
                sel[b, g, :c] = np.sort(rng.choice(mid, c, replace=False))
            cnt[b, g] = c
    slow_b = list(range(0, B, 7))
    fast_b = [b for b in range(B) if b % 7]
    sids = torch.tensor(slow_b, dtype=torch.int32, device=DEV)
    fids = torch.tensor(fast_b, dtype=torch.int32, device=DEV)
    lens64 = lens.astype(np.int64)
    bound = np.minimum(lens64, 36) + cnt.max(axis=1)
    hints = (lens[slow_b].astype(np.int32), bound[fast_b].astype(np.int32))
    res = []
    for h in (None, hints):
        dec = SFIDecoder(K, V, Hq, cap, n_sink=4, window=32, k=k, lam=0.3)
        dec.sel_idx.copy_(torch.from_numpy(sel))
        dec.sel_count.copy_(torch.from_numpy(cnt))
        dec.co_step(q, seq, sids, len(slow_b), fids, len(fast_b), select=False, len_hints=h)
        torch.cuda.synchronize()
        res.append((dec.out.cpu().numpy(), dec.evidence.cpu().numpy()))
    for b in range(B):
        assert row_rel_err(res[1][0][b], res[0][0][b]) <= OUT_TOL, b
    for b in slow_b:
        n = int(lens[b])
        assert row_rel_err(res[1][1][b, :, :n], res[0][1][b, :, :n]) <= EVID_TOL, b
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for b in slow_b[:5]:
        o_ref, _ = O.dense_step(qb[b], Kb[b], Vb[b], int(lens[b]))
        assert row_rel_err(res[1][0][b], o_ref) <= OUT_TOL, b
    for b in fast_b[:8] + [7]:
        lists = [sel[b, g, : cnt[b, g]] for g in range(Hkv)]
        o_ref = O.fast_step(qb[b], Kb[b], Vb[b], int(lens[b]), lists, 4, 32)
        assert row_rel_err(res[1][0][b], o_ref) <= OUT_TOL, b


@pytest.mark.parametrize("kdiv,nms", [(0, False), (16, False), (0, True)])
def test_layer_pipeline_matches_per_layer_calls(kdiv, nms):
    """sfi_decode_layer_step over a 3-layer stack, each layer's selection run
    inside the next layer's grids (and across the step boundary), against
    sfi_decode_step_select per layer: outputs and selections bit for bit.
    Steps: all slow, mixed, all fast, all slow, mixed; per-sequence k with
    kdiv > 0; Soft-NMS (radius 3, alpha 0.4) with nms."""
    _say(f"layer pipeline, kdiv={kdiv}, nms={nms}")
    B, Hq, Hkv, d, L = 4, 32, 8, 128, 3
    ctx = np.array([6000, 4500, 7000, 2600])
    slow = np.array([[1, 1, 1, 1], [0, 1, 0, 1], [0, 0, 0, 0], [1, 1, 1, 1], [1, 0, 0, 0]], dtype=bool)
    steps = slow.shape[0]
    cap = int(ctx.max()) + steps + 1
    plan = DecodePlan(slow, ctx, DEV, k_cap=300 if kdiv else 0, k_div=kdiv)
    kw = dict(n_sink=4, window=256, k=300, lam=0.3)
    if nms:
        kw.update(nms_radius=3, nms_alpha=0.4)
    layers = []
    for layer in range(L):
        K, V = _rand_kv(B, Hkv, cap, d, seed=90 + layer, hh=25)
        q = _rand_q((steps, B, Hq, d), seed=95 + layer)
        layers.append((K, V, q))
    pipe = [SFIDecoder(K, V, Hq, cap, **kw) for K, V, _ in layers]
    ref = [SFIDecoder(K, V, Hq, cap, **kw) for K, V, _ in layers]
    outs_p, outs_r = [], []
    pend = None
    for s in range(steps):
        for layer in range(L):
            q = layers[layer][2]
            pend = pipe[layer].layer_step(plan, s, q, pending=pend)
            ks = None if plan.k_seq is None else plan.k_seq[s]
            ref[layer].step_select(q[s], plan.seq_len[s], plan.slow_ids[s], int(plan.n_slow[s]),
                                   plan.fast_ids[s], int(plan.n_fast[s]), k_seq=ks,
                                   len_hints=ref[layer].hints(plan, s))
            outs_p.append(pipe[layer].out.clone())
            outs_r.append(ref[layer].out.clone())
    sfi.sfi_run_deferred(pend)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs_p, outs_r)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"out, step {i // L} layer {i % L}"
    for layer in range(L):
        assert torch.equal(pipe[layer].sel_idx, ref[layer].sel_idx), layer
        assert torch.equal(pipe[layer].sel_count, ref[layer].sel_count), layer
    # the last step's slow sequence against the oracle (layer 1)
    K, V, q = layers[1]
    s, b = steps - 1, 0
    n = int(plan.seq_len_host[s, b])
    kb = min(300, n // kdiv) if kdiv else 300
    r = O.slow_select(_bits(q[s, b]), _bits(K[b]), _bits(V[b]), n, lam=0.3, k=kb, n_sink=4, window=256)
    sel, cnt = pipe[1].sel_idx.cpu().numpy(), pipe[1].sel_count.cpu().numpy()
    if nms:
        ties = _check_refined(sel[b, :, :kb], cnt[b], list(r["s"]), r["lo"], r["hi"], kb, 3, 0.4, 0.0)
    else:
        ties = sum(check_selection(sel[b, g, :kb], cnt[b, g], r["s"][g], r["lo"], r["hi"], kb)
                   for g in range(Hkv))
    assert row_rel_err(pipe[1].out[b].cpu().numpy(), r["o"]) <= OUT_TOL
    _say(f"  near-tie differences: {ties}")


def _norm_sums(Kf, n):
    """fp64 sum and sum of squares of the L2 norms of rows [0, n) of each
    kv head (Kf: [Hkv][rows][d], the bf16 values as float)."""
    nu = np.sqrt((Kf[:, :n].astype(np.float64) ** 2).sum(-1))
    return np.stack([nu.sum(-1), (nu * nu).sum(-1)], axis=-1)


@pytest.mark.parametrize("paged", [False, True])
def test_norm_stats_prior_matches_the_pass(paged):
    """Key-norm statistics: a prior-forming step stores the exact sums of
    its pass, sfi_append_kv and fused appends add the new rows' norms, and a
    step whose prior comes from the statistics (key pass in its finalize)
    gives the same attention bits as the step that forms the prior from its
    pass, fused scores within the evidence tolerance and selections that
    match the oracle's Top-K."""
    _say(f"norm statistics prior, paged={paged}")
    B, Hq, Hkv, d = 4, 32, 8, 128
    lens = [6100, 4500, 7000, 2600]
    cap = 7200
    K, V = _rand_kv(B, Hkv, cap, d, seed=71, hh=30)
    q = _rand_q((B, Hq, d), seed=72)
    kw = dict(n_sink=4, window=256, k=300, lam=0.3, keep_fused=True)
    if paged:
        cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=B, Hq=Hq, Hkv=Hkv, d=d)
        table, npages = W.page_table(cfg, np.full(B, cap))
        Kp, Vp = W.to_paged(K, table, npages, 16), W.to_paged(V, table, npages, 16)
        tab = torch.from_numpy(table).to(DEV)
        mk = lambda: SFIDecoder(Kp, Vp, Hq, cap, page_table=tab, page_size=16, **kw)
    else:
        mk = lambda: SFIDecoder(K, V, Hq, cap, **kw)
    st, ex = mk(), mk()      # the statistics-prior decoder and the exact one
    all_ids = torch.arange(B, dtype=torch.int32, device=DEV)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    # step A: every sequence slow, prior from the pass: the exact sums
    for dec in (st, ex):
        dec.step_select(q, seq, all_ids, B, None, 0)
    torch.cuda.synchronize()
    kn = st.key_norm.double().cpu().numpy()
    got = st.nstat.cpu().numpy()
    for b in range(B):
        want = np.stack([kn[b, :, : lens[b]].sum(-1), (kn[b, :, : lens[b]] ** 2).sum(-1)], -1)
        np.testing.assert_allclose(got[b], want, rtol=1e-12)
    np.testing.assert_array_equal(got, ex.nstat.cpu().numpy())
    # three rows appended by sfi_append_kv, one by each step's fused append
    g = torch.Generator(device=DEV).manual_seed(73)
    rows = torch.randn((B, 4, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vrows = torch.randn((B, 4, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    seq3 = seq + 3
    before = st.nstat.clone()
    for dec in (st, ex):
        dec.append(rows[:, :3].contiguous(), vrows[:, :3].contiguous(), seq3, None, B)
    torch.cuda.synchronize()
    rb = rows.double().cpu().numpy()                          # [B][4][Hkv][d]
    nu = np.sqrt((rb ** 2).sum(-1))                           # [B][4][Hkv]
    add = np.stack([nu[:, :3].sum(1), (nu[:, :3] ** 2).sum(1)], -1)
    np.testing.assert_allclose((st.nstat - before).cpu().numpy(), add, rtol=1e-5)
    # step B: 1 and 3 slow, 0 and 2 fast, with the step's own row fused
    seq4 = seq + 4
    nr = (rows[:, 3].contiguous(), vrows[:, 3].contiguous())
    slow_ids = torch.tensor([1, 3], dtype=torch.int32, device=DEV)
    fast_ids = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    kseq = torch.tensor([300, 300, 300, 97], dtype=torch.int32, device=DEV)   # sequence 3 keeps 97
    st.step_select(q, seq4, slow_ids, 2, fast_ids, 2, new_rows=nr, use_stats=True, k_seq=kseq)
    ex.step_select(q, seq4, slow_ids, 2, fast_ids, 2, new_rows=nr, k_seq=kseq)
    torch.cuda.synchronize()
    for t in ("out", "evidence", "key_norm"):
        assert torch.equal(getattr(st, t).view(torch.int32), getattr(ex, t).view(torch.int32)), t
    a, e = st.nstat.cpu().numpy(), ex.nstat.cpu().numpy()
    np.testing.assert_allclose(a, e, rtol=1e-9)
    for b in (0, 2):      # fast sequences: the fused row's norm added
        np.testing.assert_allclose(a[b] - before.cpu().numpy()[b],
                                   add[b] + np.stack([nu[b, 3], nu[b, 3] ** 2], -1), rtol=1e-5)
    # slow sequences: selections and fused scores against the oracle, over
    # the cache as it now stands
    if paged:
        Kg = torch.stack([W.gather_paged(Kp, table, b, cap) for b in range(B)])
        Vg = torch.stack([W.gather_paged(Vp, table, b, cap) for b in range(B)])
    else:
        Kg, Vg = K, V
    Kb, Vb, qb = _bits(Kg), _bits(Vg), _bits(q)
    Kf = Kg.float().cpu().numpy()
    sel, cnt = st.sel_idx.cpu().numpy(), st.sel_count.cpu().numpy()
    sel_e, cnt_e = ex.sel_idx.cpu().numpy(), ex.sel_count.cpu().numpy()
    ties = 0
    for b in (1, 3):
        n = lens[b] + 4
        kb = 300 if b == 1 else 97
        r = O.slow_select(qb[b], Kb[b], Vb[b], n, lam=0.3, k=kb, n_sink=4, window=256)
        np.testing.assert_allclose(a[b], _norm_sums(Kf[b], n), rtol=1e-5)
        assert row_rel_err(st.fused[b, :, :n].cpu().numpy(), r["s"]) <= EVID_TOL
        for g in range(Hkv):
            ties += check_selection(sel[b, g, :kb], cnt[b, g], r["s"][g], r["lo"], r["hi"], kb)
            ties += check_selection(sel_e[b, g, :kb], cnt_e[b, g], r["s"][g], r["lo"], r["hi"], kb)
            assert np.all(sel[b, g, kb:] == -1)
    _say(f"  near-tie differences: {ties}")


def test_norm_stats_append_short_and_unlisted():
    """sfi_append_kv with key-norm statistics: T rows appended to a sequence
    holding fewer than T rows add only the rows that land (j >= 0), and a
    sequence the call does not list keeps its sums."""
    _say("norm statistics: short appends")
    B, Hq, Hkv, d, T = 3, 8, 2, 128, 8
    lens = [5, 40, 300]
    cap = 320
    K, V = _rand_kv(B, Hkv, cap, d, seed=81)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    nstat = torch.zeros((B, Hkv, 2), dtype=torch.float64, device=DEV)
    nstat[:, :, 0] = 1.0      # arbitrary earlier sums
    nstat[:, :, 1] = 2.0
    kv = sfi.with_norm_stats(sfi.make_kv(K, V, seq, Hq, cap), nstat, False)
    g = torch.Generator(device=DEV).manual_seed(82)
    kn = torch.randn((B, T, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, T, Hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    ids = torch.tensor([0, 1], dtype=torch.int32, device=DEV)     # sequence 2 not listed
    sfi.sfi_append_kv(kv, ids, 2, kn, vn, T)
    torch.cuda.synchronize()
    nu = np.sqrt((kn.double().cpu().numpy() ** 2).sum(-1))      # [B][T][Hkv]
    got = nstat.cpu().numpy()
    for b in range(B):
        t0 = max(0, T - lens[b]) if b < 2 else T                  # rows j = n - T + t >= 0
        want = np.stack([1.0 + nu[b, t0:].sum(0), 2.0 + (nu[b, t0:] ** 2).sum(0)], -1)
        np.testing.assert_allclose(got[b], want, rtol=1e-6)


def test_decode_run_with_stats_prior_vs_oracle():
    """A decode run whose steps append their own rows: after a sequence's
    first slow step, its later slow steps form the prior from the key-norm
    statistics.  Every step's output, and every slow step's fused scores and
    selection, against the oracle's decode run; the statistics at the end
    against the sums of the cache rows' norms."""
    _say("decode run, statistics prior")
    cfg = W.CONFIGS["tiny-4k"].replace(B=2, steps=48)
    K, V = W.make_kv(cfg, device=DEV)
    starts = W.sentence_starts(cfg)
    slow = O.schedule(starts, cfg.budget)
    qh = W.make_queries(cfg, starts)
    q = qh.to(DEV)
    ctx = W.context_lengths(cfg)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(qh)
    Kf = K.float().cpu().numpy()
    new_kv = W.take_decode_rows(K, V, ctx, cfg.steps)
    plan = DecodePlan(slow, ctx, DEV)
    dec = SFIDecoder(K, V, cfg.Hq, int(ctx.max()) + cfg.steps, n_sink=cfg.n_sink, window=cfg.window,
                     k=cfg.k, lam=cfg.lam, keep_fused=True)
    refs = [O.decode_run(qb[:, b], Kb[b], Vb[b], int(ctx[b]), slow[:, b], lam=cfg.lam, k=cfg.k,
                         n_sink=cfg.n_sink, window=cfg.window) for b in range(cfg.B)]
    used, ties = 0, 0
    for s in range(cfg.steps):
        used += int(dec._stats_current(plan, s))
        dec.step(plan, s, q, new_kv=new_kv)
        torch.cuda.synchronize()
        out = dec.out.cpu().numpy()
        for b in range(cfg.B):
            r = refs[b][s]
            assert row_rel_err(out[b], r["o"]) <= OUT_TOL, (s, b)
            if r["kind"] == "slow":
                sel = dec.sel_idx[b].cpu().numpy()
                cnt = dec.sel_count[b].cpu().numpy()
                for g in range(cfg.Hkv):
                    ties += check_selection(sel[g], cnt[g], r["s"][g], r["lo"], r["hi"], cfg.k)
                assert row_rel_err(dec.fused[b, :, : r["n"]].cpu().numpy(), r["s"]) <= EVID_TOL
    assert used > 0, "no step formed its prior from the statistics"
    got = dec.nstat.cpu().numpy()
    for b in range(cfg.B):
        np.testing.assert_allclose(got[b], _norm_sums(Kf[b], int(ctx[b]) + cfg.steps), rtol=1e-5)
    _say(f"  steps with the statistics prior: {used}; near-tie differences: {ties}")
    assert ties == 0


@pytest.mark.parametrize("paged", [False, True])
def test_decode_step_select_matches_separate_calls(paged):
    """sfi_decode_step_select (one call: co-launched step + the slow
    sequences' selections, prior statistics formed by the slow step) against
    sfi_decode_step + sfi_select and the oracle, with a per-sequence k."""
    _say(f"decode step + select, paged={paged}")
    B, Hq, Hkv, d = 4, 32, 8, 128
    lens = [6100, 4500, 7000, 2600]
    cap = 7100
    K, V = _rand_kv(B, Hkv, cap, d, seed=61, hh=30)
    q = _rand_q((B, Hq, d), seed=62)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kseq = torch.tensor([300, 120, 300, 64], dtype=torch.int32, device=DEV)
    kw = dict(n_sink=4, window=256, k=300, lam=0.3)
    if paged:
        cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=B, Hq=Hq, Hkv=Hkv, d=d)
        table, npages = W.page_table(cfg, np.full(B, cap))
        Kp, Vp = W.to_paged(K, table, npages, 16), W.to_paged(V, table, npages, 16)
        tab = torch.from_numpy(table).to(DEV)
        mk = lambda: SFIDecoder(Kp, Vp, Hq, cap, page_table=tab, page_size=16, **kw)
    else:
        mk = lambda: SFIDecoder(K, V, Hq, cap, **kw)
    fused, sep = mk(), mk()
    all_ids = torch.arange(B, dtype=torch.int32, device=DEV)
    # step A: every sequence slow (slow-only call); step B: 1 and 3 slow, 0 and 2 fast
    for dec, f in ((fused, True), (sep, False)):
        if f:
            dec.step_select(q, seq, all_ids, B, None, 0, k_seq=kseq)
        else:
            dec.slow(q, seq, all_ids, B, k_seq=kseq)
    torch.cuda.synchronize()
    for t in ("out", "evidence", "key_norm"):
        assert torch.equal(getattr(fused, t).view(torch.int32), getattr(sep, t).view(torch.int32)), t
    slow_ids = torch.tensor([1, 3], dtype=torch.int32, device=DEV)
    fast_ids = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    seq2 = seq + 5
    fused.step_select(q, seq2, slow_ids, 2, fast_ids, 2, k_seq=kseq)
    sep.co_step(q, seq2, slow_ids, 2, fast_ids, 2, k_seq=kseq)
    torch.cuda.synchronize()
    # slow sequences: identical kernels; fast ones read the step-A selections,
    # which may differ only in near-tie keys
    for b in (1, 3):
        assert torch.equal(fused.out[b].view(torch.int32), sep.out[b].view(torch.int32))
    assert row_rel_err(fused.out.cpu().numpy(), sep.out.cpu().numpy()) <= OUT_TOL
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    sel, cnt = fused.sel_idx.cpu().numpy(), fused.sel_count.cpu().numpy()
    ties = 0
    for b in range(B):
        n = lens[b] + 5
        kb = int(kseq[b])
        r = O.slow_select(qb[b], Kb[b], Vb[b], n if b in (1, 3) else lens[b], lam=0.3, k=kb,
                          n_sink=4, window=256)
        for g in range(Hkv):
            ties += check_selection(sel[b, g, :kb], cnt[b, g], r["s"][g], r["lo"], r["hi"], kb)
            assert np.all(sel[b, g, kb:] == -1)
    _say(f"  near-tie differences: {ties}")


# ------------------------------------------------------------------- verify

@pytest.mark.parametrize("Hq,Hkv,d,T", [(32, 8, 128, 8), (8, 2, 64, 8), (16, 8, 128, 4), (8, 8, 128, 1)])
def test_verify_matches_oracle(Hq, Hkv, d, T):
    _say(f"verify Hq={Hq} Hkv={Hkv} d={d} T={T}")
    B = 2
    lens = [3000, 1111]
    K, V = _rand_kv(B, Hkv, 3000, d, seed=Hq * 7 + T)
    q = _rand_q((B, T, Hq, d), seed=T + 100)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    vd = VegasDecoder(K, V, Hq, max(lens), T, n_sink=4, window=256, k=256)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for mode in ("all", "c2q"):
        rows = O.collect_rows(T, mode)
        mask = sum(1 << t for t in rows)
        vd.agg.fill_(123.0)
        vd.verify(q, seq, mask)
        vd.select(seq)
        torch.cuda.synchronize()
        out = vd.vout.cpu().numpy()
        agg = vd.agg.cpu().numpy()
        sel = vd.sel_idx.cpu().numpy()
        cnt = vd.sel_count.cpu().numpy()
        for b in range(B):
            n = lens[b]
            o_ref, a_ref = O.verify(qb[b], Kb[b], Vb[b], n, rows)
            for t in range(T):
                assert row_rel_err(out[b, t], o_ref[t]) <= OUT_TOL, (mode, b, t)
            P = n - T
            err = np.abs(agg[b, :P] - a_ref).max() / np.abs(a_ref).max()
            assert err <= 1e-5, (mode, b, err)
            assert np.all(agg[b, P:n] == 123.0)          # no writes past the prefix
            lo, hi = O.candidate_range(n, 4, 256)
            check_selection(sel[b, 0], cnt[b, 0], a_ref, lo, hi, 256)


@pytest.mark.parametrize("Hq,Hkv,d,T,paged", [(32, 8, 128, 8, False), (8, 2, 64, 8, True), (16, 8, 128, 4, False)])
def test_verify_raw_logits_match_oracle(Hq, Hkv, d, T, paged):
    """Raw-logit emission: the collected rows' pre-softmax logits against the
    oracle's, element by element per row; their sum (a second pass) against
    the oracle's aggregate and the in-kernel aggregate; outputs equal to the
    aggregating call's bit for bit; nothing written past the prefix."""
    _say(f"verify raw logits Hq={Hq} Hkv={Hkv} d={d} T={T} paged={paged}")
    B = 2
    lens = [2600, 905]
    cap = 2624
    K, V = _rand_kv(B, Hkv, cap, d, seed=Hq * 3 + T + 1)
    q = _rand_q((B, T, Hq, d), seed=T + 200)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    if paged:
        ps = 16
        npg = cap // ps
        table = np.random.default_rng(3).permutation(B * npg).astype(np.int32).reshape(B, npg)
        tab = torch.from_numpy(table).to(DEV)
        vd = VegasDecoder(W.to_paged(K, table, B * npg, ps), W.to_paged(V, table, B * npg, ps), Hq, cap, T,
                          n_sink=4, window=256, k=256, page_table=tab, page_size=ps, keep_raw=True)
    else:
        vd = VegasDecoder(K, V, Hq, cap, T, n_sink=4, window=256, k=256, keep_raw=True)
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for mode in ("all", "c2q"):
        rows = O.collect_rows(T, mode)
        mask = sum(1 << t for t in rows)
        vd.verify(q, seq, mask)
        torch.cuda.synchronize()
        out_agg, agg_in = vd.vout.clone(), vd.agg.clone()
        vd.raw_logits.fill_(7.0)
        vd.agg.fill_(123.0)
        vd.verify(q, seq, mask, raw=True)
        torch.cuda.synchronize()
        assert torch.equal(vd.vout.view(torch.int32), out_agg.view(torch.int32))
        raw = vd.raw_view(len(rows)).cpu().numpy()
        # nothing written past the [B][R][Hq][ld] block of this call
        assert torch.all(vd.raw_logits.view(-1)[raw.size:] == 7.0)
        agg = vd.agg.cpu().numpy()
        for b in range(B):
            n = lens[b]
            P = n - T
            _, a_ref = O.verify(qb[b], Kb[b], Vb[b], n, rows)
            for r, t in enumerate(rows):
                l_ref = O.attention_logits(qb[b, t], Kb[b], n - T + t + 1)[:, :P]
                assert row_rel_err(raw[b, r, :, :P], l_ref) <= 1e-5, (mode, b, t)
                assert np.all(raw[b, r, :, P:] == 7.0)                # nothing past the prefix
            err = np.abs(agg[b, :P] - a_ref).max() / np.abs(a_ref).max()
            assert err <= 1e-5, (mode, b, err)
            err_in = np.abs(agg[b, :P] - agg_in.cpu().numpy()[b, :P]).max() / np.abs(a_ref).max()
            assert err_in <= 1e-6, (mode, b, err_in)
            assert np.all(agg[b, P:n] == 123.0)


def test_vegas_draft_steps_with_shared_selection():
    B, Hq, Hkv, d, T = 2, 32, 8, 128, 8
    n0 = 2600
    K, V = _rand_kv(B, Hkv, n0 + 8, d, seed=31)
    q = _rand_q((B, T, Hq, d), seed=32)
    seq = torch.full((B,), n0, dtype=torch.int32, device=DEV)
    vd = VegasDecoder(K, V, Hq, n0 + 7, T, n_sink=4, window=256, k=512)
    vd.verify(q, seq, 0xFF)
    vd.select(seq)
    torch.cuda.synchronize()
    sel = vd.sel_idx.cpu().numpy()
    cnt = vd.sel_count.cpu().numpy()
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    for j in range(1, 8):
        seqj = torch.full((B,), n0 + j - 1 + 1, dtype=torch.int32, device=DEV)
        qd = _rand_q((B, Hq, d), seed=40 + j)
        vd.draft(qd, seqj)
        torch.cuda.synchronize()
        out = vd.out.cpu().numpy()
        qdb = _bits(qd)
        for b in range(B):
            lst = [sel[b, 0, : cnt[b, 0]]] * Hkv
            o_ref = O.fast_step(qdb[b], Kb[b], Vb[b], n0 + j, lst, 4, 256)
            assert row_rel_err(out[b], o_ref) <= OUT_TOL


# -------------------------------------------------------------------- paged

def test_paged_cache_matches_contiguous_and_oracle():
    _say("paged")
    cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=4, Hq=40, Hkv=8, d=128, ctx=6000, ragged_min=1000, steps=2)
    ctx = W.context_lengths(cfg)
    K, V = W.make_kv(cfg, device=DEV)
    cap = K.shape[2]
    table, npages = W.page_table(cfg, np.full(cfg.B, cap))
    Kp = W.to_paged(K, table, npages, 16)
    Vp = W.to_paged(V, table, npages, 16)
    tab = torch.from_numpy(table).to(DEV)
    lens = [int(c) + 1 for c in ctx]
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = _rand_q((cfg.B, cfg.Hq, cfg.d), seed=55)
    ml = max(lens)
    dc = SFIDecoder(K, V, cfg.Hq, ml, n_sink=4, window=256, k=128, lam=0.3)
    dp = SFIDecoder(Kp, Vp, cfg.Hq, ml, n_sink=4, window=256, k=128, lam=0.3, page_table=tab, page_size=16)
    for d_ in (dc, dp):
        d_.slow(q, seq, None, cfg.B)
        d_.fast(q, seq, None, cfg.B)
    torch.cuda.synchronize()
    assert torch.equal(dc.sel_idx, dp.sel_idx)
    assert torch.equal(dc.out.view(torch.int32), dp.out.view(torch.int32))
    Kb, Vb, qb = _bits(K), _bits(V), _bits(q)
    sel = dp.sel_idx.cpu().numpy()
    cnt = dp.sel_count.cpu().numpy()
    out = dp.out.cpu().numpy()
    for b in range(cfg.B):
        lists = [sel[b, g, : cnt[b, g]] for g in range(cfg.Hkv)]
        o_ref = O.fast_step(qb[b], Kb[b], Vb[b], lens[b], lists, 4, 256)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_step_select_then_fast(seed):
    """Seeded sweep over shapes and parameters: GQA group 1/2/4/5/8, d 64/128,
    contiguous or paged, ragged lengths from 1 to ~6000 (several below
    sinks + window), sinks 0/4/16, window 0/64/256, k 16..1000, lambda 0..1.
    One sfi_decode_step_select over a random slow/fast split (fast sequences
    use planted selections), then a fast step for every sequence a few keys
    later with the new selections; all against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    Hq, Hkv = [(8, 2), (32, 8), (40, 8), (8, 8), (16, 2), (16, 8)][rng.integers(6)]
    d = int(rng.choice([64, 128]))
    paged = bool(rng.integers(2))
    B = int(rng.integers(1, 6))
    n_sink = int(rng.choice([0, 4, 16]))
    window = int(rng.choice([0, 64, 256]))
    k = int(rng.choice([16, 200, 1000]))
    lam = float(rng.choice([0.0, 0.3, 1.0]))
    lens = [int(x) for x in rng.integers(1, 6000, size=B)]
    lens[int(rng.integers(B))] = int(rng.integers(1, n_sink + window + 8))   # short one
    adv = int(rng.integers(1, 9))
    cap = (max(lens) + adv + 15) // 16 * 16
    _say(f"random seed={seed}: Hq={Hq} Hkv={Hkv} d={d} paged={paged} B={B} lens={lens} "
         f"sinks={n_sink} window={window} k={k} lam={lam}")
    K, V = _rand_kv(B, Hkv, cap, d, seed=2000 + seed, hh=5)
    q0 = _rand_q((B, Hq, d), seed=3000 + seed)
    q1 = _rand_q((B, Hq, d), seed=4000 + seed)
    ml = max(lens) + adv
    kw = {}
    if paged:
        cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=B, Hq=Hq, Hkv=Hkv, d=d)
        table, npages = W.page_table(cfg, np.full(B, cap))
        Kd, Vd = W.to_paged(K, table, npages, 16), W.to_paged(V, table, npages, 16)
        kw = dict(page_table=torch.from_numpy(table).to(DEV), page_size=16)
    else:
        Kd, Vd = K, V
    dec = SFIDecoder(Kd, Vd, Hq, ml, n_sink=n_sink, window=window, k=k, lam=lam, **kw)
    # planted selections for the sequences that take a fast step
    sel0 = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt0 = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            c = min(k, lens[b], int(rng.integers(0, k + 1)))
            sel0[b, g, :c] = np.sort(rng.choice(lens[b], c, replace=False))
            cnt0[b, g] = c
    dec.sel_idx.copy_(torch.from_numpy(sel0))
    dec.sel_count.copy_(torch.from_numpy(cnt0))
    order = rng.permutation(B)
    n_slow = int(rng.integers(1, B + 1))
    slow_b, fast_b = [int(x) for x in order[:n_slow]], [int(x) for x in order[n_slow:]]
    seq0 = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sids = torch.tensor(slow_b, dtype=torch.int32, device=DEV)
    fids = torch.tensor(fast_b if fast_b else [0], dtype=torch.int32, device=DEV)
    dec.step_select(q0, seq0, sids, len(slow_b), fids, len(fast_b))
    torch.cuda.synchronize()
    out = dec.out.cpu().numpy()
    sel = dec.sel_idx.cpu().numpy()
    cnt = dec.sel_count.cpu().numpy()
    Kb, Vb = _bits(K), _bits(V)
    qb0, qb1 = _bits(q0), _bits(q1)
    ties = 0
    for b in slow_b:
        n = lens[b]
        r = O.slow_select(qb0[b], Kb[b], Vb[b], n, lam=lam, k=k, n_sink=n_sink, window=window)
        assert row_rel_err(out[b], r["o"]) <= OUT_TOL
        for g in range(Hkv):
            ties += check_selection(sel[b, g], cnt[b, g], r["s"][g], r["lo"], r["hi"], k)
    for b in fast_b:
        lists = [sel0[b, g, : cnt0[b, g]] for g in range(Hkv)]
        o_ref = O.fast_step(qb0[b], Kb[b], Vb[b], lens[b], lists, n_sink, window)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL
    # every sequence a few keys later, with the selections now held
    lens1 = [n + adv for n in lens]
    seq1 = torch.tensor(lens1, dtype=torch.int32, device=DEV)
    dec.fast(q1, seq1, None, B)
    torch.cuda.synchronize()
    out1 = dec.out.cpu().numpy()
    for b in range(B):
        lists = [sel[b, g, : cnt[b, g]] for g in range(Hkv)]
        o_ref = O.fast_step(qb1[b], Kb[b], Vb[b], lens1[b], lists, n_sink, window)
        assert row_rel_err(out1[b], o_ref) <= OUT_TOL
    _say(f"  near-tie differences: {ties}")


@pytest.mark.parametrize("Hq,Hkv,d,w,paged", [(32, 8, 128, 8, False), (8, 2, 64, 4, True),
                                               (8, 8, 128, 16, False), (16, 8, 128, 1, False)])
def test_slow_step_window_matches_oracle(Hq, Hkv, d, w, paged):
    """sfi_slow_step_window: every window row's output, the window evidence
    and the key norms against the oracle (ragged lengths spanning several
    workgroups, a length not a multiple of the tile); with w = 1 the evidence
    is sfi_slow_step's; the FUSED selection over it matches the oracle's."""
    _say(f"slow window Hq={Hq} Hkv={Hkv} d={d} w={w} paged={paged}")
    B, cap = 2, 3008
    K, V = _rand_kv(B, Hkv, cap, d, seed=80 + w, hh=6)
    lens = [2999, 1717]
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = _rand_q((B, w, Hq, d), seed=81 + w)
    ml = max(lens)
    ld = ml + 5
    Kc, Vc = K, V
    table = None
    if paged:
        cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=B, Hq=Hq, Hkv=Hkv, d=d)
        table, npages = W.page_table(cfg, np.full(B, cap))
        K = W.to_paged(K, table, npages, 16)
        V = W.to_paged(V, table, npages, 16)
        tab = torch.from_numpy(table).to(DEV)      # kept alive: kv holds its raw pointer
        kv = sfi.make_kv(K, V, seq, Hq, ml, tab, 16)
    else:
        kv = sfi.make_kv(K, V, seq, Hq, ml)
    wsb = sfi.sfi_slow_window_workspace_bytes(kv, w)
    assert wsb > 0
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    out = torch.full((B, w, Hq, d), float("nan"), device=DEV)
    ev = torch.full((B, Hkv, ld), float("nan"), device=DEV)
    nrm = torch.full((B, Hkv, ld), float("nan"), device=DEV)
    sfi.sfi_slow_step_window(kv, None, B, q, w, out, ev, nrm, ld, ws, wsb)
    torch.cuda.synchronize()
    Kb, Vb, qb = _bits(Kc), _bits(Vc), _bits(q)
    o_g, ev_g, nrm_g = out.cpu().numpy(), ev.cpu().numpy(), nrm.cpu().numpy()
    f_refs = []
    for b in range(B):
        n = lens[b]
        o_ref, f_ref = O.window_evidence(qb[b], Kb[b], Vb[b], n)
        f_refs.append(f_ref)
        assert row_rel_err(o_g[b], o_ref) <= OUT_TOL
        assert row_rel_err(ev_g[b, :, :n], f_ref) <= EVID_TOL
        np.testing.assert_allclose(ev_g[b, :, :n].sum(axis=1), 1.0, rtol=1e-4)
        np.testing.assert_allclose(nrm_g[b, :, :n], O.key_norms(Kb[b], n), rtol=NORM_TOL)
        assert np.isnan(ev_g[b, :, n:]).all()          # nothing past the sequence
    if w == 1:
        dec = SFIDecoder(Kc, Vc, Hq, ml, n_sink=4, window=256, k=256, lam=0.3)
        dec.slow(q[:, 0].contiguous(), seq, None, B, select=False)
        torch.cuda.synchronize()
        for b in range(B):
            n = lens[b]
            assert row_rel_err(ev_g[b, :, :n], dec.evidence[b, :, :n].cpu().numpy()) <= EVID_TOL
    # the selector over the window evidence
    k = 300
    sel, cnt, fo = _select_gpu(sfi.SFI_SCORE_FUSED, torch.nan_to_num(ev[:, :, :ml]).contiguous(),
                               torch.nan_to_num(nrm[:, :, :ml]).contiguous(), lens, k, 4, 256, lam=0.3,
                               fused=True)
    ties = 0
    for b in range(B):
        n = lens[b]
        s_ref = O.fuse(f_refs[b], O.prior(Kb[b], n), 0.3)
        lo, hi = O.candidate_range(n, 4, 256)
        for g in range(Hkv):
            ties += check_selection(sel[b, g], cnt[b, g], s_ref[g], lo, hi, k)
    _say(f"  near-tie differences: {ties}")


@pytest.mark.parametrize("paged", [False, True])
def test_fast_compact_matches_index_gather(paged):
    """sfi_compact_selected + sfi_fast_step_compact: the same outputs bit for
    bit as the index-gather fast step, and the oracle's fast step, with the
    selection a few steps old (the keys that left the window since are
    dropped), ragged lengths (one sequence shorter than sinks + window, one with fewer
    candidates than k) and a batch subset in non-sorted order."""
    _say(f"fast compact paged={paged}")
    cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=4, Hq=32, Hkv=8, d=128)
    cap = 5008
    K, V = _rand_kv(cfg.B, cfg.Hkv, cap, cfg.d, seed=70, hh=8)
    lens0 = [4900, 200, 700, 3100]          # at the selection
    adv = 37                                # fast steps later
    lens1 = [n + adv for n in lens0]
    assert max(lens1) <= cap
    kwargs = {}
    if paged:
        table, npages = W.page_table(cfg, np.full(cfg.B, cap))
        K = W.to_paged(K, table, npages, 16)
        V = W.to_paged(V, table, npages, 16)
        kwargs = dict(page_table=torch.from_numpy(table).to(DEV), page_size=16)
    ml = max(lens1)
    k = 512
    dec = SFIDecoder(K, V, cfg.Hq, ml, n_sink=4, window=256, k=k, lam=0.3, **kwargs)
    q0 = _rand_q((cfg.B, cfg.Hq, cfg.d), seed=71)
    q1 = _rand_q((cfg.B, cfg.Hq, cfg.d), seed=72)
    seq0 = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    seq1 = torch.tensor(lens1, dtype=torch.int32, device=DEV)
    dec.slow(q0, seq0, None, cfg.B)
    dec.compact(seq0, None, cfg.B)
    ids = torch.tensor([3, 0, 1, 2], dtype=torch.int32, device=DEV)
    out_i = torch.full_like(dec.out, float("nan"))
    out_c = torch.full_like(dec.out, float("nan"))
    dec.fast(q1, seq1, ids, 4, out=out_i)
    dec.fast_compact(q1, seq1, ids, 4, out=out_c)
    # a subset (its own split plan): other rows untouched
    sub = torch.tensor([2, 3], dtype=torch.int32, device=DEV)
    out_s = torch.full_like(dec.out, float("nan"))
    out_si = torch.full_like(dec.out, float("nan"))
    dec.fast_compact(q1, seq1, sub, 2, out=out_s)
    dec.fast(q1, seq1, sub, 2, out=out_si)
    torch.cuda.synchronize()
    assert torch.equal(out_i.view(torch.int32), out_c.view(torch.int32))
    assert torch.equal(out_s.view(torch.int32), out_si.view(torch.int32))
    assert torch.isnan(out_s[:2]).all() and not torch.isnan(out_s[2:]).any()
    sel = dec.sel_idx.cpu().numpy()
    cnt = dec.sel_count.cpu().numpy()
    assert cnt[1].max() == 0 and 0 < cnt[2].max() < k        # the degenerate lengths
    Kd = _bits(K) if not paged else None
    qb = _bits(q1)
    out = out_c.cpu().numpy()
    for b in range(cfg.B):
        if paged:
            Kb = W.bf16_bits(_unpage(K, table, b, cap))
            Vb = W.bf16_bits(_unpage(V, table, b, cap))
        else:
            Kb, Vb = Kd[b], _bits(V[b])
        lists = [sel[b, g, : cnt[b, g]] for g in range(cfg.Hkv)]
        o_ref = O.fast_step(qb[b], Kb, Vb, lens1[b], lists, 4, 256)
        assert row_rel_err(out[b], o_ref) <= OUT_TOL


def _unpage(P, table, b, cap):
    """Contiguous [Hkv][cap][d] rows of sequence b from a paged pool."""
    npg = (cap + 15) // 16
    pages = torch.as_tensor(table[b, :npg].astype(np.int64), device=P.device)
    return P[pages].permute(1, 0, 2, 3).reshape(P.shape[1], npg * 16, P.shape[3])[:, :cap]


# ------------------------------------------------- full size, sampled outputs

def test_full_size_llama_layer_32k_sampled():
    """8 sequences x 32K context, Hq=32/Hkv=8, d=128, k=2048: the benchmark's
    launch shapes; the oracle checks two sampled sequences."""
    cfg = W.CONFIGS["llama3-8b-layer-32k"]
    _say("full size 32K")
    K, V = W.make_kv(cfg, device=DEV)
    ctx = W.context_lengths(cfg)
    ml = int(ctx.max()) + cfg.steps
    q = _rand_q((cfg.B, cfg.Hq, cfg.d), seed=99)
    lens = [int(ctx[b]) + 1 + 13 * b for b in range(cfg.B)]
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dec = SFIDecoder(K, V, cfg.Hq, ml, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k, lam=cfg.lam,
                     keep_fused=True)
    dec.slow(q, seq, None, cfg.B)
    torch.cuda.synchronize()
    out = dec.out.cpu().numpy()
    sel = dec.sel_idx.cpu().numpy()
    cnt = dec.sel_count.cpu().numpy()
    ties = 0
    for b in (0, 5):
        n = lens[b]
        Kb = _bits(K[b, :, :n])
        Vb = _bits(V[b, :, :n])
        qb = _bits(q[b])
        r = O.slow_select(qb, Kb, Vb, n, lam=cfg.lam, k=cfg.k, n_sink=cfg.n_sink, window=cfg.window)
        assert row_rel_err(out[b], r["o"]) <= OUT_TOL
        for g in range(cfg.Hkv):
            ties += check_selection(sel[b, g], cnt[b, g], r["s"][g], r["lo"], r["hi"], cfg.k)
        # fast step 10 tokens later with the oracle's own selection as input
        sel_in = np.full((cfg.B, cfg.Hkv, cfg.k), -1, dtype=np.int32)
        cnt_in = np.zeros((cfg.B, cfg.Hkv), dtype=np.int32)
        for g in range(cfg.Hkv):
            sel_in[:, g, : len(r["sel"][g])] = r["sel"][g]
            cnt_in[:, g] = len(r["sel"][g])
        lens_f = [min(x + 10, ml) for x in lens]
        of = _fast_gpu(K, V, cfg.Hq, q, lens_f, sel_in, cnt_in, cfg.n_sink, cfg.window, cfg.Hkv)
        Kf = _bits(K[b, :, : lens_f[b]])
        Vf = _bits(V[b, :, : lens_f[b]])
        o_ref = O.fast_step(qb, Kf, Vf, lens_f[b], r["sel"], cfg.n_sink, cfg.window)
        assert row_rel_err(of[b], o_ref) <= OUT_TOL
    _say(f"  near-tie differences: {ties}")


def test_full_size_llama_layer_32k_refined_sampled():
    """The 32K benchmark shapes (8 x 32K, Hq=32/Hkv=8, k=2048) through the
    combined step + selection call with Soft-NMS (radius 4, alpha 0.5) and
    exclusivity (beta 0.5): one sampled sequence against the oracle's slow
    step, fused score and refinements."""
    cfg = W.CONFIGS["llama3-8b-layer-32k"]
    _say("full size 32K, refined selection")
    K, V = W.make_kv(cfg, device=DEV)
    ctx = W.context_lengths(cfg)
    ml = int(ctx.max()) + cfg.steps
    q = _rand_q((cfg.B, cfg.Hq, cfg.d), seed=98)
    lens = [int(ctx[b]) + 1 + 7 * b for b in range(cfg.B)]
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dec = SFIDecoder(K, V, cfg.Hq, ml, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k, lam=cfg.lam,
                     nms_radius=4, nms_alpha=0.5, excl_beta=0.5)
    slow_ids = torch.tensor([5, 2], dtype=torch.int32, device=DEV)
    fast_ids = torch.tensor([0, 1, 3, 4, 6, 7], dtype=torch.int32, device=DEV)
    dec.step_select(q, seq, slow_ids, 2, fast_ids, 6)
    torch.cuda.synchronize()
    sel, cnt = dec.sel_idx.cpu().numpy(), dec.sel_count.cpu().numpy()
    b = 5
    n = lens[b]
    r = O.slow_select(_bits(q[b]), _bits(K[b, :, :n]), _bits(V[b, :, :n]), n, lam=cfg.lam, k=cfg.k,
                      n_sink=cfg.n_sink, window=cfg.window)
    assert row_rel_err(dec.out[b].cpu().numpy(), r["o"]) <= OUT_TOL
    diff = _check_refined(sel[b], cnt[b], list(r["s"]), r["lo"], r["hi"], cfg.k, 4, 0.5, 0.5)
    _say(f"  differing keys: {diff}")
