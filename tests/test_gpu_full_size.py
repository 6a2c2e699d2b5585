"""GPU parity at the full sizes of the long-context workloads, sampled.

Each test builds one workload at its real shape with the seeded generator,
runs the HIP path in the launch configuration the benchmark times (same
decoder classes, same list capacities and batch sizes) and checks sampled
sequences against the CPU oracle, which computes them one by one:

* one layer of the 32-layer stack at 128K context (B=4, Hq=32/Hkv=8, d=128,
  k=4096, lambda 0.2): slow step + selection + a later fast step;
* two layers of that stack with the cross-layer selection pipeline, against
  the per-layer calls, bit for bit;
* Vegas verification at 64K context (B=16, T=8): outputs of every verify
  row, the aggregate over ALL rows and Collect-2-Query, the head-shared
  top-2048 selection and a draft step;
* the ragged paged batch (B=32, contexts 8K-128K, 16-token pages in a
  shuffled pool, Hq=40/Hkv=8, k = min(4096, n/16) per sequence): a first
  all-slow step and a co-launched slow + fast step.

Expected values come only from oracle/; tolerances are in parity_util.py.
"""
import sys

import numpy as np
import pytest
import torch

from dynamic_sparse_kv_amd import sfi
from dynamic_sparse_kv_amd import workload as W
from dynamic_sparse_kv_amd.runner import DecodePlan, SFIDecoder, VegasDecoder
from oracle import sfi_oracle as O

from parity_util import OUT_TOL, check_selection, row_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(t):
    return W.bf16_bits(t)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_full_size_stack_layer_128k_sampled():
    cfg = W.CONFIGS["stack32-128k"]
    layer = 5
    _say("full size: one 128K layer of the 32-layer stack")
    ctx = W.context_lengths(cfg)
    ml = int(ctx.max()) + 16
    K, V = W.make_kv(cfg, layer=layer, device=DEV, cap=ml)
    starts = W.sentence_starts(cfg, steps=16)
    q = W.make_queries(cfg, starts, layer=layer).to(DEV)
    lens = [int(ctx[b]) + 1 + 3 * b for b in range(cfg.B)]
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dec = SFIDecoder(K, V, cfg.Hq, ml, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k, lam=cfg.lam,
                     norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau)
    dec.slow(q[0], seq, None, cfg.B)
    torch.cuda.synchronize()
    out = dec.out.cpu().numpy()
    sel = dec.sel_idx.cpu().numpy()
    cnt = dec.sel_count.cpu().numpy()
    b = 2
    n = lens[b]
    Kb, Vb = _bits(K[b, :, : n + 7]), _bits(V[b, :, : n + 7])
    qb = _bits(q[:, b])
    r = O.slow_select(qb[0], Kb, Vb, n, lam=cfg.lam, k=cfg.k, n_sink=cfg.n_sink, window=cfg.window,
                      norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau)
    assert row_rel_err(out[b], r["o"]) <= OUT_TOL
    ties = sum(check_selection(sel[b, g], cnt[b, g], r["s"][g], r["lo"], r["hi"], cfg.k)
               for g in range(cfg.Hkv))
    _say(f"  near-tie differences: {ties}")
    # fast step 7 tokens later over the GPU's own (just checked) selection
    seq7 = torch.tensor([x + 7 for x in lens], dtype=torch.int32, device=DEV)
    dec.fast(q[7], seq7, None, cfg.B)
    torch.cuda.synchronize()
    of = dec.out.cpu().numpy()
    lists = [sel[b, g, : cnt[b, g]] for g in range(cfg.Hkv)]
    o_ref = O.fast_step(qb[7], Kb, Vb, n + 7, lists, cfg.n_sink, cfg.window)
    assert row_rel_err(of[b], o_ref) <= OUT_TOL
    del dec, K, V
    _free()


def test_full_size_stack_pipeline_128k():
    """Two layers of the 128K stack (B=4, k=4096, lambda 0.2) through three
    steps (all slow, then the schedule's steps 1 and 2) with each layer's
    selection run inside the next layer's grids, as the benchmark times it,
    against sfi_decode_step_select per layer: outputs and index lists bit
    for bit; one slow sequence's selection against the oracle."""
    cfg = W.CONFIGS["stack32-128k"].replace(steps=3)
    _say("full size: 128K layer pipeline, 2 layers")
    ctx = W.context_lengths(cfg)
    ml = int(ctx.max()) + cfg.steps
    starts = W.sentence_starts(cfg)
    slow = np.zeros((cfg.steps, cfg.B), dtype=bool)
    slow[0] = True
    slow[1, 1] = slow[2, 2] = True
    plan = DecodePlan(slow, ctx, DEV)
    kw = dict(n_sink=cfg.n_sink, window=cfg.window, k=cfg.k, lam=cfg.lam, norm_coef=cfg.norm_coef,
              pos_tau=cfg.pos_tau)
    layers = []
    for layer in (3, 4):
        K, V = W.make_kv(cfg, layer=layer, device=DEV, cap=ml)
        q = W.make_queries(cfg, starts, layer=layer).to(DEV)
        layers.append((K, V, q, SFIDecoder(K, V, cfg.Hq, ml, **kw), SFIDecoder(K, V, cfg.Hq, ml, **kw)))
    pend = None
    for s in range(cfg.steps):
        for K, V, q, pipe, ref in layers:
            pend = pipe.layer_step(plan, s, q, pending=pend)
            ref.step_select(q[s], plan.seq_len[s], plan.slow_ids[s], int(plan.n_slow[s]), plan.fast_ids[s],
                            int(plan.n_fast[s]), len_hints=ref.hints(plan, s))
            torch.cuda.synchronize()
            assert torch.equal(pipe.out.view(torch.int32), ref.out.view(torch.int32)), s
    sfi.sfi_run_deferred(pend)
    torch.cuda.synchronize()
    for _, _, _, pipe, ref in layers:
        assert torch.equal(pipe.sel_idx, ref.sel_idx)
        assert torch.equal(pipe.sel_count, ref.sel_count)
    _say("  pipelined = per layer, bit for bit")
    K, V, q, pipe, _ = layers[1]
    b, s = 2, 2
    n = int(plan.seq_len_host[s, b])
    r = O.slow_select(_bits(q[s, b]), _bits(K[b, :, :n]), _bits(V[b, :, :n]), n, lam=cfg.lam, k=cfg.k,
                      n_sink=cfg.n_sink, window=cfg.window, norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau)
    sel, cnt = pipe.sel_idx.cpu().numpy(), pipe.sel_count.cpu().numpy()
    ties = sum(check_selection(sel[b, g], cnt[b, g], r["s"][g], r["lo"], r["hi"], cfg.k) for g in range(cfg.Hkv))
    _say(f"  near-tie differences: {ties}")
    del layers
    _free()


def test_full_size_vegas_64k_sampled():
    cfg = W.CONFIGS["vegas-64k"]
    T = cfg.vegas_T
    _say("full size: Vegas verification at 64K, B=16, T=8")
    ctx = int(W.context_lengths(cfg).max())
    K, V = W.make_kv(cfg, device=DEV, cap=ctx + 2 * T)
    qpos = W.make_vegas_queries(cfg.replace(steps=2)).to(DEV)
    vd = VegasDecoder(K, V, cfg.Hq, ctx + 2 * T, T, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k)
    n = ctx + T
    seq = torch.full((cfg.B,), n, dtype=torch.int32, device=DEV)
    q_rows = qpos[:T].permute(1, 0, 2, 3).contiguous()
    picks = (3, 11)
    Kb = {b: _bits(K[b, :, : n + 3]) for b in picks}
    Vb = {b: _bits(V[b, :, : n + 3]) for b in picks}
    for mode in ("all", "c2q"):
        rows = O.collect_rows(T, mode)
        vd.verify(q_rows, seq, sum(1 << t for t in rows))
        vd.select(seq)
        torch.cuda.synchronize()
        vout = vd.vout.cpu().numpy()
        agg = vd.agg.cpu().numpy()
        sel = vd.sel_idx.cpu().numpy()
        cnt = vd.sel_count.cpu().numpy()
        for b in picks:
            o_ref, a_ref = O.verify(_bits(q_rows[b]), Kb[b], Vb[b], n, rows)
            for t in range(T):
                assert row_rel_err(vout[b, t], o_ref[t]) <= OUT_TOL, (mode, b, t)
            P = n - T
            err = np.abs(agg[b, :P] - a_ref).max() / np.abs(a_ref).max()
            assert err <= 1e-5, (mode, b, err)
            lo, hi = O.candidate_range(n, cfg.n_sink, cfg.window)
            ties = check_selection(sel[b, 0], cnt[b, 0], a_ref, lo, hi, cfg.k)
            _say(f"  {mode} b={b}: near-tie differences {ties}")
    # a draft step over the head-shared list (the last selection, Collect-2-Query)
    seqd = torch.full((cfg.B,), n + 3, dtype=torch.int32, device=DEV)
    vd.draft(qpos[T + 2], seqd)
    torch.cuda.synchronize()
    od = vd.out.cpu().numpy()
    for b in picks:
        lst = [sel[b, 0, : cnt[b, 0]]] * cfg.Hkv
        o_ref = O.fast_step(_bits(qpos[T + 2, b]), Kb[b], Vb[b], n + 3, lst, cfg.n_sink, cfg.window)
        assert row_rel_err(od[b], o_ref) <= OUT_TOL
    del vd, K, V
    _free()


def test_full_size_ragged_paged_sampled():
    cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(steps=4)
    _say("full size: ragged paged batch, B=32, 8K-128K contexts")
    ctx = W.context_lengths(cfg)
    caps = ctx + cfg.growth()
    table, npages = W.page_table(cfg, caps)
    Kp, Vp = W.make_paged_kv(cfg, table, npages, caps, device=DEV)
    tab = torch.from_numpy(table).to(DEV)
    starts = W.sentence_starts(cfg)
    slow = np.zeros((cfg.steps, cfg.B), dtype=bool)
    slow[0] = True
    slow[1, ::5] = True            # step 1: every fifth sequence slow, the rest fast
    plan = DecodePlan(slow, ctx, DEV, k_cap=cfg.k, k_div=cfg.k_div)
    q = W.make_queries(cfg, starts).to(DEV)
    ml = int(ctx.max()) + cfg.steps
    dec = SFIDecoder(Kp, Vp, cfg.Hq, ml, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k, lam=cfg.lam,
                     norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau, page_table=tab,
                     page_size=cfg.page_size)
    _say(f"  generated {npages} pages")
    dec.step(plan, 0, q)
    torch.cuda.synchronize()
    _say("  step 0 (all slow) done")
    out0 = dec.out.cpu().numpy()
    sel0 = dec.sel_idx.cpu().numpy()
    cnt0 = dec.sel_count.cpu().numpy()
    dec.step(plan, 1, q)           # co-launched: slow 0, 5, 10, ...; fast the others
    torch.cuda.synchronize()
    _say("  step 1 (co-launched) done")
    out1 = dec.out.cpu().numpy()
    order = np.argsort(ctx)
    picks = [int(order[0]), int(order[-1]), 10]   # shortest, longest, a slow one at step 1
    for b in picks:
        n0 = int(plan.seq_len_host[0, b])
        n1 = int(plan.seq_len_host[1, b])
        kb = min(cfg.k, n0 // cfg.k_div)
        Kb = _bits(W.gather_paged(Kp, table, b, n1))
        Vb = _bits(W.gather_paged(Vp, table, b, n1))
        qb = _bits(q[:, b])
        r = O.slow_select(qb[0], Kb, Vb, n0, lam=cfg.lam, k=kb, n_sink=cfg.n_sink, window=cfg.window,
                          norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau)
        assert row_rel_err(out0[b], r["o"]) <= OUT_TOL, b
        ties = sum(check_selection(sel0[b, g, :kb], cnt0[b, g], r["s"][g], r["lo"], r["hi"], kb)
                   for g in range(cfg.Hkv))
        assert np.all(sel0[b, :, kb:] == -1)
        _say(f"  b={b} n={n0} k={kb}: near-tie differences {ties}")
        if slow[1, b]:
            o_ref, _ = O.dense_step(qb[1], Kb, Vb, n1)
        else:
            lists = [sel0[b, g, : cnt0[b, g]] for g in range(cfg.Hkv)]
            o_ref = O.fast_step(qb[1], Kb, Vb, n1, lists, cfg.n_sink, cfg.window)
        assert row_rel_err(out1[b], o_ref) <= OUT_TOL, b
    del dec, Kp, Vp
    _free()
