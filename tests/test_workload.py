"""The seeded input generator: determinism, shapes and the planted structure."""
import numpy as np
import torch

from dynamic_sparse_kv_amd import workload as W


def _tiny():
    return W.CONFIGS["tiny-4k"].replace(ctx=300, steps=20, hh_count=5)


def test_same_seed_same_bytes():
    cfg = _tiny()
    K1, V1 = W.make_kv(cfg)
    K2, V2 = W.make_kv(cfg)
    assert torch.equal(K1.view(torch.int16), K2.view(torch.int16))
    assert torch.equal(V1.view(torch.int16), V2.view(torch.int16))
    st = W.sentence_starts(cfg)
    np.testing.assert_array_equal(st, W.sentence_starts(cfg))
    q1 = W.make_queries(cfg, st)
    q2 = W.make_queries(cfg, st)
    assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))


def test_layers_and_configs_differ():
    cfg = _tiny()
    K0, _ = W.make_kv(cfg, layer=0)
    K1, _ = W.make_kv(cfg, layer=1)
    assert not torch.equal(K0, K1)


def test_shapes_and_heavy_hitters():
    cfg = _tiny()
    K, V = W.make_kv(cfg)
    rows = cfg.ctx + cfg.steps
    cap = W.padded_capacity(rows)
    assert cap >= rows and cap % 64 == 32
    assert K.shape == (1, 2, cap, 64) and K.dtype == torch.bfloat16
    # the padding rows are zero; the drawn rows do not depend on the padding
    assert not K[:, :, rows:].any() and not V[:, :, rows:].any()
    K2, _ = W.make_kv(cfg, cap=rows)
    assert torch.equal(K[:, :, :rows].view(torch.int16), K2.view(torch.int16))
    K = K[:, :, :rows]
    cap = rows
    hh = W.heavy_hitter_positions(cfg, 0, 0, cfg.ctx)
    assert hh.shape == (2, 5) and hh.max() < cfg.ctx
    norms = K.float().norm(dim=-1)[0]
    for h in range(2):
        mask = np.zeros(cap, dtype=bool)
        mask[hh[h]] = True
        # planted rows have ~3x the norm of ordinary rows
        assert norms[h, mask].min() > 2.0 * norms[h, ~mask].median()


def test_queries_ar1_structure():
    cfg = _tiny().replace(steps=200)
    st = W.sentence_starts(cfg)
    q = W.make_queries(cfg, st).float()[:, 0].reshape(200, -1)
    cos = torch.nn.functional.cosine_similarity(q[1:], q[:-1], dim=-1).numpy()
    within = cos[~st[1:, 0]]
    across = cos[st[1:, 0]]
    assert within.mean() > 0.9 and abs(across.mean()) < 0.2


def test_ragged_and_pages():
    cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(B=6, Hkv=2, Hq=4, d=64, ctx=4096, ragged_min=256, steps=3)
    ctxs = W.context_lengths(cfg)
    assert ctxs.min() >= 256 and ctxs.max() <= 4096
    table, total = W.page_table(cfg, ctxs + cfg.growth())
    used = table[table >= 0]
    assert len(np.unique(used)) == len(used) == total
    K, _ = W.make_kv(cfg)
    pool = W.to_paged(K, table, total, cfg.page_size)
    b, pos = 3, int(ctxs[3]) - 1
    pg = table[b, pos // 16]
    assert torch.equal(pool[pg, :, pos % 16], K[b, :, pos])


def test_take_decode_rows_contiguous_and_paged():
    """The rows a run appends are moved out of the cache bit for bit: the
    returned [steps][B][T][Hkv][d] rows equal the cache rows ctx + s*T + t,
    which are then zero; the prefill is untouched (contiguous and paged)."""
    cfg = W.CONFIGS["tiny-4k"].replace(B=2, steps=5, ctx=300)
    K, V = W.make_kv(cfg)
    K0, V0 = K.clone(), V.clone()
    ctx = W.context_lengths(cfg)
    Kn, Vn = W.take_decode_rows(K, V, ctx, 2, rows_per_step=2)
    assert Kn.shape == (2, 2, 2, cfg.Hkv, cfg.d)
    for s in range(2):
        for b in range(2):
            for t in range(2):
                j = int(ctx[b]) + 2 * s + t
                assert torch.equal(Kn[s, b, t], K0[b, :, j]) and torch.equal(Vn[s, b, t], V0[b, :, j])
                assert torch.all(K[b, :, j] == 0) and torch.all(V[b, :, j] == 0)
    assert torch.equal(K[:, :, :300], K0[:, :, :300])
    cfgp = W.CONFIGS["ragged-paged-8k-128k"].replace(B=3, steps=4, ctx=9000, ragged_min=1000, Hq=8, Hkv=2)
    ctx = W.context_lengths(cfgp)
    caps = ctx + cfgp.growth()
    table, npg = W.page_table(cfgp, caps)
    Kp, Vp = W.make_paged_kv(cfgp, table, npg, caps)
    Kp0 = Kp.clone()
    Kn, Vn = W.take_decode_rows(Kp, Vp, ctx, 4, table=table)
    for b in range(3):
        full = W.gather_paged(Kp0, table, b, int(ctx[b]) + 4)
        after = W.gather_paged(Kp, table, b, int(ctx[b]) + 4)
        for s in range(4):
            assert torch.equal(Kn[s, b, 0], full[:, int(ctx[b]) + s])
        assert torch.all(after[:, int(ctx[b]):] == 0)
        assert torch.equal(after[:, :int(ctx[b])], full[:, :int(ctx[b])])
