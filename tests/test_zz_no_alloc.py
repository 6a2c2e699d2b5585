"""sfi_fast_step_noalloc (partials in the library's own device array, no
workspace) against sfi_fast_step on the same inputs, through the C ABI: two
calls in a row, the second on a smaller batch, so stale contents of the
shared array from the first call must not leak into the second."""
import sys

import numpy as np
import pytest
import torch

from dynamic_sparse_kv_amd import sfi

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(B, Hq, Hkv, d, lens, k, seed, n_sink=4, window=256):
    g = torch.Generator(device=DEV).manual_seed(seed)
    cap = max(lens) + 3
    K = torch.randn((B, Hkv, cap, d), generator=g, device=DEV).to(torch.bfloat16).contiguous()
    V = torch.randn((B, Hkv, cap, d), generator=g, device=DEV).to(torch.bfloat16).contiguous()
    q = torch.randn((B, Hq, d), generator=g, device=DEV).to(torch.bfloat16).contiguous()
    rng = np.random.default_rng(seed)
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        hi = max(n_sink, lens[b] - window)
        for h in range(Hkv):
            m = min(k, hi - n_sink)
            if m > 0:
                sel[b, h, :m] = np.sort(rng.choice(np.arange(n_sink, hi), size=m, replace=False))
                cnt[b, h] = m
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kv = sfi.make_kv(K, V, seq, Hq, max(lens))
    return kv, q, torch.from_numpy(sel).to(DEV), torch.from_numpy(cnt).to(DEV), (K, V, seq)


def _both(kv, q, sel, cnt, Hkv, k, batch_ids, batch_n, n_sink=4, window=256):
    B, Hq, d = q.shape
    ref = torch.full((B, Hq, d), 3.0, device=DEV)
    got = torch.full((B, Hq, d), 3.0, device=DEV)
    wsb = sfi.sfi_fast_workspace_bytes(kv, k, n_sink, window)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    sfi.sfi_fast_step(kv, batch_ids, batch_n, q, sel, cnt, Hkv, k, n_sink, window, ref, ws, wsb)
    sfi.sfi_fast_step_noalloc(kv, batch_ids, batch_n, q, sel, cnt, Hkv, k, n_sink, window, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_fast_step_equals_workspace_call_twice():
    # first call: 8 sequences of the 4:1 GQA shape, 2048 selected per kv head
    _say("no-alloc fast step, call 1: B=8 Hq=32 Hkv=8 d=128 k=2048")
    kv, q, sel, cnt, keep1 = _case(8, 32, 8, 128, [5000, 4100, 2600, 6000, 3000, 4500, 5200, 2400], 2048, 7)
    ref, got = _both(kv, q, sel, cnt, 8, 2048, None, 8)
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))
    assert torch.isfinite(got).all()
    # second call: a smaller batch subset of another shape (stale partials
    # of call 1 remain in the array); slots outside the subset stay untouched
    _say("no-alloc fast step, call 2: B=3 (2 listed) Hq=8 Hkv=2 d=64 k=256")
    kv2, q2, sel2, cnt2, keep2 = _case(3, 8, 2, 64, [1500, 300, 900], 256, 8)
    ids = torch.tensor([2, 0], dtype=torch.int32, device=DEV)
    ref2, got2 = _both(kv2, q2, sel2, cnt2, 2, 256, ids, 2)
    assert torch.equal(ref2.view(torch.int32), got2.view(torch.int32))
    assert torch.all(got2[1] == 3.0)
    assert not torch.all(got2[0] == 3.0) and not torch.all(got2[2] == 3.0)


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    """A call whose partials exceed the array is refused before launch."""
    _say("no-alloc fast step, oversize batch")
    B, Hq, Hkv, d = 1024, 64, 64, 128       # one split per pair: 65536 rows x 130 floats > 16 MiB
    K = torch.zeros((B, Hkv, 1, d), dtype=torch.bfloat16, device=DEV)
    seq = torch.ones(B, dtype=torch.int32, device=DEV)
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((B, Hq, d), device=DEV)
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device=DEV)
    kv = sfi.make_kv(K, K, seq, Hq, 1)
    with pytest.raises(sfi.SfiError) as e:
        sfi.sfi_fast_step_noalloc(kv, None, B, q, None, cnt, Hkv, 0, 4, 256, out)
    assert e.value.status == sfi.SFI_ERR_WORKSPACE
