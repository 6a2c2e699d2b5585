"""Host logic of the decode-loop driver that needs no GPU."""
import pytest
import torch

from dynamic_sparse_kv_amd import runner


@pytest.mark.parametrize("method", ["run_two_streams", "run_pipelined"])
def test_multi_stream_schedules_refuse_graph_capture(monkeypatch, method):
    """A multi-stream schedule called while a capture is active raises before
    it records, waits on or launches anything."""
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    dec = runner.SFIDecoder.__new__(runner.SFIDecoder)   # no device buffers needed
    args = (None, None, 0, 1, None, None) if method == "run_two_streams" else \
        (None, None, 0, 1, None, None, None, None)
    with pytest.raises(RuntimeError, match="cannot be captured"):
        getattr(dec, method)(*args)


def test_decode_plan_splits_slow_and_fast_ids():
    """DecodePlan lists each step's slow and fast sequences (disjoint, in
    ascending order) and the lengths ctx + s + 1."""
    import numpy as np
    slow = np.array([[1, 1, 1], [0, 1, 0], [0, 0, 0]], dtype=bool)
    ctx = np.array([10, 20, 30])
    plan = runner.DecodePlan(slow, ctx, "cpu")
    assert list(plan.n_slow) == [3, 1, 0] and list(plan.n_fast) == [0, 2, 3]
    assert plan.slow_ids[1, :1].tolist() == [1]
    assert plan.fast_ids[1, :2].tolist() == [0, 2]
    assert plan.seq_len[2].tolist() == [13, 23, 33]
    # fast sequences refreshed on the step before are listed apart
    assert plan.fast_new_ids[1, :2].tolist() == [0, 2] and plan.n_fast_old[1] == 0
    assert plan.n_fast_new[2] == 1 and plan.fast_new_ids[2, :1].tolist() == [1]


@pytest.mark.parametrize("k_div", [0, 16])
def test_len_hints_bound_every_fast_list(k_div):
    """DecodePlan.len_hints: slow hints are the slow sequences' lengths in
    list order; each fast hint is at least the length of that sequence's
    fast row list (sinks and window within n, plus the selection its last
    slow step made: at most k, or min(k, n_then // k_div), and at most the
    middle keys [n_sink, n_then - window) of that step) and within the
    range the library accepts; the pipelined schedule's two fast halves
    hold the same values as the fast list, split by the plan's fast ids."""
    import numpy as np
    rng = np.random.default_rng(5 + k_div)
    B, steps, n_sink, window, k = 7, 20, 4, 64, 300
    ctx = rng.integers(1, 9000, size=B)
    ctx[0] = 1
    slow = rng.random((steps, B)) < 0.3
    slow[0] = True
    plan = runner.DecodePlan(slow, ctx, "cpu", k_cap=k if k_div else 0, k_div=k_div)
    last_n = np.zeros(B, dtype=np.int64)
    for s in range(steps):
        h = plan.len_hints(s, n_sink, window, k)
        assert h is plan.len_hints(s, n_sink, window, k)          # cached
        lens = plan.seq_len_host[s].astype(np.int64)
        sl, fl = np.nonzero(slow[s])[0], np.nonzero(~slow[s])[0]
        assert h[0].dtype == np.int32 and h[0].tolist() == lens[sl].tolist()
        assert h[1].dtype == np.int32 and len(h[1]) == len(fl)
        for z, b in enumerate(fl):
            n, nt = int(lens[b]), int(last_n[b])
            cap = min(k, nt // k_div) if k_div else k
            cnt = min(cap, max(nt - n_sink - window, 0))
            ns = min(n_sink, n)
            L = ns + min(window, n - ns) + cnt
            assert L <= h[1][z] <= n_sink + window + k, (s, b)
        old = plan.fast_old_ids_host[s, : plan.n_fast_old[s]]
        new = plan.fast_new_ids_host[s, : plan.n_fast_new[s]]
        by_b = dict(zip(fl.tolist(), h[1].tolist()))
        assert h.fast_old.tolist() == [by_b[b] for b in old]
        assert h.fast_new.tolist() == [by_b[b] for b in new]
        last_n[sl] = lens[sl]
