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
