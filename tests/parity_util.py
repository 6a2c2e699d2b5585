"""Helpers shared by the GPU parity tests: error measures and selection checks.

Tolerances:
  * attention outputs: per output row (sequence, head[, verify row]),
    max|x - y| / max|y| <= 2e-3 (bf16 inputs, fp32 accumulation);
  * evidence f and fused score s: per row max|x - y| / max|y| <= 1e-4 (fp32
    logits carry ~1e-6 relative error; exp and the normaliser add a few ulp);
  * key norms: relative 1e-5;
  * selections: identical index sets except for keys whose oracle score lies
    within 1e-5 relative of the oracle's k-th score (the near-tie band); the
    number of such keys is returned so tests can report it.
"""
import numpy as np

from oracle import sfi_oracle as O

OUT_TOL = 2e-3
EVID_TOL = 1e-4
NORM_TOL = 1e-5
TIE_BAND = 1e-5


def row_rel_err(x, y):
    """max over rows of max|x - y| / max|y| (last axis = row)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    num = np.abs(x - y).max(axis=-1)
    den = np.maximum(np.abs(y).max(axis=-1), 1e-30)
    return float((num / den).max())


def check_selection(gpu_idx, gpu_cnt, score, lo, hi, k, ambiguous=None):
    """Compare one GPU index list with the oracle's Top-K of ``score``.

    Returns the number of near-tie keys that differ.  Asserts that the GPU
    list is ascending, unique, inside [lo, hi), padded with -1, of the right
    length, and that every difference lies in the near-tie band or is marked
    in the boolean mask ``ambiguous`` (keys whose refined score hangs on an
    earlier near-tie decision).
    """
    gpu_idx = np.asarray(gpu_idx)
    want = O.topk_indices(score, lo, hi, k)
    assert int(gpu_cnt) == len(want), (int(gpu_cnt), len(want))
    got = gpu_idx[: int(gpu_cnt)]
    assert np.all(gpu_idx[int(gpu_cnt):] == -1)
    if len(got):
        assert np.all(np.diff(got) > 0), "not ascending / not unique"
        assert got.min() >= lo and got.max() < hi
    diff = np.setxor1d(got, want)
    if diff.size == 0:
        return 0
    kth = O.kth_score(score, lo, hi, k)
    assert kth is not None
    band = np.abs(np.asarray(score)[diff] - kth) <= TIE_BAND * abs(kth)
    if ambiguous is not None:
        band |= np.asarray(ambiguous)[diff]
    assert band.all(), f"selection differs outside the near-tie band: {diff[~band][:10]}"
    return int(diff.size)


def nms_ambiguous(score, lo, hi, radius):
    """Keys of [lo, hi) whose Soft-NMS count depends on a near-tie: some
    candidate within ``radius`` lies within the near-tie band of it (the
    kernel compares float32 scores formed in another rounding order)."""
    s = np.asarray(score, dtype=np.float64)
    amb = np.zeros(len(s), dtype=bool)
    for dd in range(1, radius + 1):
        if hi - dd <= lo:
            break
        a, b = s[lo:hi - dd], s[lo + dd:hi]
        close = np.abs(a - b) <= TIE_BAND * np.maximum(np.abs(a), np.abs(b))
        amb[lo:hi - dd] |= close
        amb[lo + dd:hi] |= close
    return amb


def tie_band_keys(score, lo, hi, k):
    """Keys of [lo, hi) within the near-tie band of the k-th score."""
    s = np.asarray(score, dtype=np.float64)
    amb = np.zeros(len(s), dtype=bool)
    kth = O.kth_score(s, lo, hi, k)
    if kth is not None:
        amb[lo:hi] = np.abs(s[lo:hi] - kth) <= TIE_BAND * abs(kth)
    return amb
