"""Pins of the CPU oracle to facts fixed outside it.

Each test checks the oracle against something other than its own formula: a
library routine (PyTorch SDPA, SciPy), a closed form, a hand-worked fixture
under tests/golden/, brute-force enumeration, or an invariant of the
definition.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sfi_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rand_bits(rng, shape, scale=1.0):
    return _bf16(rng.standard_normal(shape) * scale)


# --------------------------------------------------------------------- inputs

def test_bf16_decoding_matches_definition():
    for hexbits, val in _gold("bf16_bits.json")["cases"]:
        got = O.bf16_to_f64(np.array([int(hexbits, 16)], dtype=np.uint16))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hexbits


def test_bf16_decoding_matches_torch():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                     # drop inf / nan
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.bf16_to_f64(bits), ref)


# ------------------------------------------------------------ O1 dense step

@pytest.mark.parametrize("Hq,Hkv,d,n", [(8, 2, 16, 37), (4, 4, 64, 5), (6, 1, 8, 50)])
def test_dense_matches_torch_sdpa(Hq, Hkv, d, n):
    rng = np.random.default_rng(Hq * 100 + n)
    q = _rand_bits(rng, (Hq, d))
    K = _rand_bits(rng, (Hkv, n + 3, d), 2.0)
    V = _rand_bits(rng, (Hkv, n + 3, d))
    o, p = O.dense_step(q, K, V, n)
    tq = torch.from_numpy(O.bf16_to_f64(q)).view(1, Hq, 1, d)
    tk = torch.from_numpy(O.bf16_to_f64(K[:, :n])).view(1, Hkv, n, d)
    tv = torch.from_numpy(O.bf16_to_f64(V[:, :n])).view(1, Hkv, n, d)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)
    np.testing.assert_allclose(o, ref.view(Hq, d).numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-13)


def test_dense_equal_keys_gives_mean_value():
    rng = np.random.default_rng(1)
    Hq, Hkv, d, n = 4, 2, 8, 11
    row = _rand_bits(rng, (d,))
    K = np.broadcast_to(row, (Hkv, n, d)).copy()
    V = _rand_bits(rng, (Hkv, n, d))
    o, p = O.dense_step(_rand_bits(rng, (Hq, d)), K, V, n)
    for h in range(Hq):
        np.testing.assert_allclose(o[h], O.bf16_to_f64(V[h // 2]).mean(axis=0), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(p[h], 1.0 / n, rtol=1e-12)


def test_dense_key_permutation_invariance():
    rng = np.random.default_rng(2)
    Hq, Hkv, d, n = 4, 2, 16, 23
    q = _rand_bits(rng, (Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    perm = rng.permutation(n)
    o1, _ = O.dense_step(q, K, V, n)
    o2, _ = O.dense_step(q, K[:, perm], V[:, perm], n)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------- O2 evidence

def test_evidence_is_group_mean_and_sums_to_one():
    rng = np.random.default_rng(3)
    Hq, Hkv, d, n = 8, 2, 16, 40
    _, p = O.dense_step(_rand_bits(rng, (Hq, d)), _rand_bits(rng, (Hkv, n, d)), _rand_bits(rng, (Hkv, n, d)), n)
    f = O.evidence(p, Hkv)
    np.testing.assert_allclose(f.sum(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(f[1], (p[4] + p[5] + p[6] + p[7]) / 4, rtol=1e-13)
    np.testing.assert_array_equal(O.evidence(p, Hq), p)          # G = 1 (MHA)


# -------------------------------------------------------------- O3 prior

def test_prior_two_keys_closed_form():
    # Two keys: population z-scores are exactly -1 and +1; t = 1.
    K = np.zeros((1, 2, 4))
    K[0, 0, 0] = 1.0
    K[0, 1, 0] = 3.0
    r = O.prior(K, 2, norm_coef=0.5, pos_tau=1024.0)
    want = math.e * (1.0 + math.exp(-1.0 / 1024.0)) / 2.0
    assert r[0, 0] / r[0, 1] == pytest.approx(want, rel=1e-14)
    assert r.sum() == pytest.approx(1.0, rel=1e-15)


def test_prior_standardisation_is_population_zscore():
    from scipy.stats import zscore
    rng = np.random.default_rng(4)
    K = rng.standard_normal((2, 30, 8))
    n = 30
    # pos_tau -> 0: the position factor is 1 for every j < t, so log-ratios expose z.
    r = O.prior(K, n, norm_coef=0.5, pos_tau=1e-9)
    nu = np.sqrt((K ** 2).sum(-1))
    z = zscore(nu, axis=1, ddof=0)
    for g in range(2):
        lr = np.log(r[g, : n - 1]) - np.log(r[g, 0])
        np.testing.assert_allclose(lr, -0.5 * (z[g, : n - 1] - z[g, 0]), rtol=1e-10, atol=1e-12)


def test_prior_monotone_and_degenerate():
    n = 64
    K = np.ones((1, n, 8))                            # all norms equal: std 0 -> z 0
    r = O.prior(K, n)
    assert np.all(np.diff(r[0]) > 0)                  # more recent -> larger at equal norm
    np.testing.assert_allclose(r.sum(), 1.0, rtol=1e-14)
    rng = np.random.default_rng(5)
    K = rng.standard_normal((1, n, 8))
    r = O.prior(K, n, pos_tau=1e-9)                   # drop the position factor
    nu = np.sqrt((K[0] ** 2).sum(-1))
    o = np.argsort(nu[: n - 1])
    assert np.all(np.diff(r[0, : n - 1][o]) < 0)       # larger norm -> smaller prior


# ------------------------------------------------------------- O4 fusion

def _kl(a, b):
    m = a > 0
    return float(np.sum(a[m] * np.log(a[m] / b[m])))


@pytest.mark.parametrize("lam", [0.0, 0.2, 0.3, 0.7, 1.0])
@pytest.mark.parametrize("n", [3, 5, 8])
def test_fusion_closed_form_is_the_minimiser(lam, n):
    from scipy.optimize import minimize
    rng = np.random.default_rng(int(lam * 10) + 100 * n)
    f = rng.dirichlet(np.ones(n))
    r = rng.dirichlet(np.ones(n))

    def obj(x):
        s = np.exp(x - x.max())
        s /= s.sum()
        return (1 - lam) * _kl(f, s) + lam * _kl(r, s)

    best = None
    for start in (np.zeros(n), rng.standard_normal(n)):
        res = minimize(obj, start, method="BFGS", options={"gtol": 1e-12, "maxiter": 10000})
        if best is None or res.fun < best.fun:
            best = res
    s_num = np.exp(best.x - best.x.max())
    s_num /= s_num.sum()
    s = O.fuse(f, r, lam)
    np.testing.assert_allclose(s, s_num, atol=2e-6)
    assert obj(np.log(s)) <= best.fun + 1e-12
    assert s.sum() == pytest.approx(1.0, rel=1e-14)


def test_fusion_endpoints():
    rng = np.random.default_rng(6)
    f = rng.dirichlet(np.ones(9))
    r = rng.dirichlet(np.ones(9))
    np.testing.assert_array_equal(O.fuse(f, r, 0.0), f)
    np.testing.assert_array_equal(O.fuse(f, r, 1.0), r)


# -------------------------------------------------------------- O5 top-k

def _brute_best_subset(score, cand, k):
    """argmax_{|T|=k} sum(score[T]); equal sums -> lexicographically smallest tuple."""
    best, best_sum = (), -math.inf
    for T in itertools.combinations(sorted(cand), k):
        sm = sum(score[i] for i in T)
        if sm > best_sum or (sm == best_sum and T < best):
            best, best_sum = T, sm
    return list(best)


def test_topk_hand_cases():
    for c in _gold("topk_hand.json")["cases"]:
        got = O.topk_indices(np.array(c["score"], dtype=float), c["lo"], c["hi"], c["k"])
        assert got.tolist() == c["expect"], c["note"]


@pytest.mark.parametrize("seed", range(40))
def test_topk_equals_subset_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 15))
    # small integer scores: exact sums and plenty of exact ties
    score = rng.integers(-3, 4, size=n).astype(float)
    lo = int(rng.integers(0, 3))
    hi = int(rng.integers(lo, n + 1))
    k = int(rng.integers(1, 7))
    cand = list(range(lo, hi))
    want = _brute_best_subset(score, cand, min(k, len(cand)))
    assert O.topk_indices(score, lo, hi, k).tolist() == want


def test_vegas_selection_equals_argmax_sum_over_subsets():
    # Section 2.A of the Vegas page: T maximises the logits summed over rows,
    # heads and members.  Tiny case, enumerated directly over that triple sum.
    rng = np.random.default_rng(7)
    T, Hq, Hkv, d, n, k, ns, W = 3, 4, 2, 8, 14, 3, 1, 4
    q = _rand_bits(rng, (T, Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    _, agg = O.verify(q, K, V, n, rows=[0, 1, 2])
    qf, Kf = O.bf16_to_f64(q), O.bf16_to_f64(K)
    lo, hi = ns, n - W
    best, best_sum = None, -math.inf
    for S in itertools.combinations(range(lo, hi), k):
        tot = sum(qf[t, h] @ Kf[h // 2, i] / math.sqrt(d) for t in range(T) for h in range(Hq) for i in S)
        if tot > best_sum:
            best, best_sum = list(S), tot
    assert O.vegas_select(agg, n, k, ns, W).tolist() == best


# ------------------------------------------------------------ O6 fast step

def test_fast_with_full_selection_equals_dense():
    rng = np.random.default_rng(8)
    Hq, Hkv, d, n, ns, W = 8, 2, 16, 300, 4, 32
    q = _rand_bits(rng, (Hq, d))
    K = _rand_bits(rng, (Hkv, n, d), 2.0)
    V = _rand_bits(rng, (Hkv, n, d))
    full = [list(range(ns, n - W))] * Hkv
    o_fast = O.fast_step(q, K, V, n, full, ns, W)
    o_dense, _ = O.dense_step(q, K, V, n)
    np.testing.assert_allclose(o_fast, o_dense, rtol=1e-12, atol=1e-14)
    # a window covering the whole cache is dense attention as well
    np.testing.assert_allclose(O.fast_step(q, K, V, n, [[]] * Hkv, ns, n), o_dense, rtol=1e-12, atol=1e-14)


def test_fast_set_composition():
    A = O.fast_key_set(100, [1, 2, 5, 50, 80, 99, -1, 200], n_sink=4, window=30)
    # sinks 0..3, window 70..99, selected 5 and 50 (1, 2 are sinks; 80, 99 in window)
    assert A.tolist() == [0, 1, 2, 3, 5, 50] + list(range(70, 100))
    assert O.fast_key_set(3, [0, 1], 4, 256).tolist() == [0, 1, 2]


def test_fast_equals_dense_over_the_attended_subset():
    # attention restricted to A equals dense attention over a cache holding only A
    rng = np.random.default_rng(9)
    Hq, Hkv, d, n, ns, W = 4, 1, 16, 120, 2, 10
    q = _rand_bits(rng, (Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    sel = [sorted(rng.choice(np.arange(ns, n - W), 17, replace=False).tolist())]
    A = O.fast_key_set(n, sel[0], ns, W)
    o_sub, _ = O.dense_step(q, K[:, A], V[:, A], len(A))
    np.testing.assert_allclose(O.fast_step(q, K, V, n, sel, ns, W), o_sub, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------- O7 schedule

def test_schedule_hand_cases():
    for c in _gold("schedule_hand.json")["cases"]:
        starts = np.zeros((c["steps"], 1), dtype=bool)
        starts[c["starts"], 0] = True
        got = O.schedule(starts, c["budget"])[:, 0].astype(int).tolist()
        assert got == c["slow"], c["note"]


@pytest.mark.parametrize("mu,budget,want", [(20.0, 16, None), (24.0, 32, None)])
def test_schedule_slow_fraction_closed_form(mu, budget, want):
    # Geometric sentence lengths make starts a Bernoulli(p = 1/mu) process; the
    # fast-run length is then a Markov chain with stationary slow fraction
    # p / (1 - (1 - p)^(budget + 1)).
    from dynamic_sparse_kv_amd.workload import SFIConfig, sentence_starts
    cfg = SFIConfig("t", 99, B=64, Hq=1, Hkv=1, d=64, ctx=1, steps=4000,
                    mean_sentence=mu, budget=budget)
    st = sentence_starts(cfg)
    frac = O.schedule(st, budget)[1:].mean()
    p = 1.0 / mu
    closed = p / (1.0 - (1.0 - p) ** (budget + 1))
    assert frac == pytest.approx(closed, abs=0.004)


# ------------------------------------------------------------- O8 verify

def test_verify_rows_are_causal_dense_steps():
    rng = np.random.default_rng(10)
    T, Hq, Hkv, d, n = 4, 8, 2, 16, 60
    q = _rand_bits(rng, (T, Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    o, agg = O.verify(q, K, V, n, rows=range(T))
    for t in range(T):
        o_t, _ = O.dense_step(q[t], K, V, n - T + t + 1)
        np.testing.assert_allclose(o[t], o_t, rtol=1e-12, atol=1e-14)
    assert agg.shape == (n - T,)


def test_verify_aggregate_linearity():
    # sum over rows and heads of q.k/sqrt(d) = (sum of the group's queries) . k / sqrt(d)
    rng = np.random.default_rng(11)
    T, Hq, Hkv, d, n = 8, 8, 2, 32, 90
    q = _rand_bits(rng, (T, Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    qf, Kf = O.bf16_to_f64(q), O.bf16_to_f64(K)
    for mode in ("all", "c2q"):
        rows = O.collect_rows(T, mode)
        _, agg = O.verify(q, K, V, n, rows=rows)
        qs = qf[rows].sum(axis=0).reshape(Hkv, Hq // Hkv, d).sum(axis=1)
        want = sum(Kf[g, : n - T] @ qs[g] for g in range(Hkv)) / math.sqrt(d)
        np.testing.assert_allclose(agg, want, rtol=1e-10, atol=1e-10)


def test_collect_two_query_special_cases():
    assert O.collect_rows(8, "c2q") == [0, 7]
    assert O.collect_rows(2, "c2q") == O.collect_rows(2, "all")
    assert O.collect_rows(1, "c2q") == [0]
    rng = np.random.default_rng(12)
    Hq, Hkv, d, n = 4, 2, 16, 30
    q = _rand_bits(rng, (1, Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    _, agg = O.verify(q, K, V, n, rows=[0])
    l = O.attention_logits(q[0], K, n)
    np.testing.assert_allclose(agg, l[:, : n - 1].sum(axis=0), rtol=1e-12)


# ------------------------------------------------------- whole slow step

def test_slow_select_invariants():
    rng = np.random.default_rng(13)
    Hq, Hkv, d, n, k, ns, W = 8, 2, 32, 700, 50, 4, 256
    q = _rand_bits(rng, (Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    r = O.slow_select(q, K, V, n, lam=0.3, k=k, n_sink=ns, window=W)
    for name in ("f", "r", "s"):
        np.testing.assert_allclose(r[name].sum(axis=1), 1.0, rtol=1e-12)
    for g in range(Hkv):
        sel = r["sel"][g]
        assert len(sel) == k and np.all(np.diff(sel) > 0)
        assert sel.min() >= ns and sel.max() < n - W
        # every selected score is >= every unselected candidate score
        cand = np.arange(ns, n - W)
        rest = np.setdiff1d(cand, sel)
        assert r["s"][g, sel].min() >= r["s"][g, rest].max()
    # lam = 1: selection no longer depends on the query
    a = O.slow_select(q, K, V, n, lam=1.0, k=k, n_sink=ns, window=W)["sel"]
    b = O.slow_select(_rand_bits(rng, (Hq, d)), K, V, n, lam=1.0, k=k, n_sink=ns, window=W)["sel"]
    for g in range(Hkv):
        np.testing.assert_array_equal(a[g], b[g])
    # context too short for any candidate
    e = O.slow_select(q, K, V, 200, lam=0.3, k=k, n_sink=ns, window=W)
    assert all(len(s) == 0 for s in e["sel"])


# ------------------------------------------------- observation-window evidence

def test_window_evidence_one_query_is_the_slow_step_evidence():
    """w = 1 reduces to the slow step: o = dense output, f = O2's evidence."""
    rng = np.random.default_rng(21)
    Hq, Hkv, d, n = 8, 2, 16, 70
    q = _rand_bits(rng, (1, Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    o, f = O.window_evidence(q, K, V, n)
    o1, p1 = O.dense_step(q[0], K, V, n)
    np.testing.assert_allclose(o[0], o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f, O.evidence(p1, Hkv), rtol=1e-12, atol=1e-15)


def test_window_evidence_is_the_mean_of_causal_slow_steps():
    """f = mean over window rows of each row's own slow-step evidence at its
    cache length n - w + t + 1, zero beyond it; rows are causal dense steps;
    f sums to 1 per kv head."""
    rng = np.random.default_rng(22)
    w, Hq, Hkv, d, n = 5, 12, 3, 16, 45
    q = _rand_bits(rng, (w, Hq, d))
    K = _rand_bits(rng, (Hkv, n, d))
    V = _rand_bits(rng, (Hkv, n, d))
    o, f = O.window_evidence(q, K, V, n)
    want = np.zeros((Hkv, n))
    for t in range(w):
        nt = n - w + t + 1
        o_t, p_t = O.dense_step(q[t], K, V, nt)
        np.testing.assert_allclose(o[t], o_t, rtol=1e-12, atol=1e-14)
        want[:, :nt] += O.evidence(p_t, Hkv)
    np.testing.assert_allclose(f, want / w, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f.sum(axis=1), 1.0, rtol=1e-12)
    # the newest keys are seen by fewer rows: key n-1 only by the last row
    _, p_last = O.dense_step(q[w - 1], K, V, n)
    np.testing.assert_allclose(f[:, n - 1], O.evidence(p_last, Hkv)[:, n - 1] / w, rtol=1e-12)


def test_window_evidence_equal_keys_closed_form():
    """All keys equal: every visible key gets probability 1/n_t in row t, so
    f_j = (1/w) sum over rows that see j of 1/(n - w + t + 1)."""
    rng = np.random.default_rng(23)
    w, Hq, Hkv, d, n = 4, 4, 2, 8, 20
    q = _rand_bits(rng, (w, Hq, d))
    row = _rand_bits(rng, (d,))
    K = np.broadcast_to(row, (Hkv, n, d)).copy()
    V = _rand_bits(rng, (Hkv, n, d))
    _, f = O.window_evidence(q, K, V, n)
    want = np.zeros(n)
    for t in range(w):
        nt = n - w + t + 1
        want[:nt] += 1.0 / nt
    for g in range(Hkv):
        np.testing.assert_allclose(f[g], want / w, rtol=1e-12)


# ------------------------------------------- Soft-NMS and cross-head exclusivity

def test_soft_nms_hand_case_and_identities():
    """Hand-computed: radius 1, alpha 0.5 over s = [0.5, 0.95, 0.9, 0.1, 0.6]:
    keys 0 and 2 have one stronger neighbour (key 1), so they halve; key 3
    has two (keys 2 and 4), so it is quartered; top-2 moves from {1, 2} to
    {1, 4}.  alpha = 0 or radius = 0 is the identity."""
    s = np.array([0.5, 0.95, 0.9, 0.1, 0.6])
    out = O.soft_nms(s, 0, 5, 1, 0.5)
    np.testing.assert_allclose(out, [0.25, 0.95, 0.45, 0.025, 0.6], rtol=1e-15)
    assert list(O.topk_indices(s, 0, 5, 2)) == [1, 2]
    assert list(O.topk_indices(out, 0, 5, 2)) == [1, 4]
    np.testing.assert_array_equal(O.soft_nms(s, 0, 5, 1, 0.0), s)
    np.testing.assert_array_equal(O.soft_nms(s, 0, 5, 0, 0.5), s)
    # outside the candidate range nothing changes; neighbours outside it do not count
    out = O.soft_nms(s, 1, 4, 1, 0.5)
    np.testing.assert_allclose(out, [0.5, 0.95, 0.45, 0.05, 0.6], rtol=1e-15)


def test_soft_nms_invariants():
    """Scores never grow; a key with no stronger candidate within the radius
    keeps its score; equal neighbours: the lower index counts as stronger."""
    rng = np.random.default_rng(31)
    s = rng.random(300)
    out = O.soft_nms(s, 10, 290, 3, 0.4)
    assert np.all(out <= s)
    for j in range(10, 290):
        nb = [i for i in range(max(10, j - 3), min(290, j + 4)) if i != j]
        if all(s[i] < s[j] for i in nb):
            assert out[j] == s[j]
    eq = np.array([0.3, 0.3, 0.3])
    np.testing.assert_allclose(O.soft_nms(eq, 0, 3, 1, 0.5), [0.3, 0.15, 0.15], rtol=1e-15)


def test_exclusivity_hand_case_and_identities():
    """Hand-computed: two heads, k = 1, both pick key 0 first; with beta 0.5
    each halves key 0 once (one other head picked it), so both move to key
    1.  beta = 0 or a single head is the plain Top-K."""
    rows = [np.array([0.9, 0.8]), np.array([0.9, 0.85])]
    out, lists = O.exclusive_topk(rows, 0, 2, 1, 0.5)
    np.testing.assert_allclose(out[0], [0.45, 0.8])
    np.testing.assert_allclose(out[1], [0.45, 0.85])
    assert [list(t) for t in lists] == [[1], [1]]
    _, lists0 = O.exclusive_topk(rows, 0, 2, 1, 0.0)
    assert [list(t) for t in lists0] == [[0], [0]]
    _, one = O.exclusive_topk(rows[:1], 0, 2, 1, 0.5)
    assert [list(t) for t in one] == [[0]]
    # a key is scaled once per OTHER head that picked it: head 0's pick
    # (key 0) is kept in head 0 and halved in head 1, and vice versa
    rows = [np.array([0.9, 0.1, 0.2]), np.array([0.1, 0.9, 0.2])]
    out, lists = O.exclusive_topk(rows, 0, 3, 1, 0.5)
    np.testing.assert_allclose(out[0], [0.9, 0.05, 0.2])
    np.testing.assert_allclose(out[1], [0.05, 0.9, 0.2])
    assert [list(t) for t in lists] == [[0], [1]]


def test_soft_nms_closed_forms_on_monotone_runs():
    """With the radius covering the whole range, a strictly decreasing run
    has every lower index ranking above, so key j keeps s_j (1 - a)^j; an
    increasing run gives (1 - a)^(n - 1 - j); a constant run ranks by index
    (the decreasing case again).  Checked against these closed forms."""
    n, a = 7, 0.3
    dec = np.linspace(1.0, 0.4, n)
    np.testing.assert_allclose(O.soft_nms(dec, 0, n, n, a), dec * (1 - a) ** np.arange(n), rtol=1e-14)
    inc = dec[::-1].copy()
    np.testing.assert_allclose(O.soft_nms(inc, 0, n, n, a), inc * (1 - a) ** (n - 1 - np.arange(n)),
                               rtol=1e-14)
    const = np.full(n, 0.5)
    np.testing.assert_allclose(O.soft_nms(const, 0, n, n, a), const * (1 - a) ** np.arange(n), rtol=1e-14)
    # radius 2 on the decreasing run: key j has min(j, 2) stronger neighbours
    np.testing.assert_allclose(O.soft_nms(dec, 0, n, 2, a), dec * (1 - a) ** np.minimum(np.arange(n), 2),
                               rtol=1e-14)


def test_exclusivity_closed_form_on_identical_rows():
    """H identical rows: every first list is the same top-k, so each picked
    key is scaled by (1 - beta)^(H - 1) in every row and the others keep
    their score; the second Top-K of that closed form is every row's list."""
    rng = np.random.default_rng(8)
    n, k, H, beta = 40, 6, 3, 0.5
    base = rng.random(n)
    rows = [base.copy() for _ in range(H)]
    out, lists = O.exclusive_topk(rows, 0, n, k, beta)
    first = O.topk_indices(base, 0, n, k)
    want = base.copy()
    want[first] *= (1 - beta) ** (H - 1)
    for g in range(H):
        np.testing.assert_allclose(out[g], want, rtol=1e-14)
        np.testing.assert_array_equal(lists[g], O.topk_indices(want, 0, n, k))
    assert set(lists[0]) != set(first)      # the penalty moved part of the list


def test_soft_nms_log_scores_hand_case():
    """RAW scores (Vegas' summed logits) are already log scores, so the
    penalty is subtracted: radius 1, alpha 0.5 over s = [-1, -2, -1.5, -3]:
    key 1 has two stronger neighbours -> -2 + 2 ln 0.5, key 3 one -> -3 +
    ln 0.5, keys 0 and 2 none.  A negative score never rises (the top-2
    stays {0, 2}); multiplying it by 0.5 would lift key 1 to -1 and
    promote it above key 2."""
    s = np.array([-1.0, -2.0, -1.5, -3.0])
    out = O.soft_nms(s, 0, 4, 1, 0.5, log_scores=True)
    ln2 = math.log(2.0)
    np.testing.assert_allclose(out, [-1.0, -2.0 - 2 * ln2, -1.5, -3.0 - ln2], rtol=1e-15)
    assert list(O.topk_indices(out, 0, 4, 2)) == [0, 2]
    assert np.all(out <= s)


def test_refinements_in_log_space_agree_between_domains():
    """The log-score reading, checked across its two forms: for positive
    scores, Soft-NMS and exclusivity on log s with additive penalties equal
    the log of the multiplicative forms on s (same ranks, same counts)."""
    rng = np.random.default_rng(12)
    s = rng.random(200) + 0.01
    for radius, alpha in ((1, 0.5), (4, 0.3), (8, 0.9)):
        mult = O.soft_nms(s, 5, 190, radius, alpha)
        logv = O.soft_nms(np.log(s), 5, 190, radius, alpha, log_scores=True)
        np.testing.assert_allclose(logv, np.log(mult), rtol=1e-12, atol=1e-12)
    rows = [rng.random(60) + 0.01 for _ in range(4)]
    out_m, lists_m = O.exclusive_topk(rows, 2, 50, 7, 0.4)
    out_l, lists_l = O.exclusive_topk([np.log(r) for r in rows], 2, 50, 7, 0.4, log_scores=True)
    for a, b, la, lb in zip(out_m, out_l, lists_m, lists_l):
        np.testing.assert_allclose(b, np.log(a), rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(la, lb)


def test_exclusivity_log_scores_hand_case():
    """Two heads of negative RAW scores, k = 1, both pick key 0 first; beta
    0.5 lowers key 0 by ln 2 in each row (one other head picked it): -1 -
    ln 2 = -1.69 < -1.2 and < -1.5, so both move to key 1."""
    rows = [np.array([-1.0, -1.2]), np.array([-1.0, -1.5])]
    out, lists = O.exclusive_topk(rows, 0, 2, 1, 0.5, log_scores=True)
    np.testing.assert_allclose(out[0], [-1.0 - math.log(2.0), -1.2], rtol=1e-15)
    np.testing.assert_allclose(out[1], [-1.0 - math.log(2.0), -1.5], rtol=1e-15)
    assert [list(t) for t in lists] == [[1], [1]]


def test_soft_nms_ranks_in_float64():
    """Two scores that are equal in float32 but not in float64 rank by their
    float64 values: the later, larger one suppresses the earlier one."""
    a = 0.5
    b = 0.5 + 1e-12                      # rounds to 0.5 in float32
    assert np.float32(a) == np.float32(b)
    out = O.soft_nms(np.array([a, b]), 0, 2, 1, 0.5)
    np.testing.assert_allclose(out, [a * 0.5, b], rtol=1e-15)


# ----------------------------------------------------------- key norms, k-th score

def test_key_norms_hand_values():
    """Pythagorean rows are exact in bf16 and give exact norms: (3, 4) -> 5,
    (5, 12) -> 13, (8, 15) -> 17, (1, 2, 2) -> 3, a sign flip changes
    nothing and a zero row gives 0; two kv heads are kept apart, and keys
    past n are not returned."""
    d = 8
    K = np.zeros((2, 6, d), dtype=np.float32)
    K[0, 0, :2] = [3, 4]
    K[0, 1, :2] = [5, 12]
    K[0, 2, 3:5] = [-8, 15]
    K[0, 3, :3] = [1, -2, 2]
    K[1, 0, 7] = -7
    K[1, 1, :] = 0.5                      # sqrt(8 * 0.25) = sqrt(2)
    K[1, 2, :4] = [2, 2, 2, 2]            # 4
    K[1, 4, :] = 1e6                      # past n: ignored
    bits = (K.view(np.uint32) >> 16).astype(np.uint16)
    nu = O.key_norms(bits, 4)
    assert nu.shape == (2, 4)
    np.testing.assert_array_equal(nu[0], [5.0, 13.0, 17.0, 3.0])
    np.testing.assert_allclose(nu[1], [7.0, math.sqrt(2.0), 4.0, 0.0], rtol=1e-15)


def test_key_norms_scale_and_agree_with_the_prior():
    """A power-of-two scale of the keys scales the norms exactly, and the
    norms are the ones the prior standardises: with two keys the population
    z-scores are -1 and +1, so the prior's ratio is fixed by which norm is
    larger (checked for the norms key_norms returns)."""
    rng = np.random.default_rng(3)
    K = rng.standard_normal((2, 5, 16)).astype(np.float32)
    bits = (K.view(np.uint32) >> 16).astype(np.uint16)
    bits4 = ((K * 4).view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(O.key_norms(bits4, 5), 4 * O.key_norms(bits, 5))
    nu = O.key_norms(bits, 2)
    r = O.prior(bits, 2, norm_coef=0.5, pos_tau=1e9)   # position factor ~2 for both keys
    for g in range(2):
        big = int(np.argmax(nu[g]))
        want = math.exp(-0.5) / (math.exp(-0.5) + math.exp(0.5))
        np.testing.assert_allclose(r[g, big], want, rtol=1e-8)


def test_kth_score_hand_cases():
    """Hand cases: s = [5, 3, 3, 1, 4] over [0, 5) sorted is 5, 4, 3, 3, 1;
    equal scores count separately; |C| <= k gives None (every candidate is
    taken); |C| = k + 1 gives the k-th, not the last; a sub-range [1, 4)
    ranks only its own keys."""
    s = np.array([5.0, 3.0, 3.0, 1.0, 4.0])
    assert O.kth_score(s, 0, 5, 1) == 5.0
    assert O.kth_score(s, 0, 5, 2) == 4.0
    assert O.kth_score(s, 0, 5, 3) == 3.0
    assert O.kth_score(s, 0, 5, 4) == 3.0          # |C| = k + 1
    assert O.kth_score(s, 0, 5, 5) is None         # |C| = k
    assert O.kth_score(s, 0, 5, 6) is None
    assert O.kth_score(s, 1, 4, 1) == 3.0
    assert O.kth_score(s, 1, 4, 2) == 3.0
    assert O.kth_score(s, 1, 4, 3) is None
    assert O.kth_score(s, 2, 2, 1) is None         # empty range


def test_kth_score_is_the_weakest_selected_score():
    """Brute force: for |C| > k the k-th score is the minimum over the
    Top-K, and exactly k - 1 candidates of the Top-K beat it strictly or
    tie it at a lower rank; every unselected candidate is <= it."""
    rng = np.random.default_rng(44)
    for _ in range(50):
        n = int(rng.integers(3, 40))
        s = rng.integers(0, 6, n).astype(np.float64)       # many ties
        lo = int(rng.integers(0, 2))
        hi = int(rng.integers(lo + 2, n + 1))
        k = int(rng.integers(1, hi - lo))
        kth = O.kth_score(s, lo, hi, k)
        sel = O.topk_indices(s, lo, hi, k)
        assert kth == s[sel].min()
        rest = np.setdiff1d(np.arange(lo, hi), sel)
        assert np.all(s[rest] <= kth)
        assert int(np.sum(s[lo:hi] > kth)) <= k - 1
