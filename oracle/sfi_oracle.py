"""CPU oracle for slow-fast decode attention and verification-guided selection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library.

Everything here is the plain definition, evaluated in float64 over the exact
bf16 input values, with NumPy primitives (a matrix product, a sort) as steps
and no blocking, fusion or reordering.

Sources (cited below by short tag):

* [SFI-it] "Slow-Fast Inference: Training-Free Inference Acceleration via
  Within-Sentence Support Stability", gist.science/it/paper/2603.12038,
  Italian technical summary ("Sommario tecnico"): section 1 (decode attention
  over the whole cached history), section 3.A (fast steps over sink tokens,
  recent window and selected memory; slow steps with dense attention at
  semantic boundaries or when the reuse budget runs out), section 3.B
  (selector: evidence from slow-step attention, prior from key norms and
  positions, closed-form reverse-KL fusion, Top-K).
* [SFI-pt] same paper, gist.science/pt/paper/2603.12038, Portuguese summary
  ("Resumo técnico"), section 2.A (fast-step cost independent of context
  length) and 2.B (fusion is an arithmetic interpolation; Top-K updates the
  index set).
* [SFI-ko] same paper, gist.science/ko/paper/2603.12038, Korean summary,
  section 2.A (window of about 256 recent tokens) and section 2.B (objective
  s = argmin (1-lam) KL(f||s) + lam KL(r||s) and its closed form
  (1-lam) f + lam r).
* [Vegas] "Vegas: Decodifica Auto-Speculativa con Attenzione Sparsa Guidata
  dalla Verifica", gist.science/it/paper/2602.07223: section 2 (verify with
  full attention, select from its logits, draft with sparse attention),
  section 2.A (selection formula: argmax over |T| = k of the attention logits
  summed over the gamma+1 verified queries and all query heads),
  section 2.B (Collect-2-Query: only the first draft query and the bonus
  query), section 3 (pre-softmax logits).

Readings where the pages leave a step open (each also listed in the design
notes): evidence f is the softmax probability of the slow-step query averaged
over the query heads of one GQA group, logits scaled by 1/sqrt(d); GQA head h
reads kv head h // G; the prior is the workload's formula (pages give only its
ingredients) -- its fidelity to the paper is parity unpinned; f, r and s live
on all n cached keys and are not renormalised over the candidates; the
candidates of the Top-K exclude the sink and window ranges, ties go to the
lower index and the result is returned ascending.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# Input decoding
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the upper half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# O1: dense attention of one decode query  [SFI-it s1, s3.A slow steps]
# ---------------------------------------------------------------------------

def attention_logits(q, K, n: int) -> np.ndarray:
    """l[h, j] = q_h . k_{h//G, j} / sqrt(d) for j < n.  q [Hq][d], K [Hkv][>=n][d]."""
    q = _as_f64(q)
    K = _as_f64(K[:, :n])
    Hq, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    l = np.empty((Hq, n))
    for h in range(Hq):
        l[h] = K[h // G] @ q[h] / math.sqrt(d)
    return l


def softmax_rows(l: np.ndarray) -> np.ndarray:
    m = l.max(axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=-1, keepdims=True)


def dense_step(q, K, V, n: int):
    """Slow (dense) step.  Returns (o [Hq][d], p [Hq][n])."""
    l = attention_logits(q, K, n)
    p = softmax_rows(l)
    Vf = _as_f64(V[:, :n])
    Hq = p.shape[0]
    G = Hq // Vf.shape[0]
    o = np.stack([p[h] @ Vf[h // G] for h in range(Hq)])
    return o, p


# ---------------------------------------------------------------------------
# O2: evidence distribution  [SFI-it s3.B; SFI-ko s2.B evidence f]
# ---------------------------------------------------------------------------

def evidence(p: np.ndarray, Hkv: int) -> np.ndarray:
    """f[g, j] = mean of p[h, j] over the G query heads of kv head g."""
    Hq, n = p.shape
    G = Hq // Hkv
    return p.reshape(Hkv, G, n).mean(axis=1)


def window_evidence(q_rows, K, V, n: int):
    """Evidence observed over a window of w queries [SFI-it s3.B: the logits
    observed in the slow step's window; reading: the window is the last w
    decode queries].  Row t (0..w-1) sits at position n - w + t and attends
    keys [0, n - w + t].  Returns (o [w][Hq][d], f [Hkv][n]) with
    f[g, j] = (1 / (w G)) sum_t sum_{h of group g} p_t[h, j], where p_t is row
    t's softmax over its visible keys (zero beyond them)."""
    q_rows = _as_f64(q_rows)
    w, Hq, d = q_rows.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    o = np.empty((w, Hq, d))
    f = np.zeros((Hkv, n))
    for t in range(w):
        nt = n - w + t + 1
        l = attention_logits(q_rows[t], K, nt)
        p = softmax_rows(l)
        Vf = _as_f64(V[:, :nt])
        for h in range(Hq):
            o[t, h] = p[h] @ Vf[h // G]
            f[h // G, :nt] += p[h]
    return o, f / (w * G)


# ---------------------------------------------------------------------------
# O3: prior from cache statistics  [SFI-it s3.B prior from key norms and
# positions; formula: the workload's choice -- parity unpinned w.r.t. pages]
# ---------------------------------------------------------------------------

def prior(K, n: int, norm_coef: float = 0.5, pos_tau: float = 1024.0) -> np.ndarray:
    """r[g, j] proportional to exp(-norm_coef z_j) (1 + exp(-(t - j)/pos_tau)).

    z_j is the key norm standardised with the population mean and standard
    deviation over the n cached keys of that kv head (z = 0 when the std is
    zero); t = n - 1 is the position of the slow-step query.
    """
    Kf = _as_f64(K[:, :n])
    nu = np.sqrt((Kf * Kf).sum(axis=-1))            # [Hkv][n]
    mu = nu.mean(axis=-1, keepdims=True)
    sd = nu.std(axis=-1, keepdims=True)             # population (ddof = 0)
    z = np.where(sd > 0, (nu - mu) / np.where(sd > 0, sd, 1.0), 0.0)
    t = n - 1
    j = np.arange(n, dtype=np.float64)
    w = np.exp(-norm_coef * z) * (1.0 + np.exp(-(t - j) / pos_tau))
    return w / w.sum(axis=-1, keepdims=True)


def key_norms(K, n: int) -> np.ndarray:
    """nu[g, j] = Euclidean norm of key j of kv head g, j < n: the norm
    statistic the prior standardises [SFI-it s3.B, key norms]."""
    Kf = _as_f64(K[:, :n])
    return np.sqrt((Kf * Kf).sum(axis=-1))


# ---------------------------------------------------------------------------
# O4: reverse-KL fusion, closed form  [SFI-ko s2.B; SFI-pt s2.B]
# ---------------------------------------------------------------------------

def fuse(f: np.ndarray, r: np.ndarray, lam: float) -> np.ndarray:
    """s = (1 - lam) f + lam r, the minimiser of (1-lam) KL(f||s) + lam KL(r||s)."""
    return (1.0 - lam) * f + lam * r


# ---------------------------------------------------------------------------
# O5: Top-K discretisation  [SFI-it s3.B; SFI-pt s2.B]
# ---------------------------------------------------------------------------

def topk_indices(score: np.ndarray, lo: int, hi: int, k: int) -> np.ndarray:
    """The min(k, |C|) best of C = [lo, hi) by (score desc, index asc), ascending."""
    lo = max(lo, 0)
    if hi <= lo or k <= 0:
        return np.zeros(0, dtype=np.int64)
    j = np.arange(lo, hi)
    s = np.asarray(score[lo:hi], dtype=np.float64)
    order = np.lexsort((j, -s))                     # primary -s, then j
    return np.sort(j[order[:k]])


def _penalise(s, m, keep: float, log_scores: bool):
    """A penalty of m log(1/keep) in log-score space: for a probability-like
    score (FUSED) log s' = log s + m log keep, i.e. s' = s keep^m; a score
    that is already a log score (RAW: Vegas' summed logits) loses
    m log(1/keep) directly."""
    if log_scores:
        return s + m * math.log(keep)
    return s * keep ** m


def soft_nms(score, lo: int, hi: int, radius: int, alpha: float, log_scores: bool = False) -> np.ndarray:
    """Soft-NMS inside one head row [SFI-it s3.B: a refinement applied to the
    log scores before the Top-K; SFI-pt s2.B: keeps neighbouring, correlated
    keys from filling the budget; the pages give no formula -- this reading:
    one pass, not greedy].  For a candidate j of [lo, hi), m_j = number of
    candidates i with 0 < |i - j| <= radius that rank above j (larger score,
    or an equal score and a lower index), compared in float64; the log score
    of j drops by m_j log(1 / (1 - alpha)) (see _penalise); other keys keep
    theirs.  Parity of this form with the paper: unpinned."""
    s = np.asarray(score, dtype=np.float64)
    out = s.copy()
    lo = max(lo, 0)
    if hi <= lo or radius <= 0 or alpha == 0.0:
        return out
    for j in range(lo, hi):
        m = 0
        for i in range(max(lo, j - radius), min(hi, j + radius + 1)):
            if i != j and (s[i] > s[j] or (s[i] == s[j] and i < j)):
                m += 1
        out[j] = _penalise(s[j], m, 1.0 - alpha, log_scores)
    return out


def exclusive_topk(rows, lo: int, hi: int, k: int, beta: float, log_scores: bool = False):
    """Cross-head exclusivity over the head rows of one sequence [SFI-it
    s3.B, SFI-pt s2.B: penalise the same key being picked by several heads;
    no formula in the pages -- this reading].  T_g = Top-K of row g;
    c_j = number of rows whose T_g holds j; the log score of row g's key j
    drops by (c_j - [j in T_g]) log(1 / (1 - beta)) (once per other head that
    picked it; see _penalise) and the Top-K is taken again.  Returns
    (rescaled rows, final lists).  Parity of this form with the paper:
    unpinned."""
    rows = [np.asarray(r, dtype=np.float64) for r in rows]
    first = [topk_indices(r, lo, hi, k) for r in rows]
    if beta == 0.0 or len(rows) < 2:
        return rows, first
    n = len(rows[0])
    c = np.zeros(n, dtype=np.int64)
    for t in first:
        c[t] += 1
    out = []
    for r, t in zip(rows, first):
        own = np.zeros(n, dtype=np.int64)
        own[t] = 1
        out.append(_penalise(r, c - own, 1.0 - beta, log_scores))
    return out, [topk_indices(r, lo, hi, k) for r in out]


def candidate_range(n: int, n_sink: int, window: int):
    """Selectable keys at a slow step of length n: [n_sink, n - window)."""
    return n_sink, max(n_sink, n - window)


def kth_score(score: np.ndarray, lo: int, hi: int, k: int) -> Optional[float]:
    """The k-th largest score over [lo, hi), counting equal scores
    separately (None when |C| <= k: every candidate is then selected and no
    near-tie decision exists).  It sets the near-tie band of the selection
    checks."""
    if hi - lo <= k:
        return None
    s = np.sort(np.asarray(score[lo:hi], dtype=np.float64))[::-1]
    return float(s[k - 1])


# ---------------------------------------------------------------------------
# O6: fast step over sinks + recent window + selected memory  [SFI-it s3.A;
# SFI-ko s2.A]
# ---------------------------------------------------------------------------

def fast_key_set(n: int, sel: Sequence[int], n_sink: int, window: int) -> np.ndarray:
    """Sorted attended set: [0, min(n_sink, n)) U [max(n_sink, n - W), n) U
    {j in sel : n_sink <= j < n - W}."""
    sinks = np.arange(0, min(n_sink, n))
    wlo = max(n_sink, n - window)
    win = np.arange(wlo, n)
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[(sel >= n_sink) & (sel < wlo)]
    return np.unique(np.concatenate([sinks, win, sel]))


def fast_step(q, K, V, n: int, sel_per_kv: Sequence[Sequence[int]], n_sink: int, window: int):
    """Attention of one query over the fast set of its kv head.  o [Hq][d]."""
    q = _as_f64(q)
    Hq, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    o = np.empty((Hq, d))
    for g in range(Hkv):
        A = fast_key_set(n, sel_per_kv[g], n_sink, window)
        Kg = _as_f64(K[g, A])
        Vg = _as_f64(V[g, A])
        for h in range(g * G, (g + 1) * G):
            l = Kg @ q[h] / math.sqrt(d)
            p = np.exp(l - l.max())
            p /= p.sum()
            o[h] = p @ Vg
    return o


# ---------------------------------------------------------------------------
# O7: schedule  [SFI-it s3.A; SFI-ko s2.A: slow at semantic boundaries or
# when the reuse budget is spent]
# ---------------------------------------------------------------------------

def schedule(starts: np.ndarray, budget: Optional[int]) -> np.ndarray:
    """slow[s, b]: step 0 is slow; later a step is slow when a sentence starts
    there, or when the previous ``budget`` steps were all fast."""
    steps, B = starts.shape
    slow = np.zeros((steps, B), dtype=bool)
    for b in range(B):
        run = 0
        for s in range(steps):
            if s == 0 or starts[s, b] or (budget is not None and run >= budget):
                slow[s, b] = True
                run = 0
            else:
                run += 1
    return slow


# ---------------------------------------------------------------------------
# Whole slow step of the selector  (O1 -> O2, O3 -> O4 -> O5)
# ---------------------------------------------------------------------------

def slow_select(q, K, V, n: int, *, lam: float, k: int, n_sink: int, window: int,
                norm_coef: float = 0.5, pos_tau: float = 1024.0):
    """Dense step plus selector.  Returns dict with o, f, r, s, sel (list per kv head)."""
    o, p = dense_step(q, K, V, n)
    Hkv = K.shape[0]
    f = evidence(p, Hkv)
    r = prior(K, n, norm_coef, pos_tau)
    s = fuse(f, r, lam)
    lo, hi = candidate_range(n, n_sink, window)
    sel = [topk_indices(s[g], lo, hi, k) for g in range(Hkv)]
    return {"o": o, "p": p, "f": f, "r": r, "s": s, "sel": sel, "lo": lo, "hi": hi}


def decode_run(q_steps, K, V, ctx: int, slow: np.ndarray, *, lam: float, k: int,
               n_sink: int, window: int, norm_coef: float = 0.5, pos_tau: float = 1024.0):
    """One sequence through a slow/fast schedule.

    Step s attends n = ctx + s + 1 keys.  Slow steps run dense attention and
    replace the selected memory; fast steps attend the fast set built from
    the last slow step's selection.  Returns a list of per-step dicts.
    """
    out = []
    sel = None
    for s in range(len(slow)):
        n = ctx + s + 1
        if slow[s]:
            r = slow_select(q_steps[s], K, V, n, lam=lam, k=k, n_sink=n_sink, window=window,
                            norm_coef=norm_coef, pos_tau=pos_tau)
            sel = r["sel"]
            out.append({"kind": "slow", "n": n, "o": r["o"], "sel": sel, "s": r["s"],
                        "f": r["f"], "lo": r["lo"], "hi": r["hi"]})
        else:
            o = fast_step(q_steps[s], K, V, n, sel, n_sink, window)
            out.append({"kind": "fast", "n": n, "o": o})
    return out


# ---------------------------------------------------------------------------
# O8: verification with aggregated logits  [Vegas s2, s2.A, s2.B, s3]
# ---------------------------------------------------------------------------

def verify(q_rows, K, V, n: int, rows: Sequence[int]):
    """T verify queries of one sequence; row t sits at position n - T + t and
    attends keys [0, n - T + t].  Returns (o [T][Hq][d], agg [n - T]) with
    agg_i = sum over t in rows and all query heads of the pre-softmax logit of
    key i, for the prefix keys i < n - T."""
    q_rows = _as_f64(q_rows)
    T, Hq, d = q_rows.shape
    o = np.empty((T, Hq, d))
    P = n - T
    agg = np.zeros(P)
    for t in range(T):
        nt = P + t + 1
        l = attention_logits(q_rows[t], K, nt)
        p = softmax_rows(l)
        Vf = _as_f64(V[:, :nt])
        G = Hq // Vf.shape[0]
        for h in range(Hq):
            o[t, h] = p[h] @ Vf[h // G]
        if t in rows:
            agg += l[:, :P].sum(axis=0)
    return o, agg


def collect_rows(T: int, mode: str) -> list:
    """Rows whose logits are aggregated: all T, or the first draft and the
    bonus query (Collect-2-Query)."""
    if mode == "all":
        return list(range(T))
    if mode == "c2q":
        return sorted({0, T - 1})
    raise ValueError(mode)


# ---------------------------------------------------------------------------
# O9: verification-guided selection  [Vegas s2.A]
# ---------------------------------------------------------------------------

def vegas_select(agg: np.ndarray, n: int, k: int, n_sink: int, window: int) -> np.ndarray:
    """Top-k of the aggregated logits over [n_sink, n - window), shared by all heads."""
    lo, hi = candidate_range(n, n_sink, window)
    hi = min(hi, len(agg))
    return topk_indices(agg, lo, hi, k)

