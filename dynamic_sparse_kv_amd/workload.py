"""Seeded synthetic inputs for the slow-fast decode attention path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no attention, no selection, no schedule decision).  Both
the HIP path (through the tests and the benchmark) and the CPU oracle are fed
from it, so the two always see the same bytes.

Shapes follow the long-context decode workloads of the Slow-Fast Inference
pages (gist.science/{it,pt,ko}/paper/2603.12038, "Slow-Fast Inference:
Training-Free Inference Acceleration via Within-Sentence Support Stability",
results section: 8K-128K contexts, GQA decoding) and of the Vegas page
(gist.science/it/paper/2602.07223, results section: up to 128K contexts,
multi-query verification).  No dataset item is reproduced: keys, values and
queries are Gaussian, with planted high-norm "heavy hitter" keys and
sentence-structured queries so that attention has stable, shifting support.

Random streams are keyed by ``SeedSequence([seed_key, layer, b, kind])``.
Large tensors are drawn with a ``torch.Generator`` on the device they are
used on; the same seed on another device gives other (equally valid) bytes, so
every consumer that needs the values on the host copies them from the tensor
that the device path reads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

KIND = {"K": 0, "V": 1, "HH": 2, "Q": 3, "SCHED": 4, "CTX": 5, "PAGES": 6}


@dataclasses.dataclass(frozen=True)
class SFIConfig:
    """One synthetic decode workload."""

    name: str
    seed_key: int          # first key of the workload's random streams
    B: int
    Hq: int
    Hkv: int
    d: int
    ctx: int                      # prefill length (ragged: upper bound)
    steps: int                    # decode steps (Vegas: iterations)
    n_sink: int = 4
    window: int = 256
    k: int = 256
    lam: float = 0.3
    norm_coef: float = 0.5
    pos_tau: float = 1024.0
    mean_sentence: float = 20.0
    budget: int = 16              # max consecutive fast steps
    hh_count: Optional[int] = None   # heavy hitters per (b, kv-head)
    hh_frac: Optional[float] = None  # ... or as a fraction of ctx
    hh_scale: float = 3.0
    rho: float = 0.95
    layers: int = 1
    vegas_T: int = 0              # verify rows per sequence (0 = SFI config)
    ragged_min: int = 0           # >0: log-uniform ctx in [ragged_min, ctx]
    page_size: int = 0            # >0: paged KV pool
    slow_prob: float = 0.0        # >0: Bernoulli slow steps instead of sentences
    k_div: int = 0                # >0: k = min(k, n // k_div)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def heavy_hitters(self, ctx: int) -> int:
        if self.hh_count is not None:
            return min(self.hh_count, ctx)
        if self.hh_frac is not None:
            return min(int(round(self.hh_frac * ctx)), ctx)
        return 0

    def growth(self) -> int:
        """Rows appended after the prefill over the whole run."""
        if self.vegas_T:
            return self.steps * self.vegas_T + self.vegas_T
        return self.steps

    def replace(self, **kw) -> "SFIConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Tiny single layer: every step fits the oracle in seconds.
    "tiny-4k": SFIConfig("tiny-4k", 1, B=1, Hq=8, Hkv=2, d=64, ctx=4096, steps=64,
                    k=256, lam=0.3, hh_count=32),
    # Llama-3-8B-shaped layer at 32K context.
    "llama3-8b-layer-32k": SFIConfig("llama3-8b-layer-32k", 2, B=8, Hq=32, Hkv=8, d=128, ctx=32768,
                    steps=256, k=2048, lam=0.3, hh_frac=0.01),
    # 32-layer stack at 128K context.
    "stack32-128k": SFIConfig("stack32-128k", 3, B=4, Hq=32, Hkv=8, d=128, ctx=131072,
                    steps=128, k=4096, lam=0.2, mean_sentence=24.0, budget=32,
                    hh_frac=0.005, layers=32),
    # Verification-guided selection at 64K context, 8 verify rows.
    "vegas-64k": SFIConfig("vegas-64k", 4, B=16, Hq=32, Hkv=8, d=128, ctx=65536, steps=64,
                    k=2048, hh_frac=0.01, vegas_T=8),
    # Ragged long-reasoning batch, paged KV, Bernoulli slow steps.
    "ragged-paged-8k-128k": SFIConfig("ragged-paged-8k-128k", 5, B=32, Hq=40, Hkv=8, d=128, ctx=131072,
                    steps=512, k=4096, lam=0.3, hh_frac=0.01, ragged_min=8192,
                    page_size=16, slow_prob=1.0 / 20.0, k_div=16),
}


def seed_for(cfg: SFIConfig, layer: int, b: int, kind: str) -> int:
    ss = np.random.SeedSequence([cfg.seed_key, layer, b, KIND[kind]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def context_lengths(cfg: SFIConfig) -> np.ndarray:
    """Prefill length per sequence (int64 [B])."""
    if not cfg.ragged_min:
        return np.full(cfg.B, cfg.ctx, dtype=np.int64)
    rng = np.random.default_rng(seed_for(cfg, 0, 0, "CTX"))
    u = rng.uniform(math.log(cfg.ragged_min), math.log(cfg.ctx), size=cfg.B)
    return np.floor(np.exp(u)).astype(np.int64)


def heavy_hitter_positions(cfg: SFIConfig, layer: int, b: int, ctx: int) -> np.ndarray:
    """Planted positions, int64 [Hkv][count], uniform without replacement in [0, ctx)."""
    cnt = cfg.heavy_hitters(ctx)
    rng = np.random.default_rng(seed_for(cfg, layer, b, "HH"))
    out = np.empty((cfg.Hkv, cnt), dtype=np.int64)
    for h in range(cfg.Hkv):
        out[h] = np.sort(rng.choice(ctx, size=cnt, replace=False))
    return out


def padded_capacity(rows: int) -> int:
    """Row capacity of a contiguous cache that holds ``rows`` rows: rounded up
    to 64 rows, plus 32.  A (sequence, kv head) stride that is an exact
    multiple of a large power of two can alias in the HBM channel mapping:
    on one MI355X a stride of 2^23 + 2^16 bytes (33024 rows of 256 B) made
    the cold fast step 2x and the dense step 15 % slower than the padded
    neighbours (layout only; nothing computed)."""
    return -(-int(rows) // 64) * 64 + 32


def make_kv(cfg: SFIConfig, layer: int = 0, device="cpu", cap: Optional[int] = None):
    """Contiguous K, V caches, bf16 [B][Hkv][cap][d].

    Entries are N(0,1); heavy-hitter key rows are scaled by ``hh_scale``
    before the single round-to-nearest-even conversion to bf16.  Rows past the
    prefill are the tokens a decode run appends; they are drawn up front so
    the cache only has to grow its length.  Without ``cap`` the run's rows
    are drawn and the capacity is padded (padded_capacity; the padding rows
    are zero); with ``cap``, all cap rows are drawn.
    """
    ctxs = context_lengths(cfg)
    rows = int(ctxs.max()) + cfg.growth() if cap is None else cap
    cap = padded_capacity(rows) if cap is None else cap
    K = torch.zeros((cfg.B, cfg.Hkv, cap, cfg.d), dtype=torch.bfloat16, device=device)
    V = torch.zeros_like(K)
    for b in range(cfg.B):
        gk = torch.Generator(device=device).manual_seed(seed_for(cfg, layer, b, "K"))
        x = torch.randn((cfg.Hkv, rows, cfg.d), generator=gk, device=device, dtype=torch.float32)
        hh = heavy_hitter_positions(cfg, layer, b, int(ctxs[b]))
        if hh.size:
            for h in range(cfg.Hkv):
                idx = torch.as_tensor(hh[h], device=device)
                x[h, idx] *= cfg.hh_scale
        K[b, :, :rows] = x.to(torch.bfloat16)
        del x
        gv = torch.Generator(device=device).manual_seed(seed_for(cfg, layer, b, "V"))
        V[b, :, :rows] = torch.randn((cfg.Hkv, rows, cfg.d), generator=gv, device=device,
                                     dtype=torch.float32).to(torch.bfloat16)
    return K, V


def sentence_starts(cfg: SFIConfig, steps: Optional[int] = None) -> np.ndarray:
    """bool [steps][B]: True where a new sentence starts at that decode step.

    Sentence lengths are Geometric on {1, 2, ...} with mean ``mean_sentence``;
    the first sentence starts at step 0.  For Bernoulli configs the array
    holds independent draws with probability ``slow_prob`` instead.
    """
    steps = cfg.steps if steps is None else steps
    out = np.zeros((steps, cfg.B), dtype=bool)
    for b in range(cfg.B):
        rng = np.random.default_rng(seed_for(cfg, 0, b, "SCHED"))
        if cfg.slow_prob > 0:
            out[:, b] = rng.random(steps) < cfg.slow_prob
            continue
        s = 0
        while s < steps:
            out[s, b] = True
            s += int(rng.geometric(1.0 / cfg.mean_sentence))
    return out


def make_queries(cfg: SFIConfig, starts: np.ndarray, layer: int = 0) -> torch.Tensor:
    """AR(1) decode queries, bf16 [steps][B][Hq][d] (host tensor).

    Within a sentence q_t = rho q_{t-1} + sqrt(1 - rho^2) e_t, at a sentence
    start q_t = e_t, with e_t ~ N(0, I); the state is kept in fp32 and each
    emitted query is rounded once to bf16.
    """
    steps = starts.shape[0]
    out = torch.empty((steps, cfg.B, cfg.Hq, cfg.d), dtype=torch.bfloat16)
    c = math.sqrt(1.0 - cfg.rho * cfg.rho)
    for b in range(cfg.B):
        g = torch.Generator().manual_seed(seed_for(cfg, layer, b, "Q"))
        eps = torch.randn((steps, cfg.Hq, cfg.d), generator=g, dtype=torch.float32)
        x = eps[0].clone()
        out[0, b] = x.to(torch.bfloat16)
        for s in range(1, steps):
            if starts[s, b]:
                x = eps[s].clone()
            else:
                x = cfg.rho * x + c * eps[s]
            out[s, b] = x.to(torch.bfloat16)
    return out


def make_vegas_queries(cfg: SFIConfig, layer: int = 0) -> torch.Tensor:
    """Per-position queries for verification runs, bf16 [positions][B][Hq][d].

    One AR(1) stream per sequence over decode positions: iteration ``it``
    verifies positions ``it*T .. it*T+T-1`` and drafts the following T-1
    positions, so a draft query and the verify query of the same position
    are identical.
    """
    positions = cfg.steps * cfg.vegas_T + cfg.vegas_T
    starts = sentence_starts(cfg, steps=positions)
    return make_queries(cfg, starts, layer=layer)


def page_table(cfg: SFIConfig, ctxs_cap: np.ndarray):
    """Shuffled page table for a paged pool.

    Returns (table int32 [B][max_pages], n_pages) where the pages of all
    sequences are a seeded permutation of one pool.
    """
    ps = cfg.page_size
    pages = [(int(c) + ps - 1) // ps for c in ctxs_cap]
    total = int(sum(pages))
    maxp = int(max(pages))
    rng = np.random.default_rng(seed_for(cfg, 0, 0, "PAGES"))
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((cfg.B, maxp), -1, dtype=np.int32)
    o = 0
    for b, p in enumerate(pages):
        table[b, :p] = perm[o:o + p]
        o += p
    return table, total


def to_paged(K: torch.Tensor, table: np.ndarray, n_pages: int, page_size: int) -> torch.Tensor:
    """Scatter a contiguous [B][Hkv][cap][d] cache into a pool [P][Hkv][page][d]."""
    B, Hkv, cap, d = K.shape
    pool = torch.zeros((n_pages, Hkv, page_size, d), dtype=K.dtype, device=K.device)
    for b in range(B):
        npg = int((table[b] >= 0).sum())
        rows = min(npg * page_size, cap)
        src = torch.zeros((Hkv, npg * page_size, d), dtype=K.dtype, device=K.device)
        src[:, :rows] = K[b, :, :rows]
        idx = torch.as_tensor(table[b, :npg].astype(np.int64), device=K.device)
        pool[idx] = src.view(Hkv, npg, page_size, d).permute(1, 0, 2, 3)
    return pool


def make_paged_kv(cfg: SFIConfig, table: np.ndarray, n_pages: int, caps: np.ndarray, layer: int = 0,
                  device="cpu"):
    """Paged K, V pools [n_pages][Hkv][page][d] drawn sequence by sequence.

    Sequence b owns cache rows [0, caps[b]) in the pages table[b][0 ..]; its
    rows are N(0,1) with planted heavy-hitter keys scaled by ``hh_scale``,
    each rounded once to bf16, from the same seeded streams as make_kv (a
    draw of caps[b] rows per head, so the bytes differ from make_kv's, which
    draws the batch-wide capacity).  Pool pages nobody owns stay zero.
    """
    ps = cfg.page_size
    ctxs = context_lengths(cfg)
    Kp = torch.zeros((n_pages, cfg.Hkv, ps, cfg.d), dtype=torch.bfloat16, device=device)
    Vp = torch.zeros_like(Kp)
    for b in range(cfg.B):
        cap = int(caps[b])
        npg = (cap + ps - 1) // ps
        idx = torch.as_tensor(table[b, :npg].astype(np.int64), device=device)
        for which, pool in (("K", Kp), ("V", Vp)):
            gen = torch.Generator(device=device).manual_seed(seed_for(cfg, layer, b, which))
            x = torch.zeros((cfg.Hkv, npg * ps, cfg.d), dtype=torch.float32, device=device)
            x[:, :cap] = torch.randn((cfg.Hkv, cap, cfg.d), generator=gen, device=device,
                                     dtype=torch.float32)
            if which == "K":
                hh = heavy_hitter_positions(cfg, layer, b, int(ctxs[b]))
                for h in range(cfg.Hkv):
                    if hh.shape[1]:
                        x[h, torch.as_tensor(hh[h], device=device)] *= cfg.hh_scale
            pool[idx] = x.to(torch.bfloat16).view(cfg.Hkv, npg, ps, cfg.d).permute(1, 0, 2, 3)
            del x
    return Kp, Vp


def gather_paged(pool: torch.Tensor, table: np.ndarray, b: int, n: int) -> torch.Tensor:
    """Rows [0, n) of sequence b from a paged pool, as [Hkv][n][d] (a copy)."""
    ps = pool.shape[2]
    npg = (n + ps - 1) // ps
    idx = torch.as_tensor(table[b, :npg].astype(np.int64), device=pool.device)
    rows = pool[idx].permute(1, 0, 2, 3).reshape(pool.shape[1], npg * ps, pool.shape[3])
    return rows[:, :n].contiguous()


def take_decode_rows(K: torch.Tensor, V: torch.Tensor, ctx: np.ndarray, steps: int, rows_per_step: int = 1,
                     table: Optional[np.ndarray] = None):
    """Move the rows a decode run appends out of the cache.

    Row t of step s of sequence b is cache row ctx[b] + s * rows_per_step + t.
    Returns (K_new, V_new), each [steps][B][rows_per_step][Hkv][d] (copies of
    those rows), and zeroes the rows in K and V, so that a run which appends
    them before each step (sfi_append_kv) sees the same bytes as the cache
    drawn up front.  Contiguous caches are [B][Hkv][cap][d]; with ``table``
    they are paged pools [P][Hkv][page][d].  Layout only: nothing computed.
    """
    T = rows_per_step
    B = len(ctx)
    if table is None:
        Hkv, d = K.shape[1], K.shape[3]
    else:
        Hkv, d = K.shape[1], K.shape[3]
        ps = K.shape[2]
    Kn = torch.empty((steps, B, T, Hkv, d), dtype=K.dtype, device=K.device)
    Vn = torch.empty_like(Kn)
    for b in range(B):
        pos = int(ctx[b]) + torch.arange(steps * T, device=K.device)
        if table is None:
            for src, dst in ((K, Kn), (V, Vn)):
                rows = src[b][:, pos]                                   # [Hkv][steps*T][d]
                dst[:, b] = rows.permute(1, 0, 2).reshape(steps, T, Hkv, d)
                src[b][:, pos] = 0
        else:
            tab = torch.as_tensor(table[b].astype(np.int64), device=K.device)
            pg, off = tab[pos // ps], pos % ps
            for src, dst in ((K, Kn), (V, Vn)):
                rows = src[pg, :, off]                                  # [steps*T][Hkv][d]
                dst[:, b] = rows.reshape(steps, T, Hkv, d)
                src[pg, :, off] = 0
    return Kn, Vn


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a tensor as a host uint16 array."""
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
