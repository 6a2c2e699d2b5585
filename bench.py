"""Decode-attention throughput of the slow/fast mix on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: one Llama-3-8B-shaped attention layer (B=8, Hq=32, Hkv=8, d=128)
at 32K context, bf16 KV resident in HBM, 4 sinks + 256-token window + 2048
selected keys per kv head, lambda 0.3, sentence-driven schedule (mean
sentence 20 tokens, reuse budget 16).  A step is one decode step of the whole
batch: every sequence takes either a slow step (dense attention with
evidence, then the selector) or a fast step (sparse attention), as the
schedule says.  The K timed steps are replayed from one HIP graph; inputs are
on the device before the clock starts.

Printed: one JSON line with the throughput, a roofline record for the
dominant call (algorithmic bytes / duration from HIP events on the launch
stream in a second, eager pass over the same steps, each call preceded by a
1 GiB read that evicts L2 and the Infinity Cache), and the CPU oracle's
throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama3_8b_layer_32k.json")
METRIC = "decode attn tokens/s (slow+fast mix) at 32K/128K ctx; % HBM roofline/kernel"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(kind, n, cfg):
    """Bytes the method must move for one sequence-step (per layer)."""
    Hkv, Hq, d, k = cfg.Hkv, cfg.Hq, cfg.d, cfg.k
    if kind == "dense":
        return n * Hkv * 4 * d + Hq * d * 6
    if kind == "slow":
        return n * Hkv * 4 * d + Hq * d * 6 + n * Hkv * 8
    if kind == "select":
        return n * Hkv * 8 + k * Hkv * 4
    if kind == "fast":
        rows = min(cfg.n_sink, n) + min(cfg.window, n) + k
        return rows * Hkv * 4 * d + k * Hkv * 4 + Hq * d * 6
    raise ValueError(kind)


def kernel_source_hash():
    """sha256 over every HIP source of the library: counter-derived traffic
    is reported only while the kernels are the ones it was measured on."""
    import hashlib
    csrc = os.path.join(ROOT, "dynamic_sparse_kv_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".h")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kind, alg_bytes_per_launch):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE
    measurement (measured/algorithmic ratio of this call kind on this
    workload, scaled to this run's launches), or None if the kernels changed."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash() or kind not in t.get("ratio", {}):
        return None
    return int(round(t["ratio"][kind] * alg_bytes_per_launch))


def cpu_baseline(cfg, K, V, q_host, slow, ctx, budget_s=20.0):
    """The oracle, untuned, on a bounded sample: slow and fast steps of
    sequence 0; per-kind mean time x the run's slow fraction -> tokens/s."""
    import torch
    from oracle import sfi_oracle as O
    from dynamic_sparse_kv_amd.workload import bf16_bits

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    b = 0
    n_max = int(ctx[b]) + slow.shape[0]
    Kb = bf16_bits(K[b, :, :n_max])
    Vb = bf16_bits(V[b, :, :n_max])
    qb = bf16_bits(q_host[:, b])
    t_slow, t_fast = [], []
    sel = None
    t_start = time.perf_counter()
    for s in range(slow.shape[0]):
        n = int(ctx[b]) + s + 1
        t0 = time.perf_counter()
        if slow[s, b] or sel is None:
            r = O.slow_select(qb[s], Kb, Vb, n, lam=cfg.lam, k=cfg.k, n_sink=cfg.n_sink,
                              window=cfg.window, norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau)
            sel = r["sel"]
            t_slow.append(time.perf_counter() - t0)
        else:
            O.fast_step(qb[s], Kb, Vb, n, sel, cfg.n_sink, cfg.window)
            t_fast.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s and len(t_slow) >= 1 and len(t_fast) >= 2:
            break
    frac = float(slow.mean())
    per_tok = frac * np.mean(t_slow) + (1 - frac) * np.mean(t_fast)
    return {
        "value": round(1.0 / per_tok, 3),
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"sequence 0 of the same workload: {len(t_slow)} slow + {len(t_fast)} fast "
                   f"steps (NumPy fp64), mean per kind weighted by the run's slow fraction "
                   f"{frac:.4f}; {time.perf_counter() - t_start:.1f} s of CPU work"),
        "slow_step_s": round(float(np.mean(t_slow)), 4),
        "fast_step_s": round(float(np.mean(t_fast)), 4),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (a known-size kernel "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from dynamic_sparse_kv_amd import sfi
    from dynamic_sparse_kv_amd import workload as W
    from dynamic_sparse_kv_amd.runner import DecodePlan, SFIDecoder

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sfi.lib()
    dev = "cuda"
    if args.calib_copy:
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = W.CONFIGS[args.config]
    K_steps, W_steps = args.steps, args.warmup
    plan_steps = max(K_steps, W_steps, 1)
    cfg = cfg.replace(steps=plan_steps)

    _log(f"[bench] generating {cfg.name} inputs")
    K, V = W.make_kv(cfg, device=dev)
    ctx = W.context_lengths(cfg)
    starts = W.sentence_starts(cfg)
    slow = sfi.sfi_schedule(starts, cfg.budget).astype(bool)
    q_host = W.make_queries(cfg, starts)
    q = q_host.to(dev)
    plan = DecodePlan(slow, ctx, dev)
    max_len = int(ctx.max()) + plan_steps
    dec = SFIDecoder(K, V, cfg.Hq, max_len, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k,
                     lam=cfg.lam, norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def run_steps(n_steps):
        for s in range(n_steps):
            dec.step(plan, s, q, stream)

    _log(f"[bench] warmup {W_steps} steps")
    run_steps(W_steps)
    torch.cuda.synchronize()

    # ---- headline: K steps replayed from one HIP graph -------------------
    use_graph = not args.no_graph
    side = torch.cuda.Stream()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for s in range(K_steps):
                    dec.step(plan, s, q, side)
        torch.cuda.synchronize()
        g.replay()                      # untimed replay (first launch of the graph)
        torch.cuda.synchronize()
        _log("[bench] timing graph replay")
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t0
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(K_steps)
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t0
    tokens = cfg.B * K_steps
    value = tokens / t_total

    # ---- eager pass: HIP events around every call, each call preceded by a
    # 1 GiB read that evicts L2 and the Infinity Cache and keeps the stream
    # busy while the host enqueues the call and its events ----------------
    _log("[bench] per-call timing pass")
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    calls = {"step": [], "slow": [], "select": [], "fast": []}
    bytes_by = {"step": [], "slow": [], "select": [], "fast": []}
    ev = []

    def timed(kind, fn, nbytes):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ev.append((kind, e0, e1, nbytes))

    for s in range(K_steps):
        ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
        lens = plan.seq_len_host[s]
        sb = sum(algorithmic_bytes("slow", int(lens[b]), cfg) for b in np.nonzero(plan.slow[s])[0])
        fb = sum(algorithmic_bytes("fast", int(lens[b]), cfg) for b in np.nonzero(~plan.slow[s])[0])
        selb = sum(algorithmic_bytes("select", int(lens[b]), cfg) for b in np.nonzero(plan.slow[s])[0])
        if ns and nf:   # the co-launched slow + fast pass the step runs, then the selector
            timed("step", lambda: dec.co_step(q[s], plan.seq_len[s], plan.slow_ids[s], ns,
                                              plan.fast_ids[s], nf, stream, select=False), sb + fb)
        elif ns:
            timed("slow", lambda: dec.slow(q[s], plan.seq_len[s], plan.slow_ids[s], ns, stream,
                                           select=False), sb)
        elif nf:
            timed("fast", lambda: dec.fast(q[s], plan.seq_len[s], plan.fast_ids[s], nf, stream), fb)
        if ns:
            timed("select", lambda: dec.slow_select_only(plan.seq_len[s], plan.slow_ids[s], ns, stream),
                  selb)
    torch.cuda.synchronize()
    del flush
    for kind, a, b_, nbytes in ev:
        calls[kind].append(a.elapsed_time(b_) * 1e-3)
        bytes_by[kind].append(nbytes)
    per_call = {}
    for kind in calls:
        if calls[kind]:
            t = float(np.mean(calls[kind]))
            by = float(np.mean(bytes_by[kind]))
            per_call[kind] = {"launches": len(calls[kind]), "avg_us": round(t * 1e6, 2),
                              "total_ms": round(sum(calls[kind]) * 1e3, 3),
                              "alg_bytes_per_launch": int(by),
                              "alg_GBps": round(by / t / 1e9, 1)}
    dom = max(per_call, key=lambda k_: per_call[k_]["total_ms"])
    dc = per_call[dom]
    achieved = dc["alg_GBps"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, dc["alg_bytes_per_launch"]),
                "kernel": {"step": "sfi_decode_step: co-launched slow + fast partial and finalize kernels",
                           "slow": "sfi_slow_step: split-K partial + finalize kernels",
                           "select": "sfi_select: four chunk-parallel selector kernels (norm sums, prior, keys + bucket sort, pick)",
                           "fast": "sfi_fast_step: gather partial + finalize kernels"}[dom]}

    # ---- all-dense comparator: every sequence dense every step -----------
    _log("[bench] dense comparator")
    all_ids = torch.arange(cfg.B, dtype=torch.int32, device=dev)
    n_dense = min(K_steps, 64)
    if use_graph:
        gd = torch.cuda.CUDAGraph()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(gd, stream=side):
                for s in range(n_dense):
                    dec.dense(q[s], plan.seq_len[s], all_ids, cfg.B, side)
        torch.cuda.synchronize()
        gd.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gd.replay()
        torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        for s in range(n_dense):
            dec.dense(q[s], plan.seq_len[s], all_ids, cfg.B, stream)
        torch.cuda.synchronize()
    t_dense = (time.perf_counter() - t0) / n_dense
    dense_tps = cfg.B / t_dense

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": round(t_total / K_steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one attention layer, B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} "
                               f"d={cfg.d}, ctx {cfg.ctx}, fast state {cfg.n_sink}+{cfg.window}+{cfg.k}, "
                               f"lambda {cfg.lam}, {K_steps} decode steps",
                   "global_batch": cfg.B, "seq_len": cfg.ctx, "parallelism": "none (1 GPU)",
                   "slow_fraction": round(float(plan.slow[:K_steps].mean()), 4),
                   "timing": "hip graph replay, one stream" if use_graph else "eager, one stream"},
        "roofline": roofline,
        "per_call": per_call,
        "dense_tokens_per_s": round(dense_tps, 1),
        "fast_vs_dense_speedup": round(value / dense_tps, 2),
    }
    if not args.no_cpu_baseline:
        _log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(cfg, K, V, q_host, slow[:K_steps], ctx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
