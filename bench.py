"""Decode-attention throughput of the slow/fast mix on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--replicas R] [--no-cpu-baseline]

Workload: one Llama-3-8B-shaped attention layer (B=8, Hq=32, Hkv=8, d=128)
at 32K context, bf16 KV resident in HBM, 4 sinks + 256-token window + 2048
selected keys per kv head, lambda 0.3, sentence-driven schedule (mean
sentence 20 tokens, reuse budget 16).  A step is one decode step of the whole
batch: every sequence appends its new K/V row, then takes either a slow step
(dense attention with evidence, then the selector) or a fast step (sparse
attention), as the schedule says.

Headline (cold): R independent copies of the layer (own seeded K/V and
queries, same schedule) run each step in turn, so between two steps of one
copy the other copies stream more than the 256 MB Infinity Cache holds; the
K x R layer-steps are replayed from one HIP graph, value = B K R / time
(tokens/s of one layer), median of 3 replays.  The copies are scheduled as
the layers of a model would be: a copy's selection runs inside the next
copy's grids (sfi_decode_layer_step), so it completes before that copy's
next step; the same replay with every selection inside its own step call
(sfi_decode_step_select) is reported beside it, and so are the same K steps
of one copy alone (warm: its fast rows stay cached).

Per call: each call kind is timed with HIP events on the launch stream over
a region of R back-to-back launches on the R copies (cold), after a 1 GiB
read that evicts L2 and the Infinity Cache; the roofline record is the
dominant call's algorithmic bytes per launch / its average launch duration.
The CPU oracle's throughput on a bounded sample of the same workload is
reported as the baseline.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak of one MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama3_8b_layer_32k.json")
LEGS_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_long_context_legs.json")

# --record-calls: (workload, kind, algorithmic bytes) of every timed eager
# call in launch order, and a one-element fill kernel after each call
# (outside its events) that closes the call's dispatch segment for the
# counter reducer.
CALL_LOG = None
_MARK = None


def _mark_call(leg, kind, nbytes):
    if CALL_LOG is None:
        return
    _MARK.zero_()
    CALL_LOG.append([leg, kind, int(nbytes)])
METRIC = "decode attn tokens/s (slow+fast mix) at 32K/128K ctx; % HBM roofline/kernel"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(kind, n, cfg, k=None):
    """Bytes the method must move for one sequence-step (per layer); k
    overrides the configured list length (per-sequence k)."""
    Hkv, Hq, d = cfg.Hkv, cfg.Hq, cfg.d
    k = cfg.k if k is None else k
    if kind == "dense":
        return n * Hkv * 4 * d + Hq * d * 6
    if kind == "slow":
        return n * Hkv * 4 * d + Hq * d * 6 + n * Hkv * 8
    if kind == "select":
        return n * Hkv * 8 + k * Hkv * 4
    if kind == "fast":
        rows = min(cfg.n_sink, n) + min(cfg.window, n) + k
        return rows * Hkv * 4 * d + k * Hkv * 4 + Hq * d * 6
    if kind == "append":                 # the step's new K and V rows: read, then written to the cache
        return Hkv * 2 * d * 2 * 2
    if kind == "append_fused":           # the same rows written by the step call that reads them
        return Hkv * 2 * d * 2
    if kind.startswith("slow_window"):   # w rows: K and V, K again for the evidence
        w = int(kind[len("slow_window"):])
        return n * Hkv * 6 * d + w * Hq * d * 6 + n * Hkv * 8
    raise ValueError(kind)


def percall_list(slow, ctx, cfg, steps):
    """The eager per-call pass of the headline workload, in launch order:
    (kind, step, algorithmic bytes).  A step with both slow and fast
    sequences runs them co-launched ("step"), then the selector."""
    out = []
    ab = algorithmic_bytes("append_fused", 0, cfg)    # each call appends its sequences' rows
    for s in range(steps):
        lens = ctx + s + 1
        sl, fa = np.nonzero(slow[s])[0], np.nonzero(~slow[s])[0]
        sb = sum(algorithmic_bytes("slow", int(lens[b]), cfg) + ab for b in sl)
        fb = sum(algorithmic_bytes("fast", int(lens[b]), cfg) + ab for b in fa)
        selb = sum(algorithmic_bytes("select", int(lens[b]), cfg) for b in sl)
        if len(sl) and len(fa):
            out.append(("step", s, sb + fb))
        elif len(sl):
            out.append(("slow", s, sb))
        elif len(fa):
            out.append(("fast", s, fb))
        if len(sl):
            # the same step as one sfi_decode_step_select call (what the
            # graph replays; a step with every sequence slow is its own
            # kind), then the selector alone
            out.append(("step_select" if len(fa) else "slow_select", s, sb + fb + selb))
            out.append(("select", s, selb))
    return out


def traffic_from_counters(d, steps):
    """HBM bytes per call kind from two rocprofv3 counter runs of
    bench.py --no-graph --steps S --warmup 1 --no-cpu-baseline --calib-copy
      --record-calls d/fetch/calls.json
    (d/fetch with FETCH_SIZE, d/write with WRITE_SIZE).  The dispatch streams
    of the two runs are paired in order; FETCH_SIZE and WRITE_SIZE are scaled
    by what they read for the plain 256 MiB copy the run starts with.  Every
    timed eager call is the run of dispatches between its 1 GiB flush read
    (the last reduction before it) and the marker fill kernel after it, in
    the order of the recorded calls.  Writes the headline's summary beside the
    profiles (per kind), the long-context workloads' one (per workload and
    kind), and prints markdown tables."""
    import csv

    def load(which):
        rows = list(csv.DictReader(open(os.path.join(d, which, "bench_counter_collection.csv"))))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return rows
    F, Wr = load("fetch"), load("write")
    assert len(F) == len(Wr), (len(F), len(Wr))
    for a, b in zip(F, Wr):
        assert a["Kernel_Name"] == b["Kernel_Name"]
    # the runtime's buffer fills (torch's reduction output) belong to no call
    keep = [i for i, r in enumerate(F) if "fillBuffer" not in r["Kernel_Name"]]
    F, Wr = [F[i] for i in keep], [Wr[i] for i in keep]
    ci = next(i for i, r in enumerate(F) if "copyBuffer" in r["Kernel_Name"])
    copy_kib = (1 << 26) * 4 / 1024
    fs = copy_kib / float(F[ci]["Counter_Value"])
    ws = copy_kib / float(Wr[ci]["Counter_Value"])
    with open(os.path.join(d, "fetch", "calls.json")) as fh:
        calls = json.load(fh)
    segs, last_flush = [], None
    for i, r in enumerate(F):
        nm = r["Kernel_Name"]
        if "reduce_kernel" in nm:
            last_flush = i
        elif "FillFunctor" in nm and last_flush is not None:
            # a timed call: a 1 GiB flush read, then only library kernels
            lo = last_flush + 1
            big = float(F[last_flush]["Counter_Value"]) * fs > 512 * 1024
            if big and i > lo and all("sfi" in F[j]["Kernel_Name"] for j in range(lo, i)):
                segs.append((lo, i))
            last_flush = None
    assert len(segs) == len(calls), (len(segs), len(calls))
    flush_gib = sorted(set(round(float(F[lo - 1]["Counter_Value"]) * fs / 1048576, 3) for lo, _ in segs))
    tot = {}
    for (lo, hi), (leg, kind, alg) in zip(segs, calls):
        assert hi > lo and all("sfi" in F[i]["Kernel_Name"] for i in range(lo, hi)), (leg, kind)
        fb = sum(float(F[i]["Counter_Value"]) for i in range(lo, hi)) * fs * 1024
        wb = sum(float(Wr[i]["Counter_Value"]) for i in range(lo, hi)) * ws * 1024
        t = tot.setdefault(leg, {}).setdefault(kind, [0.0, 0.0, 0, 0])
        t[0] += fb; t[1] += wb; t[2] += alg; t[3] += 1
    dd = os.path.relpath(d) if os.path.isabs(d) else d.rstrip("/")
    cmds = [f"rocprofv3 --pmc {c} --output-format csv -d {dd}/{w} -o bench -- python3 -u "
            f"bench.py --no-graph --steps {steps} --warmup 1 --no-cpu-baseline --calib-copy "
            f"--record-calls {dd}/{w}/calls.json" for c, w in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))]
    cal = {"copy_bytes": 1 << 28, "fetch_kib_read": float(F[ci]["Counter_Value"]),
           "write_kib_read": float(Wr[ci]["Counter_Value"]), "fetch_scale": round(fs, 4),
           "write_scale": round(ws, 4), "flush_reads_gib": flush_gib}

    def summary(per_kind):
        return ({k: round((v[0] + v[1]) / v[2], 4) for k, v in per_kind.items() if v[2] > 0},
                {k: {"calls": v[3], "fetch": int(v[0]), "write": int(v[1]), "algorithmic": int(v[2])}
                 for k, v in per_kind.items()})
    from dynamic_sparse_kv_amd import workload as W
    cfg = W.CONFIGS["llama3-8b-layer-32k"].replace(steps=steps)
    ratio, totals = summary(tot.get("headline", {}))
    res = {"workload": f"{cfg.name} (B={cfg.B}, Hq={cfg.Hq}, Hkv={cfg.Hkv}, d={cfg.d}, ctx {cfg.ctx}, "
                       f"{cfg.n_sink}+{cfg.window}+{cfg.k}, lambda {cfg.lam}), eager pass over decode steps "
                       f"0..{steps - 1}",
           "commands": cmds, "calibration": cal, "ratio": ratio, "totals_bytes": totals,
           "kernel_source_sha256": kernel_source_hash()}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(res, fh, indent=1)
    legs = {}
    for leg, per_kind in tot.items():
        if leg == "headline":
            continue
        r_, t_ = summary(per_kind)
        legs[leg] = {"ratio": r_, "totals_bytes": t_}
    if legs:
        with open(LEGS_TRAFFIC_FILE, "w") as fh:
            json.dump({"commands": cmds, "calibration": cal, "legs": legs,
                       "kernel_source_sha256": kernel_source_hash()}, fh, indent=1)
    print(f"calibration: FETCH_SIZE {F[ci]['Counter_Value']} KiB, WRITE_SIZE {Wr[ci]['Counter_Value']} KiB "
          f"for a 256 MiB copy -> scales {fs:.4f}, {ws:.4f}; flush reads {flush_gib} GiB")
    print("| workload | call | calls | fetch MB | write MB | algorithmic MB | measured / algorithmic |")
    print("|---|---|---|---|---|---|---|")
    for leg, per_kind in tot.items():
        for k, v in per_kind.items():
            ratio_s = f"{(v[0] + v[1]) / v[2]:.4f}" if v[2] > 0 else "-"
            print(f"| {leg} | {k} | {v[3]} | {v[0] / 1e6:.2f} | {v[1] / 1e6:.2f} | {v[2] / 1e6:.2f} | {ratio_s} |")


def _short_kernel(name):
    import re
    n = name.replace("(anonymous namespace)::", "").replace("sfi::", "").replace("void ", "")
    return re.sub(r"\(.*", "", n)


def kernel_stats(d):
    """Markdown summary of a rocprofv3 --kernel-trace run (d/bench_kernel_trace.csv):
    per kernel, every launch, then the launches of the graph replays (runs
    of at least 300 library launches under 30 us apart)."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "bench_kernel_trace.csv"))))
    ks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short_kernel(r["Kernel_Name"]))
                for r in rows)

    def table(items, title):
        per = {}
        for s0, e0, n in items:
            per.setdefault(n, []).append((e0 - s0) / 1000.0)
        tot = sum(sum(v) for v in per.values())
        print(f"{title}\n")
        print("| kernel | launches | avg us | median us | min us | max us | total ms | % of kernel time |")
        print("|---|---|---|---|---|---|---|---|")
        for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            if sum(v) < 0.001 * tot:
                continue
            print(f"| `{n[:80]}` | {len(v)} | {np.mean(v):.2f} | {np.median(v):.2f} | {min(v):.2f} | "
                  f"{max(v):.2f} | {sum(v) / 1e3:.3f} | {100 * sum(v) / tot:.2f} |")
        print()
    table(ks, "All launches")
    bursts, cur = [], [ks[0]]
    for k in ks[1:]:
        if k[0] - cur[-1][1] < 30000:
            cur.append(k)
        else:
            bursts.append(cur)
            cur = [k]
    bursts.append(cur)
    runs = [x for x in bursts if len(x) >= 300 and all("at::" not in k[2] for k in x)]
    if runs:
        span = sum((b[-1][1] - b[0][0]) for b in runs) / 1000.0
        busy = sum(e0 - s0 for b in runs for s0, e0, _ in b) / 1000.0
        table([k for b in runs for k in b],
              f"Graph replays: {sum(len(b) for b in runs)} launches in {len(runs)} back-to-back runs, "
              f"{span:.1f} us from first start to last end, {busy:.1f} us inside kernels")


def mfma_stats(d):
    """MFMA use per kernel from one rocprofv3 --pmc run of
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
    (d/bench_counter_collection.csv): bf16 MFMA flops per launch (MOPS x
    512), the MFMA busy share of the SIMDs over the dispatch's active cycles
    (busy / (active / 8 XCDs x 1024 SIMDs)), and the flop rate over those
    cycles at 2.4 GHz."""
    import csv
    per = {}
    for r in csv.DictReader(open(os.path.join(d, "bench_counter_collection.csv"))):
        key = (int(r["Dispatch_Id"]), _short_kernel(r["Kernel_Name"]))
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    agg = {}
    for (_, n), c in per.items():
        a = agg.setdefault(n, [0, 0.0, 0.0, 0.0])
        a[0] += 1
        a[1] += c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        a[2] += c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        a[3] += c.get("GRBM_GUI_ACTIVE", 0.0) / 8
    print("| kernel | launches | bf16 MFMA GFLOP per launch | active cycles per launch | MFMA busy (of SIMD cycles) "
          "| TFLOP/s over active cycles |")
    print("|---|---|---|---|---|---|")
    for n, (cnt, fl, busy, act) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        if fl <= 0:
            continue
        util = busy / (act * 1024) if act > 0 else float("nan")
        tf = fl / (act / 2.4e9) / 1e12 if act > 0 else float("nan")
        print(f"| `{n[:70]}` | {cnt} | {fl / cnt / 1e9:.2f} | {act / cnt:.0f} | {util:.4f} | {tf:.1f} |")


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


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(cfg, K, V, q_host, slow, ctx, budget_s=15.0):
    """The oracle, untuned, on a bounded sample: the slow and fast steps of
    sequences 0, 1, ... in step order until about budget_s of CPU work; the
    per-kind mean time x the run's slow fraction -> tokens/s."""
    from oracle import sfi_oracle as O
    from dynamic_sparse_kv_amd.workload import bf16_bits

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    t_slow, t_fast = [], []
    t_start = time.perf_counter()
    seqs = 0
    for b in range(slow.shape[1]):
        n_max = int(ctx[b]) + slow.shape[0]
        Kb = bf16_bits(K[b, :, :n_max])
        Vb = bf16_bits(V[b, :, :n_max])
        qb = bf16_bits(q_host[:, b])
        sel = None
        seqs += 1
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
        if time.perf_counter() - t_start > budget_s:
            break
    frac = float(slow.mean())
    per_tok = frac * np.mean(t_slow) + (1 - frac) * np.mean(t_fast)
    return {
        "value": round(1.0 / per_tok, 3),
        "unit": "tokens/s",
        "cores": int(cores),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"sequences 0..{seqs - 1} of copy 0 of the same workload in step order: {len(t_slow)} slow + "
                   f"{len(t_fast)} fast steps (NumPy fp64), mean per kind weighted by the run's slow "
                   f"fraction {frac:.4f}; {time.perf_counter() - t_start:.1f} s of CPU work"),
        "slow_step_s": round(float(np.mean(t_slow)), 4),
        "fast_step_s": round(float(np.mean(t_fast)), 4),
    }


def _graph_time(fn, side, stream, reps=3):
    """Capture fn(side) into one HIP graph, replay once untimed, then time
    `reps` replays; returns (median seconds, list of seconds, graph)."""
    import torch
    g = torch.cuda.CUDAGraph()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), ts, g


def host_stall_mask(ts):
    """Samples to keep: a region whose time exceeds 4x the median of its kind
    (every region of a kind has the same composition) waited for the host
    (the flush read ran out before the region was enqueued, e.g. a
    garbage-collection pause), so the GPU sat idle inside it.  Such samples
    are dropped from the per-call averages and counted."""
    ts = np.asarray(ts, dtype=np.float64)
    return ts <= 4.0 * float(np.median(ts))


class RegionTimer:
    """HIP events on the launch stream around a region of back-to-back
    launches of one call kind on different data (the R copies of a layer,
    the layers of a stack), after a 1 GiB read that evicts L2 and the
    Infinity Cache and keeps the stream busy while the host enqueues the
    region.  A launch's duration is the region's time / its launches.  (A
    region replayed from a HIP graph instead measured a few microseconds
    more per replay: the graph launch's own start-up.)"""

    def __init__(self, dev, stream, leg):
        import torch
        self.torch = torch
        self.flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.stream = stream
        self.leg = leg
        self.ev = []

    def __call__(self, kind, fns, nbytes, flops=0.0):
        """fns: the region's launches, each called with the stream to issue
        on; nbytes / flops: per launch (mean)."""
        t = self.torch
        self.flush.sum()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for fn in fns:
            fn(self.stream)
        e1.record(self.stream)
        _mark_call(self.leg, kind, nbytes * len(fns))
        self.ev.append((kind, e0, e1, len(fns), nbytes, flops))

    def summary(self):
        self.torch.cuda.synchronize()
        agg = {}
        for kind, a, b, nl, nbytes, flops in self.ev:
            d = agg.setdefault(kind, [[], [], [], []])
            d[0].append(a.elapsed_time(b) * 1e-3 / nl)
            d[1].append(nbytes)
            d[2].append(flops)
            d[3].append(nl)
        out = {}
        for kind, (ts, bs, fs, nls) in agg.items():
            keep = host_stall_mask(ts)
            ts = np.asarray(ts)[keep]
            bs = np.asarray(bs)[keep]
            fs = np.asarray(fs)[keep]
            t = float(np.mean(ts))
            by = float(np.mean(bs))
            rec = {"launches": int(np.asarray(nls)[keep].sum()), "regions": int(keep.sum()),
                   "host_stalls_dropped": int((~keep).sum()), "avg_us": round(t * 1e6, 2),
                   "total_ms": round(float(np.sum(ts * np.asarray(nls)[keep])) * 1e3, 3),
                   "alg_bytes_per_launch": int(by), "alg_GBps": round(by / t / 1e9, 1),
                   "frac_of_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
            if any(fs):
                fl = float(np.mean(fs))
                rec["TFLOPs"] = round(fl / t / 1e12, 2)
                rec["mfma_util_bf16"] = round(fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
            out[kind] = rec
        del self.flush
        return out


def _step_bytes(plan, s, cfg, kseq=None):
    """Algorithmic bytes of step s: (slow share, fast share, selections); the
    shares include the fused append of their sequences' rows."""
    lens = plan.seq_len_host[s]
    sl_b, fa_b = np.nonzero(plan.slow[s])[0], np.nonzero(~plan.slow[s])[0]
    k = (lambda b: None) if kseq is None else (lambda b: int(kseq[s, b]))
    ab = algorithmic_bytes("append_fused", 0, cfg)
    sb = sum(algorithmic_bytes("slow", int(lens[b]), cfg) + ab for b in sl_b)
    fb = sum(algorithmic_bytes("fast", int(lens[b]), cfg, k=k(b)) + ab for b in fa_b)
    selb = sum(algorithmic_bytes("select", int(lens[b]), cfg, k=k(b)) for b in sl_b)
    return sb, fb, selb


def leg_stack128k(timed_steps=24, dense_steps=4):
    """32 attention layers of the Llama-3-8B shape at 128K context, B=4,
    4+256+4096, lambda 0.2, sentence schedule shared by the layers; one token
    passes all 32 layers (independent seeded KV and queries per layer), each
    layer appending its new K/V row first."""
    import torch
    from dynamic_sparse_kv_amd import sfi
    from dynamic_sparse_kv_amd import workload as W
    from dynamic_sparse_kv_amd.runner import DecodePlan, SFIDecoder
    dev = "cuda"
    steps = timed_steps + 1
    cfg = W.CONFIGS["stack32-128k"].replace(steps=steps)
    ctx = W.context_lengths(cfg)
    starts = W.sentence_starts(cfg)
    slow = sfi.sfi_schedule(starts, cfg.budget).astype(bool)
    plan = DecodePlan(slow, ctx, dev)
    max_len = int(ctx.max()) + steps
    decs, qs, nks = [], [], []
    _log(f"[bench] stack32-128k: generating {cfg.layers} layers")
    for layer in range(cfg.layers):
        K, V = W.make_kv(cfg, layer=layer, device=dev)
        nks.append(W.take_decode_rows(K, V, ctx, steps))
        qs.append(W.make_queries(cfg, starts, layer=layer).to(dev))
        decs.append(SFIDecoder(K, V, cfg.Hq, max_len, n_sink=cfg.n_sink, window=cfg.window,
                               k=cfg.k, lam=cfg.lam, norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau))
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for layer in range(cfg.layers):      # step 0: every sequence slow (first selection)
        decs[layer].step(plan, 0, qs[layer], stream, new_kv=nks[layer])
    torch.cuda.synchronize()

    def run(st):
        for s in range(1, steps):
            for layer in range(cfg.layers):
                decs[layer].step(plan, s, qs[layer], st, new_kv=nks[layer])

    def run_pipe(st):
        # each layer's selection runs inside the next layer's grids (the last
        # layer's inside the next step's first layer), one flush at the end
        pend = None
        for s in range(1, steps):
            for layer in range(cfg.layers):
                pend = decs[layer].layer_step(plan, s, qs[layer], pending=pend, stream=st, new_kv=nks[layer])
        sfi.sfi_run_deferred(pend, st)

    _log("[bench] stack32-128k: timing graph replay (selections pipelined across layers)")
    t_total, ts_pipe, g = _graph_time(run_pipe, side, stream)
    del g
    value = cfg.B * timed_steps / t_total
    _log("[bench] stack32-128k: timing graph replay (selection after each layer)")
    t_layer, _, g = _graph_time(run, side, stream)
    del g

    timer = RegionTimer(dev, stream, "stack32-128k")
    L = range(cfg.layers)
    for s in range(1, steps):
        ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
        sids, fids = plan.slow_list(s), plan.fast_list(s)
        sb, fb, selb = _step_bytes(plan, s, cfg)
        sl = plan.seq_len[s]
        nr = [(nks[l][0][s], nks[l][1][s]) for l in L]
        if ns and nf:
            timer("step", [lambda st, d=decs[l], q=qs[l][s], r=nr[l]: d.co_step(q, sl, sids, ns, fids, nf, st,
                                                                                select=False, new_rows=r)
                           for l in L], sb + fb)
        elif ns:
            timer("slow", [lambda st, d=decs[l], q=qs[l][s], r=nr[l]: d.slow(q, sl, sids, ns, st, select=False,
                                                                             new_rows=r)
                           for l in L], sb)
        elif nf:
            timer("fast", [lambda st, d=decs[l], q=qs[l][s], r=nr[l]: d.fast(q, sl, fids, nf, st, new_rows=r)
                           for l in L], fb)
        if ns:
            timer("select", [lambda st, d=decs[l]: d.slow_select_only(sl, sids, ns, st) for l in L], selb)
    for s in range(1, 1 + dense_steps):
        db = sum(algorithmic_bytes("dense", int(n), cfg) for n in plan.seq_len_host[s])
        timer("dense", [lambda st, d=decs[l], q=qs[l][s]: d.dense(q, plan.seq_len[s], None, cfg.B, st)
                        for l in L], db)
    per_call = timer.summary()

    def run_dense(st):
        for s in range(1, 1 + dense_steps):
            for layer in range(cfg.layers):
                decs[layer].dense(qs[layer][s], plan.seq_len[s], None, cfg.B, st)

    _log("[bench] stack32-128k: dense comparator")
    t_dense, _, g = _graph_time(run_dense, side, stream)
    del g
    dense_tps = cfg.B * dense_steps / t_dense
    res = {"workload": f"{cfg.name}: {cfg.layers} layers, B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d}, "
                       f"ctx {cfg.ctx}, fast state {cfg.n_sink}+{cfg.window}+{cfg.k}, lambda {cfg.lam}, "
                       f"{timed_steps} decode steps after a first all-slow step, each layer appending its row",
           "tokens_per_s": round(value, 1), "ms_per_step": round(t_total / timed_steps * 1e3, 4),
           "replays_s": [round(x, 6) for x in ts_pipe],
           "tokens_per_s_selection_per_layer": round(cfg.B * timed_steps / t_layer, 1),
           "slow_fraction": round(float(plan.slow[1:].mean()), 4),
           "timing": "hip graph replay, one stream, median of 3; tokens_per_s with each layer's selection run "
                     "inside the next layer's grids (sfi_decode_layer_step), tokens_per_s_selection_per_layer "
                     "with it after each layer (sfi_decode_step_select); per_call: regions of the 32 layers' "
                     "launches (cold), hip events",
           "per_call": per_call, "dense_tokens_per_s": round(dense_tps, 2),
           "speedup_vs_dense": round(value / dense_tps, 2)}
    del decs, qs, nks
    torch.cuda.empty_cache()
    return res


def leg_vegas64k(iters=12):
    """Verification-guided selection at 64K context, B=16, T=8 verify rows:
    per iteration the T verified rows are appended, verify (all T rows,
    logits aggregated in-kernel), top-2048 of the aggregate per sequence, 7
    sparse draft steps (each appending its row); ALL rows and Collect-2-Query
    (first and last row) aggregates, and the raw-logit emission mode."""
    import torch
    from dynamic_sparse_kv_amd import workload as W
    from dynamic_sparse_kv_amd.runner import VegasDecoder
    dev = "cuda"
    cfg = W.CONFIGS["vegas-64k"].replace(steps=iters)
    T = cfg.vegas_T
    ctx_a = W.context_lengths(cfg)
    ctx = int(ctx_a.max())
    _log("[bench] vegas-64k: generating")
    K, V = W.make_kv(cfg, device=dev)
    cap = K.shape[2]
    kn, vn = W.take_decode_rows(K, V, ctx_a, iters + 1, rows_per_step=T)   # [iters+1][B][T][Hkv][d]
    # a draft's own row: row j - 1 of the next iteration's verified rows
    dk = [[kn[it + 1][:, j - 1:j].contiguous() for j in range(1, T)] for it in range(iters)]
    dv = [[vn[it + 1][:, j - 1:j].contiguous() for j in range(1, T)] for it in range(iters)]
    qpos = W.make_vegas_queries(cfg).to(dev)           # [positions][B][Hq][d]
    vd = VegasDecoder(K, V, cfg.Hq, cap, T, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k, keep_raw=True)
    q_rows = [qpos[it * T: it * T + T].permute(1, 0, 2, 3).contiguous() for it in range(iters)]
    seq_v = [torch.full((cfg.B,), ctx + T * (it + 1), dtype=torch.int32, device=dev) for it in range(iters)]
    seq_d = [[torch.full((cfg.B,), ctx + T * (it + 1) + j, dtype=torch.int32, device=dev)
              for j in range(1, T)] for it in range(iters)]
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    masks = {"all": (1 << T) - 1, "collect2": 1 | (1 << (T - 1))}

    def iteration(it, mask, st, raw=False):
        vd.append(kn[it], vn[it], seq_v[it], stream=st)
        vd.verify(q_rows[it], seq_v[it], mask, stream=st, raw=raw)
        vd.select(seq_v[it], stream=st)
        for j in range(1, T):
            vd.draft(qpos[it * T + T + j - 1], seq_d[it][j - 1], stream=st, new_rows=(dk[it][j - 1], dv[it][j - 1]))

    res = {"workload": f"{cfg.name}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d}, ctx {ctx}, "
                       f"T={T} verify rows, top-{cfg.k} of the aggregated logits + {cfg.n_sink} sinks + "
                       f"{cfg.window} window, {T - 1} drafts per iteration, {iters} iterations; rows appended",
           "tokens_per_iteration": f"{T} per sequence (all drafts accepted)"}
    for name, mask in masks.items():
        iteration(0, mask, stream)
        torch.cuda.synchronize()
        t_total, _, g = _graph_time(lambda st: [iteration(it, mask, st) for it in range(iters)], side, stream)
        del g
        res[f"tokens_per_s_{name}"] = round(cfg.B * T * iters / t_total, 1)
        res[f"ms_per_iteration_{name}"] = round(t_total / iters * 1e3, 4)
    timer = RegionTimer(dev, stream, "vegas-64k")
    d, Hq, Hkv = cfg.d, cfg.Hq, cfg.Hkv
    for it in range(min(iters, 4)):
        n = ctx + T * (it + 1)
        vbytes = cfg.B * (n * Hkv * 4 * d + (n - T) * 4 + T * Hq * d * 6)
        vflops = cfg.B * 4.0 * d * T * Hq * n
        for name, mask in masks.items():
            timer(f"verify_{name}", [lambda st: vd.verify(q_rows[it], seq_v[it], mask, stream=st)], vbytes, vflops)
            # raw-logit emission: the collected rows' pre-softmax logits written
            # out and read back by the aggregation pass
            nrow = bin(mask).count("1")
            timer(f"verify_raw_{name}", [lambda st: vd.verify(q_rows[it], seq_v[it], mask, stream=st, raw=True)],
                  vbytes + 2 * cfg.B * nrow * Hq * (n - T) * 4, vflops)
        timer("select", [lambda st: vd.select(seq_v[it], stream=st)], cfg.B * ((n - T) * 4 + cfg.k * 4))
        for j in (1, T - 1):
            rows = cfg.n_sink + cfg.window + cfg.k
            timer("draft", [lambda st: vd.draft(qpos[it * T + T + j - 1], seq_d[it][j - 1], stream=st,
                                                new_rows=(dk[it][j - 1], dv[it][j - 1]))],
                  cfg.B * (rows * Hkv * 4 * d + cfg.k * 4 + Hq * d * 6 + algorithmic_bytes("append_fused", 0, cfg)))
    res["per_call"] = timer.summary()
    del vd, K, V, qpos, q_rows
    torch.cuda.empty_cache()
    return res


def leg_ragged_paged(timed_steps=32, dense_steps=4):
    """Ragged long-reasoning batch: B=32 sequences, contexts log-uniform in
    [8K, 128K], paged bf16 KV in 16-token pages (shuffled pool), Hq=40
    Hkv=8 d=128, 4+256+min(4096, n/16) keys, lambda 0.3, each sequence
    slow with probability 1/20 per step (step 0 slow), each step appending
    its rows.  Graph: slow and fast shares of a step co-launched in one grid
    on one stream.  Two streams: slow steps and selector on one stream, fast
    steps on another, co-running (eager, hip events around the run).  Every
    call carries the host row-count hints, so each sequence gets the
    workgroups of its own length."""
    import torch
    from dynamic_sparse_kv_amd import sfi
    from dynamic_sparse_kv_amd import workload as W
    from dynamic_sparse_kv_amd.runner import DecodePlan, SFIDecoder
    dev = "cuda"
    steps = timed_steps + 1
    cfg = W.CONFIGS["ragged-paged-8k-128k"].replace(steps=steps)
    ctx = W.context_lengths(cfg)
    caps = ctx + cfg.growth()
    table, npages = W.page_table(cfg, caps)
    _log(f"[bench] ragged-paged: generating {npages} pages")
    Kp, Vp = W.make_paged_kv(cfg, table, npages, caps, device=dev)
    nk = W.take_decode_rows(Kp, Vp, ctx, steps, table=table)
    tab = torch.from_numpy(table).to(dev)
    starts = W.sentence_starts(cfg)
    slow = sfi.sfi_schedule(starts, -1).astype(bool)
    plan = DecodePlan(slow, ctx, dev, k_cap=cfg.k, k_div=cfg.k_div)
    q = W.make_queries(cfg, starts).to(dev)
    max_len = int(ctx.max()) + steps
    dec = SFIDecoder(Kp, Vp, cfg.Hq, max_len, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k,
                     lam=cfg.lam, norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau, page_table=tab,
                     page_size=cfg.page_size)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    dec.step(plan, 0, q, stream, new_kv=nk)
    torch.cuda.synchronize()

    def run(st):
        for s in range(1, steps):
            dec.step(plan, s, q, st, new_kv=nk)

    _log("[bench] ragged-paged: timing graph replay")
    t_total, _, g = _graph_time(run, side, stream)
    del g
    value = cfg.B * timed_steps / t_total

    # eager runs timed with hip events: two streams (slow + selector on one,
    # fast on the other) and, for comparison, the one-stream co-launched step
    _log("[bench] ragged-paged: two-stream eager run")
    sb_stream = torch.cuda.Stream()
    outs = torch.zeros((steps, cfg.B, cfg.Hq, cfg.d), dtype=torch.float32, device=dev)

    def eager(fn):
        ts = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts[1:]))          # the first run is untimed
    t_two = eager(lambda: dec.run_two_streams(plan, q, 1, steps, stream, sb_stream, out_steps=outs, new_kv=nk))
    t_one = eager(lambda: [dec.step(plan, s, q, stream, new_kv=nk) for s in range(1, steps)])

    kseq = np.minimum(cfg.k, plan.seq_len_host // cfg.k_div)
    timer = RegionTimer(dev, stream, "ragged-paged")
    for s in range(1, steps):
        ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
        sids, fids = plan.slow_list(s), plan.fast_list(s)
        sb, fb, selb = _step_bytes(plan, s, cfg, kseq)
        ks = plan.k_seq[s]
        sl = plan.seq_len[s]
        nr = (nk[0][s], nk[1][s])
        lh = dec.hints(plan, s)
        if ns and nf:
            timer("step", [lambda st: dec.co_step(q[s], sl, sids, ns, fids, nf, st, select=False, new_rows=nr,
                                                  len_hints=lh)], sb + fb)
        elif ns:
            timer("slow", [lambda st: dec.slow(q[s], sl, sids, ns, st, select=False, new_rows=nr,
                                               len_hints=lh)], sb)
        elif nf:
            timer("fast", [lambda st: dec.fast(q[s], sl, fids, nf, st, new_rows=nr, len_hints=lh)], fb)
        if ns:
            timer("select", [lambda st: dec.slow_select_only(sl, sids, ns, st, k_seq=ks)], selb)
    for s in range(1, 1 + dense_steps):
        db = sum(algorithmic_bytes("dense", int(n), cfg) for n in plan.seq_len_host[s])
        timer("dense", [lambda st: dec.dense(q[s], plan.seq_len[s], None, cfg.B, st,
                                             len_hints=plan.seq_len_host[s])], db)
    per_call = timer.summary()

    def run_dense(st):
        for s in range(1, 1 + dense_steps):
            dec.dense(q[s], plan.seq_len[s], None, cfg.B, st, len_hints=plan.seq_len_host[s])

    t_dense, _, g = _graph_time(run_dense, side, stream)
    del g
    dense_tps = cfg.B * dense_steps / t_dense
    res = {"workload": f"{cfg.name}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d}, ctx log-uniform in "
                       f"[{cfg.ragged_min}, {cfg.ctx}] (mean {int(ctx.mean())}), paged {cfg.page_size}-token "
                       f"pages ({npages} in a shuffled pool), fast state {cfg.n_sink}+{cfg.window}+"
                       f"min({cfg.k}, n/{cfg.k_div}), lambda {cfg.lam}, slow probability {cfg.slow_prob:.3f}, "
                       f"{timed_steps} steps after a first all-slow step, rows appended",
           "tokens_per_s": round(value, 1), "ms_per_step": round(t_total / timed_steps * 1e3, 4),
           "tokens_per_s_two_streams": round(cfg.B * timed_steps / t_two, 1),
           "tokens_per_s_one_stream_eager": round(cfg.B * timed_steps / t_one, 1),
           "slow_fraction": round(float(plan.slow[1:].mean()), 4),
           "timing": "tokens_per_s: hip graph replay, one stream (slow and fast shares co-launched in one grid), "
                     "median of 3; tokens_per_s_two_streams: eager, slow steps + selector on one stream and "
                     "fast steps on another, hip events around the run, median of 3; "
                     "tokens_per_s_one_stream_eager: the graph's calls issued eagerly; per_call: eager, cold",
           "per_call": per_call, "dense_tokens_per_s": round(dense_tps, 1),
           "speedup_vs_dense": round(value / dense_tps, 2)}
    del dec, Kp, Vp, q, nk
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--replicas", type=int, default=8,
                    help="independent copies of the layer stepped in turn (cold headline)")
    ap.add_argument("--config", default="llama3-8b-layer-32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="stack32-128k,vegas-64k,ragged-paged",
                    help="extra workloads measured after the headline (comma list, or 'none')")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--traffic", metavar="DIR",
                    help="no GPU run: derive per-call HBM traffic from the two counter runs under DIR "
                         "(DIR/fetch, DIR/write; see traffic_from_counters) and rewrite the traffic summary")
    ap.add_argument("--record-calls", metavar="PATH",
                    help="write the timed eager calls (workload, kind, algorithmic bytes) to PATH as "
                         "json, each followed by a marker kernel, for the counter reducer")
    ap.add_argument("--kernel-stats", metavar="DIR",
                    help="no GPU run: markdown per-kernel summary of a rocprofv3 --kernel-trace csv run in DIR")
    ap.add_argument("--mfma-stats", metavar="DIR",
                    help="no GPU run: markdown MFMA summary of a rocprofv3 --pmc csv run in DIR (see mfma_stats)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (a known-size kernel "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.traffic:
        traffic_from_counters(args.traffic, args.steps)
        return
    if args.kernel_stats:
        kernel_stats(args.kernel_stats)
        return
    if args.mfma_stats:
        mfma_stats(args.mfma_stats)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from dynamic_sparse_kv_amd import sfi
    from dynamic_sparse_kv_amd import workload as W
    from dynamic_sparse_kv_amd.runner import DecodePlan, SFIDecoder, stats_prior_steps

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sfi.lib()
    dev = "cuda"
    global CALL_LOG, _MARK
    if args.record_calls:
        CALL_LOG = []
        _MARK = torch.zeros(1, dtype=torch.float32, device=dev)
    if args.calib_copy:
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = W.CONFIGS[args.config]
    K_steps, W_steps, R = args.steps, args.warmup, max(1, args.replicas)
    plan_steps = max(K_steps, W_steps, 1)
    cfg = cfg.replace(steps=plan_steps)

    _log(f"[bench] generating {cfg.name} inputs, {R} copies of the layer")
    ctx = W.context_lengths(cfg)
    starts = W.sentence_starts(cfg)
    slow = sfi.sfi_schedule(starts, cfg.budget).astype(bool)
    plan = DecodePlan(slow, ctx, dev)
    max_len = int(ctx.max()) + plan_steps
    reps = []
    for r in range(R):
        K, V = W.make_kv(cfg, layer=r, device=dev)
        nk = W.take_decode_rows(K, V, ctx, plan_steps)
        q_host = W.make_queries(cfg, starts, layer=r)
        dec = SFIDecoder(K, V, cfg.Hq, max_len, n_sink=cfg.n_sink, window=cfg.window, k=cfg.k,
                         lam=cfg.lam, norm_coef=cfg.norm_coef, pos_tau=cfg.pos_tau)
        reps.append({"K": K, "V": V, "nk": nk, "q_host": q_host, "q": q_host.to(dev), "dec": dec})
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()

    def run_steps(st, s0, s1, copies, pipelined=True):
        # The copies stand in for the layers of a model.  Pipelined (several
        # copies): each copy's selection runs inside the next copy's grids
        # (sfi_decode_layer_step), the last copy's inside the next step's
        # first copy, one flush at the end; every selection still completes
        # before its own copy's next step.  Otherwise each step call runs its
        # selection itself (sfi_decode_step_select).
        if pipelined and len(copies) > 1:
            pend = None
            for s in range(s0, s1):
                for rp in copies:
                    pend = rp["dec"].layer_step(plan, s, rp["q"], pending=pend, stream=st, new_kv=rp["nk"])
            sfi.sfi_run_deferred(pend, st)
            return
        for s in range(s0, s1):
            for rp in copies:
                rp["dec"].step(plan, s, rp["q"], st, new_kv=rp["nk"])

    _log(f"[bench] warmup {W_steps} steps")
    run_steps(stream, 0, W_steps, reps)
    torch.cuda.synchronize()

    # ---- headline: K steps x R copies replayed from one HIP graph (cold) ----
    use_graph = not args.no_graph
    warm_tps = inline_tps = None
    if use_graph:
        _log("[bench] timing graph replays (cold: copies in turn)")
        t_total, ts_cold, g = _graph_time(lambda st: run_steps(st, 0, K_steps, reps), side, stream)
        del g
        _log("[bench] timing graph replays (cold, each copy's selection in its own step call)")
        t_inline, _, g = _graph_time(lambda st: run_steps(st, 0, K_steps, reps, pipelined=False), side, stream)
        del g
        inline_tps = cfg.B * K_steps * R / t_inline
        _log("[bench] timing graph replays (warm: one copy)")
        t_warm, ts_warm, g = _graph_time(lambda st: run_steps(st, 0, K_steps, reps[:1]), side, stream)
        del g
        warm_tps = cfg.B * K_steps / t_warm
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(stream, 0, K_steps, reps)
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t0
        ts_cold = [t_total]
    value = cfg.B * K_steps * R / t_total

    # ---- per call: regions of R launches on the R copies (cold) -------------
    _log("[bench] per-call timing pass")
    timer = RegionTimer(dev, stream, "headline")
    decs = [rp["dec"] for rp in reps]
    # the combined calls form their prior from the key-norm statistics where
    # the run does (the statistics' values at this point are the run's end
    # state: the work is the same, the selections are not the run's)
    use_st = stats_prior_steps(plan)
    for kind, s, nbytes in percall_list(plan.slow, ctx, cfg, K_steps):
        ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
        sl = plan.seq_len[s]
        sids, fids = plan.slow_list(s), plan.fast_list(s)
        # every step call appends its sequences' rows (fused append), as in the run
        mk = {"step": lambda d, q, st, r: d.co_step(q, sl, sids, ns, fids, nf, st, select=False, new_rows=r),
              "slow": lambda d, q, st, r: d.slow(q, sl, sids, ns, st, select=False, new_rows=r),
              "fast": lambda d, q, st, r: d.fast(q, sl, fids, nf, st, new_rows=r),
              "select": lambda d, q, st, r: d.slow_select_only(sl, sids, ns, st),
              # informational: not a roofline candidate (its selector part is latency-bound)
              "step_select": lambda d, q, st, r: d.step_select(q, sl, sids, ns, fids, nf, st, new_rows=r,
                                                               use_stats=bool(use_st[s])),
              "slow_select": lambda d, q, st, r: d.step_select(q, sl, sids, ns, fids, nf, st, new_rows=r,
                                                               use_stats=bool(use_st[s]))}[kind]
        timer(kind, [lambda st, d=rp["dec"], q=rp["q"][s], r=(rp["nk"][0][s], rp["nk"][1][s]): mk(d, q, st, r)
                     for rp in reps], nbytes)
    # The combined call again for the same slow steps, with Soft-NMS (radius
    # 4, alpha 0.5) and cross-head exclusivity (beta 0.5) on: the cost of the
    # score refinements (informational; the pages give no constants, so the
    # headline runs without them).  Last, since it replaces the selections.
    for kind, s, nbytes in percall_list(plan.slow, ctx, cfg, K_steps):
        if kind != "step_select":     # the mixed steps (every sequence slow is timed above)
            continue
        ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
        sl = plan.seq_len[s]
        sids, fids = plan.slow_list(s), plan.fast_list(s)

        def refined(d, q, st):
            d.params.nms_radius, d.params.nms_alpha, d.params.excl_beta = 4, 0.5, 0.5
            try:
                d.step_select(q, sl, sids, ns, fids, nf, st)
            finally:
                d.params.nms_radius, d.params.nms_alpha, d.params.excl_beta = 0, 0.0, 0.0
        timer("step_select_refined", [lambda st, d=rp["dec"], q=rp["q"][s]: refined(d, q, st) for rp in reps], nbytes)
    # Every sequence slow at once (the full slow step and the dense
    # comparator's call), and the observation-window slow step over the last
    # 8 queries, for every sequence (informational).
    wq = 8
    s_w = min(plan_steps, wq) - 1
    sl_w = plan.seq_len[s_w]
    lens_w = plan.seq_len_host[s_w]
    timer("slow_all", [lambda st, d=rp["dec"], q=rp["q"][s_w]: d.slow(q, sl_w, None, cfg.B, st, select=False)
                       for rp in reps], sum(algorithmic_bytes("slow", int(n), cfg) for n in lens_w))
    timer("dense", [lambda st, d=rp["dec"], q=rp["q"][s_w]: d.dense(q, sl_w, None, cfg.B, st) for rp in reps],
          sum(algorithmic_bytes("dense", int(n), cfg) for n in lens_w))
    if plan_steps >= wq:
        q_wins = [rp["q"][s_w - wq + 1:s_w + 1].permute(1, 0, 2, 3).contiguous() for rp in reps]
        out_w = torch.empty((cfg.B, wq, cfg.Hq, cfg.d), dtype=torch.float32, device=dev)
        ws_wb = sfi.sfi_slow_window_workspace_bytes(decs[0].kv, wq)
        ws_w = torch.empty(ws_wb, dtype=torch.uint8, device=dev)

        def window(d, qw, st):
            d.kv.seq_len = sl_w.data_ptr()
            sfi.sfi_slow_step_window(d.kv, None, cfg.B, qw, wq, out_w, d.evidence, d.key_norm, d.ld, ws_w, ws_wb,
                                     st)
        window(decs[0], q_wins[0], stream)    # untimed first launch of the window kernels
        for _ in range(2):
            timer("slow_window8", [lambda st, d=d, qw=qw: window(d, qw, st) for d, qw in zip(decs, q_wins)],
                  sum(algorithmic_bytes("slow_window8", int(n), cfg) for n in lens_w))
    per_call = timer.summary()
    # the roofline record is for the HBM-streaming attention calls of the
    # schedule; the selector (a few MB per call, latency-bound) and the
    # combined call are reported in per_call only
    dom = max((k_ for k_ in per_call if k_ in ("step", "slow", "fast")), key=lambda k_: per_call[k_]["total_ms"])
    dc = per_call[dom]
    achieved = dc["alg_GBps"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, dc["alg_bytes_per_launch"]),
                "call": dom, "avg_launch_us": dc["avg_us"], "alg_bytes_per_launch": dc["alg_bytes_per_launch"],
                "kernel": {"step": "sfi_decode_step: co-launched slow + fast partial kernel and finalize kernel",
                           "slow": "sfi_slow_step: split-K partial + finalize kernels",
                           "fast": "sfi_fast_step: gather partial + finalize kernels"}[dom]}

    # ---- all-dense comparator: every sequence dense every step (cold) -------
    _log("[bench] dense comparator")
    n_dense = min(K_steps, 8)
    if use_graph:
        t_d, _, g = _graph_time(lambda st: [rp["dec"].dense(rp["q"][s], plan.seq_len[s], None, cfg.B, st)
                                            for s in range(n_dense) for rp in reps], side, stream)
        del g
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(n_dense):
            for rp in reps:
                rp["dec"].dense(rp["q"][s], plan.seq_len[s], None, cfg.B, stream)
        torch.cuda.synchronize()
        t_d = time.perf_counter() - t0
    dense_tps = cfg.B * n_dense * R / t_d

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": round(t_total / (K_steps * R) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one attention layer, B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} "
                               f"d={cfg.d}, ctx {cfg.ctx}, fast state {cfg.n_sink}+{cfg.window}+{cfg.k}, "
                               f"lambda {cfg.lam}, {K_steps} decode steps (each appends its K/V row)",
                   "global_batch": cfg.B, "seq_len": cfg.ctx, "parallelism": "none (1 GPU)",
                   "slow_fraction": round(float(plan.slow[:K_steps].mean()), 4),
                   "copies": R,
                   "timing": ("hip graph replay, one stream, median of 3 replays; cold: the step's "
                              f"layer-steps of {R} independent copies of the layer run in turn, value = "
                              "tokens/s of one layer" if use_graph else "eager, one stream") +
                             "; the copies are scheduled as the layers of a model: each copy's selection "
                             "runs inside the next copy's grids (sfi_decode_layer_step); "
                             "tokens_per_s_selection_per_copy: each step with slow sequences is one "
                             "sfi_decode_step_select call that runs its own selection"},
        "roofline": roofline,
        "warm_tokens_per_s": None if warm_tps is None else round(warm_tps, 1),
        "tokens_per_s_selection_per_copy": None if inline_tps is None else round(inline_tps, 1),
        "replays_s": [round(x, 6) for x in ts_cold],
        "per_call": per_call,
        "dense_tokens_per_s": round(dense_tps, 1),
        "fast_vs_dense_speedup": round(value / dense_tps, 2),
    }
    if not args.no_cpu_baseline:
        _log("[bench] cpu baseline (oracle)")
        rp = reps[0]
        result["cpu_baseline"] = cpu_baseline(cfg, rp["K"], rp["V"], rp["q_host"], slow[:K_steps], ctx)
    legs = [x for x in args.legs.split(",") if x and x != "none"]
    if legs:
        del reps, decs
        torch.cuda.empty_cache()
        result["legs"] = {}
        for leg in legs:
            fn = {"stack32-128k": leg_stack128k, "vegas-64k": leg_vegas64k,
                  "ragged-paged": leg_ragged_paged}[leg]
            result["legs"][leg] = fn()
    print(json.dumps(result), flush=True)
    if CALL_LOG is not None:
        with open(args.record_calls, "w") as fh:
            json.dump(CALL_LOG, fh)


if __name__ == "__main__":
    main()
