#!/usr/bin/env python3
"""Throughput of the causal lightning indexer and its group-shared (PIVOT) variant on one MI355X.

By default every specified workload runs in this one process and ONE JSON
line is printed.  Its headline is the largest single-GPU workload: PIVOT-Refine
at L = 262144 with FP8 queries and keys (groups of 128 consecutive queries, a
shared proxy scan to 8192 candidates, each member's own re-score and top-2048),
one step = proxy build + proxy scan + candidate select + gathered re-score +
per-query select ("PIVOT: Efficient Query-Group Indexing for Token-Level
Sparse Attention", Abstract).  The same workload's dense scan (the full-scan
baseline on the same inputs), PIVOT-Reuse, and PIVOT-Refine at the cheapest
(group size, budget) of a sweep that reached a recall of 0.99 are timed
beside it as legs, and the other four workloads (the 1024-token float32 and 32K-token bfloat16 dense
prefills, the 8 x 2 decode step over 131072 FP8 keys with its decode grouping,
and PIVOT-Refine at 131072 bfloat16 tokens) follow as sub-records.

For every leg: milliseconds per step (wall clock over the timed steps, inputs
resident in HBM), pairs scored per second (all heads of a causal (query, key)
pair count once; a grouped leg counts the pairs it actually scores - proxy
plus re-score - and also reports dense pairs divided by its time), top-k
queries per second, the per-kernel times of the same steps (HIP events the
library records on the launch stream, in a second run so that the events stay
out of the step time), the roofline of the leg's dominant kernel against that
kernel's own peak (MFMA for prefill scans at the dtype the MFMAs run in; HBM
for the decode scans), and for grouped legs the speedup over the dense leg
and the recall of the dense top-k over every query.  The CPU oracle is timed
on a bounded sample of each workload on this host.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexer query·key pairs scored/sec + top-k queries/sec; %MFMA / %HBM peak"
HEADLINE = "grouped_fp8_L262144_G128_C8192_k2048"
ORDER = ["prefill_f32_L1024_H16_d64_k128", "prefill_bf16_L32768_H64_d128_k2048",
         "decode_fp8k_B8_mtp2_n131072_H64_d128_k2048", "grouped_refine_bf16_L131072_G64_C8192_k2048",
         HEADLINE]

# PIVOT-Refine at the cheapest (group size, candidate budget) of a sweep on
# these inputs whose recall of the dense top-k, averaged over every query,
# reached 0.99 (262K fp8: G 32, C 16384 gave 0.996 where G 64, C 16384 gave
# 0.9897; 131K bf16: G 16, C 16384 gave 0.994 where G 32, C 16384 gave 0.984)
RECALL99 = {"grouped_fp8_L262144_G128_C8192_k2048": (32, 16384),
            "grouped_refine_bf16_L131072_G64_C8192_k2048": (16, 16384)}

# MI355X published dense peaks (no sparsity), TFLOP/s, and HBM3E GB/s.
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0

# sources of the kernels whose HBM traffic the committed PMC runs measured,
# and of the launcher that sets their launch shapes (chunking, grids)
KERNEL_SOURCES = ["sparse_attention_token_causal_amd/csrc/score.hip",
                  "sparse_attention_token_causal_amd/csrc/split.hip",
                  "sparse_attention_token_causal_amd/csrc/common.hpp",
                  "sparse_attention_token_causal_amd/csrc/kernels.hpp",
                  "sparse_attention_token_causal_amd/csrc/api.cpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernel_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(n_q, q_pos0):
    """Causal (query, key) pairs of one sequence: sum over t of pos(t) + 1."""
    first, last = q_pos0 + 1, q_pos0 + n_q
    return (first + last) * n_q // 2


def group_limits(wl, G):
    n_g = -(-wl.n_q // G)
    return [wl.q_pos0 + min((g + 1) * G, wl.n_q) - 1 for g in range(n_g)]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, leg):
    """HBM bytes per launch of a leg's dominant kernel from committed rocprofv3
    PMC runs, if they were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{workload}/{leg}")
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return None


def spread_order(n):
    """0..n-1 ordered so that every prefix is spread evenly (bisection), last element first."""
    order, seen, step = [n - 1], {n - 1}, n
    while step >= 1:
        for t in range(step // 2 if step > 1 else 0, n, max(step, 1)):
            if t not in seen:
                seen.add(t)
                order.append(t)
        if step == 1:
            break
        step //= 2
    return order


# ----------------------------------------------------------------------------
# legs: each returns a callable step and what one step computes


class Leg:
    def __init__(self, name, step, pairs, queries, kernel, bound, dtype, flops=0.0, hbm_bytes=0.0):
        self.name, self.step, self.pairs, self.queries = name, step, pairs, queries
        self.kernel, self.bound, self.dtype = kernel, bound, dtype
        self.flops, self.hbm_bytes = flops, hbm_bytes
        self.out = None  # the output of the last step on input set 0 (for recall)


def make_legs(S, wl, sets, dev, which):
    """Legs of one workload over the input sets (one set, or four rotating key
    caches for decode so that the key reads come from HBM, not the 256 MB
    Infinity Cache)."""
    import torch
    inp = sets[0]
    H, d, B, K = wl.heads, wl.dim, wl.batch, wl.topk
    fl = 2 * H * d
    dtype = {"fp8": "fp8", "f32": "f32"}.get(wl.q_fmt, "bf16")
    decode = wl.n_q < wl.n_k
    kb = {"fp8": 1, "bf16": 2, "f32": 4}
    key_bytes = B * wl.n_k * (d * kb[wl.k_fmt] + (4 if wl.k_fmt == "fp8" else 0))
    dense_pairs = B * causal_pairs(wl.n_q, wl.q_pos0)
    a = lambda x: dict(q_scale=x["q_scale"], k_scale=x["k_scale"], q_pos0=wl.q_pos0)
    p0 = S.make_problem(inp["q"], inp["k"], inp["w"], **a(inp))
    legs = []
    it = [0]

    def rot():
        i = it[0] % len(sets)
        it[0] += 1
        return i

    if "dense" in which:
        ws = torch.empty(S.workspace_bytes(p0, S.IDX_OP_SCORE_TOPK, topk=K), dtype=torch.uint8, device=dev)
        outs = [torch.empty((B, wl.n_q, K), dtype=torch.int32, device=dev) for _ in sets]
        leg = Leg("dense", None, dense_pairs, B * wl.n_q, "score", "hbm" if decode else "mfma", dtype,
                  flops=dense_pairs * fl,
                  hbm_bytes=key_bytes + B * wl.n_q * (H * d * kb[wl.q_fmt] + 4 * H + (4 if wl.q_fmt == "fp8" else 0)))

        def step_dense(leg=leg, ws=ws, outs=outs):
            i = rot()
            x = sets[i]
            S.score_topk(x["q"], x["k"], x["w"], K, workspace=ws, out=outs[i], **a(x))
            leg.out = outs[0]
        leg.step = step_dense
        legs.append(leg)

    for variant in ("refine", "reuse", "refine_r99"):
        if variant not in which or not wl.group or (variant == "refine_r99" and wl.name not in RECALL99):
            continue
        G, C = RECALL99[wl.name] if variant == "refine_r99" else (wl.group, wl.n_cand if variant == "refine" else K)
        lim = group_limits(wl, G)
        n_g = len(lim)
        proxy_pairs = B * sum(x + 1 for x in lim)
        refine_pairs = B * sum(min(G, wl.n_q - g * G) * min(C, lim[g] + 1) for g in range(n_g)) \
            if variant != "reuse" else 0
        ws_p = torch.empty(S.workspace_bytes(p0, S.IDX_OP_GROUP_PROXY_SCAN, G, C), dtype=torch.uint8, device=dev)
        ws_r = torch.empty(max(S.workspace_bytes(p0, S.IDX_OP_REFINE_TOPK, G, C, K), 1), dtype=torch.uint8,
                           device=dev)
        cands = [torch.empty((B, n_g, C), dtype=torch.int32, device=dev) for _ in sets]
        outs = [torch.empty((B, wl.n_q, K), dtype=torch.int32, device=dev) for _ in sets]
        # the dominant kernel: the re-score for prefill Refine, the proxy scan
        # otherwise (Reuse's broadcast is cheap; a decode group's proxy scan
        # streams the whole key cache)
        if decode:
            kernel, bound, kdt, fl_k = "proxy_scan", "hbm", "bf16", proxy_pairs * fl
        elif variant != "reuse":
            kernel, bound, kdt, fl_k = "gather_scan", "mfma", dtype, refine_pairs * fl
        else:
            kernel, bound, kdt, fl_k = "proxy_scan", "mfma", "bf16", proxy_pairs * fl
        leg = Leg(variant, None, proxy_pairs + refine_pairs, B * wl.n_q, kernel, bound, kdt, flops=fl_k,
                  hbm_bytes=key_bytes + B * n_g * (H * d * 2 + 4 * H))
        leg.group, leg.n_cand = G, C

        def step_grouped(leg=leg, G=G, C=C, variant=variant, ws_p=ws_p, ws_r=ws_r, cands=cands, outs=outs):
            i = rot()
            x = sets[i]
            S.group_proxy_scan(x["q"], x["k"], x["w"], G, C, workspace=ws_p, out=cands[i], **a(x))
            if variant != "reuse":
                S.refine_topk(x["q"], x["k"], x["w"], cands[i], G, K, workspace=ws_r, out=outs[i], **a(x))
            else:
                S.reuse_topk(cands[i], G, wl.n_q, wl.n_k, q_pos0=wl.q_pos0, out=outs[i])
            leg.out = outs[0]
        leg.step = step_grouped
        legs.append(leg)
    return legs


def time_leg(S, leg, steps, warmup):
    """Wall-clock ms per step over `steps` timed steps (after `warmup`), then
    the library's per-kernel HIP-event times over as many more steps."""
    import torch
    for _ in range(warmup):
        leg.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        leg.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    S.profile_read()
    S.profile_enable(True)
    t2 = time.perf_counter()
    for _ in range(steps):
        leg.step()
    torch.cuda.synchronize()
    ms_ev = (time.perf_counter() - t2) / steps * 1e3
    S.profile_enable(False)
    prof = S.profile_read()
    kern = {k: (v[0] / steps, v[1] / steps) for k, v in prof.items() if v[1]}
    return ms, ms_ev, kern


def roofline(leg, kern, workload):
    """The leg's dominant kernel against its own peak.  Its algorithmic work
    per step (FLOPs, or HBM bytes for a scan that streams the keys) over its
    summed launch time per step (a long scan runs as several equal chunks)."""
    kms, launches = kern.get(leg.kernel, (0.0, 0.0))
    if kms <= 0:
        return None
    r = {"bound": leg.bound, "kernel": leg.kernel, "launches_per_step": launches, "ms_per_step": kms,
         "launch_ms": kms / max(launches, 1e-9)}
    if leg.bound == "mfma":
        ach = leg.flops / (kms * 1e-3) / 1e12
        r.update(achieved=ach, peak=PEAK_TFLOPS[leg.dtype], unit="TFLOP/s", frac=ach / PEAK_TFLOPS[leg.dtype],
                 dtype=leg.dtype, flops_per_step=leg.flops)
    else:
        ach = leg.hbm_bytes / (kms * 1e-3) / 1e9
        r.update(achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s", frac=ach / PEAK_HBM_GBS, bytes_per_step=leg.hbm_bytes)
    r["traffic"] = measured_traffic(workload, leg.name)
    return r


def recall_all(approx, exact, chunk=16384):
    """Recall of every query's dense top-k (sort + batched binary search on the GPU)."""
    import torch
    from sparse_attention_token_causal_amd.calibrate import recall
    a = approx.reshape(-1, approx.shape[-1])
    e = exact.reshape(-1, exact.shape[-1])
    rs = torch.cat([recall(a[i:i + chunk], e[i:i + chunk]) for i in range(0, a.shape[0], chunk)])
    return {"mean": float(rs.mean()), "min": float(rs.min()), "queries": int(rs.numel()),
            "p01": float(torch.quantile(rs.float(), 0.01))}


# ----------------------------------------------------------------------------
# the CPU oracle on a bounded sample (test infrastructure; timed here only)


def oracle_keys(O, synth, inp, b):
    ks = None if inp["k_scale"] is None else inp["k_scale"][b].cpu().numpy()
    return O.real_values(synth.raw_numpy(inp["k"][b]), synth.fmt_of(inp["k"]), ks)


def oracle_queries(O, synth, inp, b, t0, t1):
    import numpy as np
    qs = None if inp["q_scale"] is None else inp["q_scale"][b, t0:t1].cpu().numpy()
    q = O.real_values(synth.raw_numpy(inp["q"][b, t0:t1]), synth.fmt_of(inp["q"]), qs)
    return q, inp["w"][b, t0:t1].cpu().numpy().astype(np.float64)


def cpu_baseline(wl, inp, variant, seconds, G=None, C=None):
    """The oracle as it stands, timed on evenly spaced queries (dense) or whole
    groups (Refine, Reuse) of the same inputs, until about `seconds` of CPU
    work or the whole workload; key decoding is outside the timed region."""
    import numpy as np
    import oracle as O
    from sparse_attention_token_causal_amd import synth

    pairs = units = 0
    el = 0.0
    seqs = 0
    total_units = 0
    for b in range(wl.batch):
        k = oracle_keys(O, synth, inp, b)
        seqs += 1
        if variant == "dense":
            order = spread_order(wl.n_q)
            total_units += wl.n_q
        else:
            G = G or wl.group
            C = C or (wl.n_cand if variant == "refine" else wl.topk)
            lim = group_limits(wl, G)
            order = spread_order(len(lim))
            total_units += len(lim)
        t0 = time.perf_counter()
        for u in order:
            if variant == "dense":
                q, w = oracle_queries(O, synth, inp, b, u, u + 1)
                p = wl.q_pos0 + u
                I = O.causal_scores(q, k, w, np.array([p]))
                O.select_topk(I[0, : p + 1], np.arange(p + 1), wl.topk)
                pairs += p + 1
            else:
                g0, g1 = u * G, min((u + 1) * G, wl.n_q)
                q, w = oracle_queries(O, synth, inp, b, g0, g1)
                qb, wb = O.round_proxy(*O.proxy_means(q, w, G), wl.q_fmt)
                P = O.proxy_scores(qb, wb, k, np.array([lim[u]]))
                cand = O.proxy_candidates(P, np.array([lim[u]]), C)
                pairs += lim[u] + 1
                if variant != "reuse":
                    O.refine_topk(q, k, w, cand, G, wl.q_pos0 + g0, wl.topk)
                    pairs += (g1 - g0) * min(C, lim[u] + 1)
                else:
                    O.reuse_topk(cand, G, wl.q_pos0 + g0, g1 - g0, wl.topk)
            units += 1
            if el + time.perf_counter() - t0 > seconds:
                break
        el += time.perf_counter() - t0
        if el > seconds:
            break
    unit, one = ("queries", "query") if variant == "dense" else ("groups", "group")
    whole = units == total_units
    what = (f"every {one} of every sequence" if whole else
            f"{units} evenly spaced {unit} (the last first) of {seqs} sequence(s)")
    threads = blas_threads()
    return {"value": pairs / el, "unit": "pairs/s", "cores": int(threads or len(os.sched_getaffinity(0))),
            "kind": "oracle", "host_cores": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "sample": f"{what}, {variant} path ({pairs} pairs scored, float64 NumPy, {el:.1f} s)"}


# ----------------------------------------------------------------------------


def run_workload(S, wl, which, steps, warmup, cpu_secs, headline_leg, dev):
    """Times the legs of one workload; returns {leg: record}.  cpu_secs: the
    CPU oracle's time budget per leg (0: none)."""
    import torch
    from sparse_attention_token_causal_amd.synth import make_inputs

    decode = wl.n_q < wl.n_k
    log(f"[bench] {wl.name}: generating inputs")
    sets = [make_inputs(wl, dev)]
    if decode:
        sets += [make_inputs(wl.scaled(seed=wl.seed + i), dev) for i in range(1, 4)]
    torch.cuda.synchronize()
    legs = make_legs(S, wl, sets, dev, which)
    rec = {}
    dense = None
    for leg in legs:
        if leg.name == headline_leg:
            k_steps, k_warm = steps, warmup
        elif decode:  # about 75 us per step: enough steps to spread the first launch's latency
            k_steps, k_warm = max(steps, 200), max(warmup, 5)
        elif wl.n_q >= 131072 and leg.name in ("dense", "refine_r99"):
            k_steps, k_warm = min(steps, 10), min(warmup, 2)
        else:
            k_steps, k_warm = steps, warmup
        log(f"[bench] {wl.name} {leg.name}: warmup {k_warm}, timing {k_steps} steps")
        ms, ms_ev, kern = time_leg(S, leg, k_steps, k_warm)
        r = {"ms_per_step": ms, "steps": k_steps, "warmup": k_warm, "pairs_per_step": leg.pairs,
             **({"group": leg.group, "n_cand": leg.n_cand} if hasattr(leg, "group") else {}),
             "pairs_per_s": leg.pairs / (ms * 1e-3), "queries_per_s": leg.queries / (ms * 1e-3),
             "kernels_ms_per_step": {k: v[0] for k, v in kern.items()},
             "ms_per_step_with_kernel_events": ms_ev, "roofline": roofline(leg, kern, wl.name)}
        if leg.name == "dense":
            dense = (leg, r)
        elif dense is not None:
            # every query's dense top-k on the same inputs (input set 0: each
            # leg's output for it is from the last step that used it)
            dleg, dr = dense
            r["dense_equivalent_pairs_per_s"] = dleg.pairs / (ms * 1e-3)
            r["speedup_vs_dense"] = dr["ms_per_step"] / ms
            r["recall_vs_dense"] = recall_all(leg.out, dleg.out)
        rf = r["roofline"]
        log(f"[bench]   {ms:.3f} ms/step, {r['pairs_per_s']:.3g} pairs/s"
            + (f", {rf['kernel']} {100 * rf['frac']:.1f}% of the {rf['bound']} peak" if rf else "")
            + (f", speedup {r['speedup_vs_dense']:.2f}x, recall {r['recall_vs_dense']['mean']:.4f}"
               if "recall_vs_dense" in r else ""))
        rec[leg.name] = r
    for leg in legs:
        secs = cpu_secs.get(leg.name, 0.0)
        if secs > 0:
            log(f"[bench] {wl.name} {leg.name}: timing the CPU oracle for ~{secs:.0f} s")
            rec[leg.name]["cpu_baseline"] = cpu_baseline(wl, sets[0], leg.name, secs, getattr(leg, "group", None),
                                                         getattr(leg, "n_cand", None))
    del legs, sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the headline leg")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", help="'all' or one workload name (for profiling runs)")
    ap.add_argument("--legs", default="dense,refine,reuse,refine_r99",
                    help="legs to run (subset of dense,refine,reuse,refine_r99)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle time for the headline leg")
    ap.add_argument("--cpu-leg-seconds", type=float, default=3.0, help="CPU oracle time for every other leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB (4 times): the known-size reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings to HBM bytes")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the indexer path is "
                                   "built and measured on one MI355X; a multi-GPU split is a "
                                   "design note only", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = 1 << 28  # float32 elements: 1 GiB read + 1 GiB written per copy
        x = torch.ones(n, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(4):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_copy": 4 * n,
                          "bytes_written_per_copy": 4 * n, "copies": 4}))
        return
    import sparse_attention_token_causal_amd as S
    from sparse_attention_token_causal_amd.synth import WORKLOADS

    dev = torch.device("cuda:0")
    names = ORDER if args.workload == "all" else [args.workload]
    head = HEADLINE if args.workload == "all" else args.workload
    which = set(args.legs.split(","))
    results = {}
    head_leg = None
    for name in names:
        wl = WORKLOADS[name]
        wl_which = which if wl.group else {"dense"} & which
        leg0 = "refine" if (wl.group and wl.n_q == wl.n_k and "refine" in wl_which) else sorted(wl_which)[0]
        if name == head:
            head_leg = leg0
        cpu = {} if args.no_cpu_baseline else {
            leg: (args.cpu_seconds if (name == head and leg == head_leg) else args.cpu_leg_seconds)
            for leg in wl_which}
        results[name] = run_workload(S, wl, wl_which, args.steps, args.warmup, cpu,
                                     head_leg if name == head else None, dev)

    wl = WORKLOADS[head]
    h = results[head][head_leg]
    dtype = {"fp8": "fp8", "f32": "f32"}.get(wl.q_fmt, "bf16")
    out = {
        "metric": METRIC,
        "value": h["pairs_per_s"],
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": h["warmup"],
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "path": {"refine": "PIVOT-Refine", "reuse": "PIVOT-Reuse",
                                                 "refine_r99": "PIVOT-Refine at the recall-0.99 setting",
                                                 "dense": "dense scan"}[head_leg],
                   "batch": wl.batch, "n_q": wl.n_q, "n_k": wl.n_k, "heads": wl.heads, "dim": wl.dim,
                   "topk": wl.topk, "group": h.get("group", wl.group), "n_cand": h.get("n_cand", wl.n_cand),
                   "q_storage": wl.q_fmt,
                   "k_storage": wl.k_fmt, "parallelism": "single GPU"},
        "queries_per_s": h["queries_per_s"],
        "roofline": h["roofline"],
        "cpu_baseline": h.get("cpu_baseline"),
        "legs": results[head],
        "workloads": {n: r for n, r in results.items() if n != head},
    }
    for k in ("dense_equivalent_pairs_per_s", "speedup_vs_dense", "recall_vs_dense"):
        if k in h:
            out[k] = h[k]
    log(f"[bench] headline {wl.name} {head_leg}: {h['ms_per_step']:.3f} ms/step, {h['pairs_per_s']:.4g} pairs/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
