#!/usr/bin/env python3
"""Throughput of the causal lightning indexer on one MI355X.

One step = one call of the hot path on one batch of synthetic input that is
already resident in HBM.  The default workload is the dense causal scan +
per-query top-k at L = 32768, 64 heads, d = 128, bfloat16 q/k, k = 2048
(``prefill_bf16_L32768_H64_d128_k2048``); other workloads (decode, PIVOT
grouped) can be selected with --workload.

Prints one JSON line: pairs scored per second (all heads of a causal
(query, key) pair count once), top-k queries per second, the score kernel's
achieved MFMA rate against the bf16/fp8 dense peak (per-launch HIP events
recorded by the library on the launch stream, in a second run of the same
steps so that the events stay out of the step time), and the CPU oracle timed
on a bounded sample of the same workload on this host's cores.
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
DEFAULT_WORKLOAD = "prefill_bf16_L32768_H64_d128_k2048"

# MI355X published dense peaks (no sparsity), TFLOP/s, and HBM3E GB/s.
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0

# sources of the scan kernels whose HBM traffic the committed PMC runs measured
KERNEL_SOURCES = ["sparse_attention_token_causal_amd/csrc/score.hip",
                  "sparse_attention_token_causal_amd/csrc/split.hip",
                  "sparse_attention_token_causal_amd/csrc/common.hpp",
                  "sparse_attention_token_causal_amd/csrc/kernels.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernel_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(n_q, n_k, q_pos0, limits=None):
    """Sum over rows of (limit + 1) keys; limits default to q_pos0 + t."""
    if limits is None:
        first = q_pos0 + 1
        last = q_pos0 + n_q
        return (first + last) * n_q // 2
    return int(sum(int(x) + 1 for x in limits))


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per scan launch from committed rocprofv3 PMC runs ({workload:
    record}), if they were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def make_step(S, wl, inp, dev):
    """Returns (step(), pairs_per_step, flops_per_step, queries_per_step, dtype, kind)."""
    import torch
    from sparse_attention_token_causal_amd.synth import make_inputs

    H, d = wl.heads, wl.dim
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    dense_pairs = wl.batch * causal_pairs(wl.n_q, wl.n_k, wl.q_pos0)
    dtype = "fp8" if wl.q_fmt == "fp8" else ("f32" if wl.q_fmt == "f32" else "bf16")
    if wl.group == 0 or wl.name.startswith("decode") or wl.name.startswith("prefill"):
        if wl.n_q < wl.n_k:
            # decode: the key cache (134 MB) fits the 256 MB Infinity Cache, so the
            # steps rotate over four independent caches (>= 540 MB) to time HBM reads
            sets = [inp] + [make_inputs(wl.scaled(seed=wl.seed + i), dev) for i in range(1, 4)]
            outs = [torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.int32, device=dev) for _ in sets]
            p = S.make_problem(inp["q"], inp["k"], inp["w"], **a)
            ws = torch.empty(S.workspace_bytes(p, S.IDX_OP_SCORE_TOPK, topk=wl.topk), dtype=torch.uint8,
                             device=dev)
            it = [0]

            def step():
                x = sets[it[0] % len(sets)]
                S.score_topk(x["q"], x["k"], x["w"], wl.topk, q_scale=x["q_scale"], k_scale=x["k_scale"],
                             q_pos0=wl.q_pos0, workspace=ws, out=outs[it[0] % len(sets)])
                it[0] += 1
            return step, dense_pairs, dense_pairs * 2 * H * d, wl.batch * wl.n_q, dtype, "decode"
        p = S.make_problem(inp["q"], inp["k"], inp["w"], **a)
        # exactly the workspace the library asks for
        ws = torch.empty(S.workspace_bytes(p, S.IDX_OP_SCORE_TOPK, topk=wl.topk), dtype=torch.uint8, device=dev)
        out = torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.int32, device=dev)

        def step():
            S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, workspace=ws, out=out, **a)
        return step, dense_pairs, dense_pairs * 2 * H * d, wl.batch * wl.n_q, dtype, "dense"

    # PIVOT grouped: one proxy scan to C candidates, then each member's Refine
    import numpy as np
    G, C, K = wl.group, wl.n_cand, wl.topk
    n_g = -(-wl.n_q // G)
    lim = [wl.q_pos0 + min((g + 1) * G, wl.n_q) - 1 for g in range(n_g)]
    proxy_pairs = wl.batch * causal_pairs(n_g, wl.n_k, 0, lim)
    refine_pairs = wl.batch * sum(min(G, wl.n_q - g * G) * min(C, lim[g] + 1) for g in range(n_g))
    p = S.make_problem(inp["q"], inp["k"], inp["w"], **a)
    ws_p = torch.empty(S.workspace_bytes(p, S.IDX_OP_GROUP_PROXY_SCAN, G, C), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(max(S.workspace_bytes(p, S.IDX_OP_REFINE_TOPK, G, C, K),
                           wl.batch * wl.n_q * C * 4), dtype=torch.uint8, device=dev)
    out = torch.empty((wl.batch, wl.n_q, K), dtype=torch.int32, device=dev)

    def step():
        cand = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, C, workspace=ws_p, **a)
        S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, K, workspace=ws_r, out=out, **a)
    pairs = proxy_pairs + refine_pairs
    return step, pairs, pairs * 2 * H * d, wl.batch * wl.n_q, dtype, "refine"


def cpu_baseline(wl, inp, seconds):
    """The oracle as it stands, on evenly spaced queries of the same inputs,
    sequence after sequence, until about `seconds` of CPU work or the whole
    workload (the decode workloads are small); returns the JSON object."""
    import numpy as np
    import oracle as O
    from sparse_attention_token_causal_amd import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))
    n = wl.n_q
    order = []
    # evenly spaced queries, refined by bisection so any prefix of the list is spread out
    step = n
    seen = set()
    while step >= 1 and len(order) < n:
        for t in range(step // 2 if step > 1 else 0, n, max(step, 1)):
            if t not in seen:
                seen.add(t)
                order.append(t)
        if step == 1:
            break
        step //= 2
    pairs = 0
    done = 0
    el = 0.0
    seqs = 0
    for b in range(wl.batch):
        ks = None if inp["k_scale"] is None else inp["k_scale"][b].cpu().numpy()
        k = O.real_values(synth.raw_numpy(inp["k"][b]), synth.fmt_of(inp["k"]), ks)
        seqs += 1
        t0 = time.perf_counter()
        for t in order:
            qs = None if inp["q_scale"] is None else inp["q_scale"][b, t:t + 1].cpu().numpy()
            q = O.real_values(synth.raw_numpy(inp["q"][b, t:t + 1]), synth.fmt_of(inp["q"]), qs)
            w = inp["w"][b, t:t + 1].cpu().numpy().astype(np.float64)
            lim = np.array([wl.q_pos0 + t])
            I = O.causal_scores(q, k, w, lim)
            O.select_topk(I[0, : lim[0] + 1], np.arange(lim[0] + 1), wl.topk)
            pairs += int(lim[0]) + 1
            done += 1
            if el + time.perf_counter() - t0 > seconds:
                break
        el += time.perf_counter() - t0
        if el > seconds:
            break
    whole = seqs == wl.batch and done == wl.batch * n
    what = "every query of every sequence" if whole else f"{done} evenly spaced queries of {seqs} sequence(s)"
    return {"value": pairs / el, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what} ({pairs} causal pairs, float64 NumPy, {el:.1f} s, key decoding "
                      f"excluded); queries/s {done / el:.3g}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200 for a decode workload, 20 otherwise)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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
    from sparse_attention_token_causal_amd.synth import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] workload {wl.name}: generating inputs")
    inp = make_inputs(wl, dev)
    torch.cuda.synchronize()
    step, pairs, flops, queries, dtype, kind = make_step(S, wl, inp, dev)
    # enough steps that the first launch's latency is spread thin: a decode
    # step is about 75 us of device time
    steps = args.steps if args.steps is not None else (200 if kind == "decode" else 20)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: the steps alone.  The per-kernel durations come from a
    # second run of the same steps with the library's HIP events around each
    # launch (on the launch stream); the events add a few microseconds per
    # launch, which matters for the short decode step, so they stay out of
    # the step time.
    log(f"[bench] timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    s_per_step = (t1 - t0) / steps
    S.profile_read()  # drop anything recorded before
    S.profile_enable(True)
    torch.cuda.synchronize()
    log(f"[bench] timing the kernels of {steps} more steps (HIP events per launch)")
    t2 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    S.profile_enable(False)
    prof = S.profile_read()
    score_ms, score_n = prof["score"]
    sel_ms, sel_n = prof["select"]
    per_launch_ms = score_ms / max(score_n, 1)
    launches_per_step = score_n / steps
    flops_per_launch = flops / max(launches_per_step, 1e-9)
    achieved = flops_per_launch / (per_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    traffic = measured_traffic(wl.name)
    roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic,
            "kernel": "score (Q.K^T on MFMA + fused ReLU/weight/head-sum epilogue)",
            "launch_ms": per_launch_ms, "flops_per_launch": flops_per_launch}
    if kind == "decode":
        # the decode scan streams the key cache: algorithmic bytes per launch =
        # keys (+ per-token scales) + queries + head weights, each read once
        kb = {"fp8": 1, "bf16": 2, "f32": 4}[wl.k_fmt]
        qb = {"fp8": 1, "bf16": 2, "f32": 4}[wl.q_fmt]
        key_bytes = wl.batch * wl.n_k * (wl.dim * kb + (4 if wl.k_fmt == "fp8" else 0))
        q_bytes = wl.batch * wl.n_q * (wl.heads * wl.dim * qb + wl.heads * 4 + (4 if wl.q_fmt == "fp8" else 0))
        alg = (key_bytes + q_bytes) / max(launches_per_step, 1e-9)
        gbs = alg / (per_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "traffic": traffic,
                "kernel": "split-key scan (streams the key cache; MFMA + fused epilogue)",
                "launch_ms": per_launch_ms, "bytes_per_launch": alg, "flops_per_launch": flops_per_launch}
    result = {
        "metric": METRIC,
        "value": pairs / s_per_step,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": s_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "n_q": wl.n_q, "n_k": wl.n_k,
                   "heads": wl.heads, "dim": wl.dim, "topk": wl.topk, "q_storage": wl.q_fmt,
                   "k_storage": wl.k_fmt, "parallelism": "single GPU"},
        "queries_per_s": queries / s_per_step,
        "pairs_per_step": pairs,
        "kernels_ms_per_step": {k: v[0] / steps for k, v in prof.items() if v[1]},
        "ms_per_step_with_kernel_events": (t3 - t2) / steps * 1e3,
        "roofline": roof,
        "cpu_baseline": None,
    }
    log(f"[bench] {result['ms_per_step']:.3f} ms/step, score {per_launch_ms:.3f} ms/launch "
        f"({roof['achieved']:.1f} {roof['unit']}, {100 * roof['frac']:.1f}% of the {roof['bound']} peak), select "
        f"{sel_ms / max(sel_n, 1):.3f} ms/launch")
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
