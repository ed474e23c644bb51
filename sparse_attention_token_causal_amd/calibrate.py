"""Candidate-budget calibration: recall and speed of the approximate paths.

``python -m sparse_attention_token_causal_amd.calibrate`` runs, on seeded
synthetic prefill inputs of one or more lengths, the dense indexer (the
exact top-k), PIVOT-Refine and PIVOT-Reuse over a grid of (group size G,
candidate budget C), block-mean routing + Refine over a grid of (block
size, blocks kept), and IVF routing + Refine over a grid of (clusters,
refit interval, Lloyd iterations, insert batch, budget) - the index build
timed with the path - all through the library's C ABI on one GPU.  For every
setting it reports the recall of the dense top-k (mean and minimum over the
queries) and the time of the whole path, and picks the cheapest setting that
reaches a recall target.

What the pages ask for that this measures:

* "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention",
  Abstract: group size and candidate budget trade recall for speed; the
  grouping is training-free, so the choice is a calibration, not a retraining.
* "ADIndex Restructures Sparse-Attention Indexing with Group-Level
  Distillation", "Three Core Components" (layer-wise calibration) and
  "Deployment Guidance": measure candidate hit rates and pick conservative
  sharing levels that avoid recall loss (here: the model-free part of that
  calibration, a sweep against the dense top-k on synthetic inputs).
* "AttentionIndex Architecture ...", "KEY FINDINGS" and "Why Positional
  Blocks Lose Recall": at a fixed candidate budget the recall of contiguous
  block routing decays as the context grows; grouping keys by similarity
  (an inverted file, "An Inverted File With Causal Versions") is the fix
  the page describes.

Recall is |S_t & D_t| / |D_t| with D_t the dense top-k of query t, computed
on the GPU with a sort and a batched binary search.  This is measurement
tooling: it uses torch for recall arithmetic and timing only.
"""

import argparse
import json
import sys

import torch

from . import block_route, group_proxy_scan, ivf_build, ivf_route, refine_topk, reuse_topk, score_topk
from .synth import Workload, make_inputs


def recall(approx, exact):
    """Per-row recall of `exact` (int32 [..., k], -1 padded) by `approx` (-1 padded)."""
    e = torch.sort(exact.reshape(-1, exact.shape[-1]), dim=-1).values
    a = approx.reshape(-1, approx.shape[-1]).to(e.dtype)
    pos = torch.searchsorted(e, a.contiguous()).clamp(max=e.shape[-1] - 1)
    hit = (torch.gather(e, 1, pos) == a) & (a >= 0)
    n = (e >= 0).sum(dim=1).clamp(min=1)
    r = hit.sum(dim=1).to(torch.float64) / n.to(torch.float64)
    return r.reshape(exact.shape[:-1])


def _timed(fn, reps):
    fn()  # warm up (and allocate)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        out = fn()
    t1.record()
    torch.cuda.synchronize()
    return out, t0.elapsed_time(t1) / reps


def workload(L, seed=0, rho=0.98, topk=2048, keys="heavy", key_groups=0):
    """The 32K-token prefill recipe at length L (bf16, AR(1) queries, heavy-tailed keys);
    ``keys="clustered"`` swaps in `key_groups` similarity groups scattered over positions."""
    return Workload(f"calib_bf16_L{L}", 1, L, L, 64, 128, "bf16", "bf16", "ar1", keys, rho=rho,
                    topk=topk, seed=seed, clusters=key_groups, spread=0.5)


def sweep(L, pivot_grid, block_grid, ivf_grid=(), reps=2, seed=0, dev=None, keys="heavy", key_groups=0):
    """Rows of {path, L, setting, budget, recall_mean, recall_min, ms} for one length.

    ivf_grid: (G, clusters, refit, iterations, insert batch, budget) tuples;
    their ``ms`` includes the index build, also reported alone as ``build_ms``.
    """
    dev = dev or torch.device("cuda:0")
    wl = workload(L, seed, keys=keys, key_groups=key_groups)
    inp = make_inputs(wl, dev)
    q, k, w = inp["q"], inp["k"], inp["w"]
    K = wl.topk
    dense, ms_dense = _timed(lambda: score_topk(q, k, w, K), reps)
    rows = [dict(path="dense", L=L, setting="-", budget=L, recall_mean=1.0, recall_min=1.0, ms=ms_dense)]

    def add(path, setting, budget, idx, ms):
        r = recall(idx, dense)
        rows.append(dict(path=path, L=L, setting=setting, budget=budget, recall_mean=float(r.mean()),
                         recall_min=float(r.min()), ms=ms))

    for G, C in pivot_grid:
        def refine():
            cand = group_proxy_scan(q, k, w, G, C)
            return refine_topk(q, k, w, cand, G, K)
        idx, ms = _timed(refine, reps)
        add("pivot-refine", f"G={G} C={C}", C, idx, ms)
    for G in sorted({g for g, _ in pivot_grid}):
        def reuse():
            top = group_proxy_scan(q, k, w, G, K)
            return reuse_topk(top, G, L, L)
        idx, ms = _timed(reuse, reps)
        add("pivot-reuse", f"G={G}", K, idx, ms)
    for G, blk, keep in block_grid:
        def blocks():
            cand = block_route(q, k, w, G, blk, keep)
            return refine_topk(q, k, w, cand, G, K)
        idx, ms = _timed(blocks, reps)
        add("block-refine", f"G={G} block={blk} keep={keep}", blk * keep, idx, ms)
    for G, m, R, T, b, C in ivf_grid:
        def ivf():
            index = ivf_build(k, m, R, T)
            cand = ivf_route(q, k, w, index, G, b, C)
            return refine_topk(q, k, w, cand, G, K)
        idx, ms = _timed(ivf, reps)
        add("ivf-refine", f"G={G} m={m} R={R} T={T} b={b}", C, idx, ms)
        _, rows[-1]["build_ms"] = _timed(lambda: ivf_build(k, m, R, T), reps)
    return rows


def choose(rows, target):
    """The fastest approximate setting whose mean recall reaches `target` (None if none does)."""
    ok = [r for r in rows if r["path"] != "dense" and r["recall_mean"] >= target]
    return min(ok, key=lambda r: r["ms"]) if ok else None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--lengths", default="16384,32768,65536")
    ap.add_argument("--groups", default="16,64")
    ap.add_argument("--budgets", default="4096,8192,16384")
    ap.add_argument("--block", type=int, default=64)
    ap.add_argument("--clusters", default="256", help="IVF clusters per version (comma list)")
    ap.add_argument("--refit", type=int, default=4096, help="IVF refit interval (keys)")
    ap.add_argument("--iters", type=int, default=2, help="IVF Lloyd iterations per refit")
    ap.add_argument("--insert-batch", type=int, default=512, help="IVF insert batch (keys)")
    ap.add_argument("--target", type=float, default=0.9)
    ap.add_argument("--reps", type=int, default=2)
    ap.add_argument("--keys", default="heavy", choices=["heavy", "clustered"],
                    help="key distribution: heavy-tailed i.i.d. rows, or similarity groups scattered over positions")
    ap.add_argument("--key-groups", type=int, default=512, help="similarity groups of the clustered keys")
    ap.add_argument("--json", action="store_true", help="one JSON object per line instead of a table")
    a = ap.parse_args(argv)
    groups = [int(x) for x in a.groups.split(",")]
    budgets = [int(x) for x in a.budgets.split(",")]
    all_rows = []
    for L in (int(x) for x in a.lengths.split(",")):
        pivot = [(G, C) for G in groups for C in budgets if C < L]
        blocks = [(G, a.block, C // a.block) for G in groups for C in budgets if C < L]
        ivfs = [(G, int(m), a.refit, a.iters, a.insert_batch, C) for G in groups for m in a.clusters.split(",")
                for C in budgets if a.refit <= C < L]
        rows = sweep(L, pivot, blocks, ivfs, reps=a.reps, keys=a.keys, key_groups=a.key_groups)
        all_rows += rows
        for r in rows:
            if a.json:
                print(json.dumps(r), flush=True)
            else:
                extra = f"  (index build {r['build_ms']:.2f} ms)" if "build_ms" in r else ""
                print(f"L={r['L']:7d} {r['path']:13s} {r['setting']:30s} budget {r['budget']:7d}  "
                      f"recall {r['recall_mean']:.4f} (min {r['recall_min']:.4f})  {r['ms']:8.2f} ms{extra}",
                      flush=True)
        best = choose(rows, a.target)
        print(f"L={L}: fastest setting with mean recall >= {a.target}: "
              f"{'none' if best is None else best['path'] + ' ' + best['setting']}", flush=True)
    return all_rows


if __name__ == "__main__":
    main()
    sys.exit(0)
