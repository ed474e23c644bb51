"""GPU vs oracle parity of the routed candidate generators at full size.

Block-mean routing and IVF routing on the 32K-token bf16 prefill workload in
the configuration the calibration sweep times (G = 16; blocks of 64 keys,
128 kept; 256 clusters, refits every 4096 keys, 2 Lloyd iterations, insert
batches of 512, a budget of 8192).  Every candidate and Refine row is checked
for the invariants that hold at any size; sampled groups are checked against
the oracle on the GPU's own inputs to each stage (proxy, representatives,
scores within tolerance, routing exact as sets), and the IVF index is checked
whole: lists exactly the stable grouping of the assignment, assignment a
nearest stored centroid, one Lloyd iteration the stored means of the
previous published lists.
"""

import gc

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.calibrate import workload
from sparse_attention_token_causal_amd.synth import make_inputs

from parity import assert_same_sets, check_rows_valid, check_scores, check_stored_mean, cuda, real_inputs, sets
from test_gpu_ivf import check_index, close_stored, means_of, stored, to64

pytestmark = pytest.mark.gpu

L, G, TOPK = 32768, 16, 2048


def free():
    gc.collect()
    torch.cuda.empty_cache()


def sample_groups(n_g, count=12):
    return sorted(set([0, n_g - 1] + list(np.linspace(0, n_g - 1, count).astype(int))))


def check_refine(ridx, cand, lim_q, topk, group):
    """Every Refine row: distinct, causal, -1 padded; sampled rows inside their group's candidates."""
    check_rows_valid(ridx, lim_q, topk)
    for t in np.linspace(0, ridx.shape[0] - 1, 64).astype(int):
        assert sets(ridx[t : t + 1])[0] <= sets(cand[t // group : t // group + 1])[0]


def test_block_route_L32768():
    dev = cuda()
    wl = workload(L)
    blk, keep = 64, 128
    print(f"\n[full] block routing {wl.name} block {blk} keep {keep}", flush=True)
    inp = make_inputs(wl, dev)
    cand, km, bsc, pq, pw = S.block_route(inp["q"], inp["k"], inp["w"], G, blk, keep, return_means=True,
                                         return_scores=True, return_proxy=True)
    ridx = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, TOPK)
    torch.cuda.synchronize()
    q, k, w = real_inputs(inp)
    cand, bsc, ridx = cand.cpu().numpy()[0], bsc.cpu().numpy()[0], ridx.cpu().numpy()[0]
    km_f, pq_f, pw_f = to64(km)[0], to64(pq)[0], pw.cpu().numpy().astype(np.float64)[0]
    free()
    n_g = L // G
    lim = O.proxy_limits(L, G, 0)
    n_full = (lim + 1) // blk
    # every candidate row: distinct, inside the prefix, the kept blocks plus the partial tail
    check_rows_valid(cand, lim, cand.shape[1], expect_counts=np.minimum(keep, n_full) * blk + (lim + 1 - n_full * blk))
    # block means: every block, within one bf16 step of the rounded mean (plus
    # the float32 accumulation bound)
    ref = stored(O.block_means(k[0], blk), "bf16")
    check_stored_mean(km_f, ref, k[0], [(j, min(j + blk, L)) for j in range(0, L, blk)], "bf16", "block means")
    sg = sample_groups(n_g)
    qb, wb = O.proxy_means(q[0], w[0], G)
    for g in sg:
        refq, _ = O.round_proxy(qb[g : g + 1], wb[g : g + 1], "bf16")
        check_stored_mean(pq_f[g : g + 1], refq, q[0], [(g * G, (g + 1) * G)], "bf16", f"proxy {g}")
        f = int(n_full[g])
        B = np.full(bsc.shape[1], -np.inf)
        B[:f] = np.maximum(km_f[:f] @ pq_f[g].T, 0.0) @ pw_f[g]
        check_scores(bsc[g : g + 1], B[None], f"block scores g={g}")
        top = O.select_topk(bsc[g, :f].astype(np.float64), np.arange(f), keep)
        own = np.concatenate([np.arange(j * blk, (j + 1) * blk) for j in top] + [np.arange(f * blk, int(lim[g]) + 1)])
        assert_same_sets(cand[g : g + 1], [own], f"block candidates g={g}")
    check_refine(ridx, cand, np.arange(L), TOPK, G)


def test_ivf_route_L32768():
    dev = cuda()
    wl = workload(L)
    m, R, T, b_ins, C = 256, 4096, 2, 512, 8192
    print(f"\n[full] IVF {wl.name} m={m} R={R} T={T} b={b_ins} C={C}", flush=True)
    inp = make_inputs(wl, dev)
    idx0 = S.ivf_build(inp["k"], m, R, 0, return_assign=True)
    idx1 = S.ivf_build(inp["k"], m, R, 1, return_assign=True)
    idx = S.ivf_build(inp["k"], m, R, T, return_assign=True)
    cand, sc, pq, pw = S.ivf_route(inp["q"], inp["k"], inp["w"], idx, G, b_ins, C, return_scores=True,
                                   return_proxy=True)
    ridx = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, TOPK)
    torch.cuda.synchronize()
    q, k, w = real_inputs(inp)
    scale = np.abs(k).max()
    # the whole index, for each build: lists = stable grouping, assignment = a nearest centroid
    v0 = check_index(idx0, k, R, "T=0")[0]
    v1 = check_index(idx1, k, R, "T=1")[0]
    vT = check_index(idx, k, R, f"T={T}")[0]
    del idx0, idx1
    # one iteration: stored means of the previous published lists (version 1: of the initial keys')
    prev, prev_a = v0[0]
    for v in range(L // R):
        close_stored(v1[v][0], means_of(k[0], prev_a, (v + 1) * R, prev, "bf16", "means"), "bf16", scale,
                     f"T=1 v={v}")
        prev, prev_a = v1[v]
    cand, sc, ridx = cand.cpu().numpy()[0], sc.cpu().numpy()[0], ridx.cpu().numpy()[0]
    pq_f, pw_f = to64(pq)[0], pw.cpu().numpy().astype(np.float64)[0]
    free()
    n_g = L // G
    lim = O.proxy_limits(L, G, 0)
    check_rows_valid(cand, lim, C)
    sg = sample_groups(n_g)
    qb, wb = O.proxy_means(q[0], w[0], G)
    S_ref = np.full((len(sg), m), -np.inf)
    for i, g in enumerate(sg):
        refq, _ = O.round_proxy(qb[g : g + 1], wb[g : g + 1], "bf16")
        check_stored_mean(pq_f[g : g + 1], refq, q[0], [(g * G, (g + 1) * G)], "bf16", f"proxy {g}")
        u = (int(lim[g]) + 1) // R
        if u >= 1:
            S_ref[i] = np.maximum(vT[u - 1][0] @ pq_f[g].T, 0.0) @ pw_f[g]
    check_scores(sc[sg], S_ref, "cluster scores")
    c_own, _, _ = O.ivf_route(pq_f[sg], pw_f[sg], vT, lim[sg], R, b_ins, C, scores=sc[sg])
    assert_same_sets(cand[sg], c_own, "IVF candidates")
    check_refine(ridx, cand, np.arange(L), TOPK, G)
