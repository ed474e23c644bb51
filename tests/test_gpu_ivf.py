"""GPU vs oracle parity of IVF routing with causal index versions (through the C ABI).

Chain, stage by stage on the GPU's own inputs to each stage:

* lists: for every version, the members, offsets and prefix counts are
  exactly the stable grouping of the GPU's own assignment (keys of the
  window in key order per cluster, -1 beyond the window);
* assignment: each key's cluster is a nearest stored centroid of the GPU's
  own centroids (exact float64 distances), within the float32 rounding of
  the distance, and exactly the nearest wherever the margin exceeds it;
* centroids: iterations = 0 leaves the initial keys (stored, within one
  bfloat16 step); one iteration gives the stored mean of each cluster of the
  previous assignment the GPU published (within one bfloat16 step, float32
  tolerance for float32 keys), empty clusters keeping their centroid;
* routing: the stored proxy is the rounded group mean; the cluster scores on
  the GPU's own proxy and centroids match the oracle within the score
  tolerance; the candidates equal the oracle's walk on the GPU's own scores
  and lists (exact, as sets); Refine over them is valid;
* end to end on similarity groups scattered over positions (no near-ties):
  the whole index and the candidates equal the oracle's own; with a budget
  holding every prefix key, Refine over the IVF candidates is the dense top-k.

Shapes cover bfloat16, FP8 and float32 keys, 16/32/64 heads, d = 64 and 128,
ragged tiles and windows, cluster counts that are not multiples of 32 and
the maximum 1024, prefill groups and decode.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.synth import Workload, make_inputs

from parity import AGREEMENT, assert_same_sets, band_agreement, check_rows_valid, check_scores, \
    check_stored_mean, cuda, real_inputs, sets

pytestmark = pytest.mark.gpu

TILE = 128

# (workload, clusters m, refit R, iterations T, insert batch b, budget C)
CASES = [
    (Workload("ivf_bf16_L1000_G16", 1, 1000, 1000, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
              topk=64, group=16, seed=41), 32, 256, 2, 128, 512),
    (Workload("ivf_fp8_L900_G64_m100", 1, 900, 900, 64, 128, "fp8", "fp8", "ar1", "heavy", rho=0.99,
              topk=40, group=64, seed=42), 100, 256, 1, 128, 384),
    (Workload("ivf_f32_B2_L700_H16_d64_G5", 2, 700, 700, 16, 64, "f32", "f32", "normal8", "normal8",
              topk=11, group=5, seed=43), 20, 128, 3, 128, 256),
    (Workload("ivf_decode_bf16q_fp8k_B3_n5000", 3, 2, 5000, 64, 128, "bf16", "fp8", "ar1", "heavy", rho=0.98,
              topk=100, group=2, seed=44), 64, 1024, 2, 256, 2048),
    (Workload("ivf_bf16_L1300_H32_d64_m1024", 1, 1300, 1300, 32, 64, "bf16", "bf16", "normal8", "heavy",
              topk=20, group=32, seed=45), 1024, 1024, 1, 128, 1024),
    # one cluster: every key in the single list
    (Workload("ivf_m1_decode_bf16_B2_n4370", 2, 3, 4370, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
              topk=132, group=36, seed=47), 1, 2048, 1, 256, 3686),
    # keys shorter than the refit interval: no version, empty index arrays
    (Workload("ivf_short_bf16_L600_R1024_noversion", 1, 600, 600, 32, 64, "bf16", "bf16", "normal8", "heavy",
              topk=20, group=8, seed=46), 64, 1024, 1, 128, 1024),
]


def ulp_bf16(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 7)


def stored(x, k_fmt):
    return O.ivf_store(x, "f32" if k_fmt == "f32" else "bf16")


def close_stored(gpu, ref, k_fmt, scale, what):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    if k_fmt == "f32":
        ok = np.abs(gpu - ref) <= 1e-5 * np.abs(ref) + 1e-6 * scale
    else:
        ok = np.abs(gpu - ref) <= np.maximum(ulp_bf16(ref) * 1.0001, 1e-6 * scale)
    assert ok.all(), f"{what}: {int((~ok).sum())} centroid elements beyond tolerance"


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_index(idx, k, R, what):
    """Lists, offsets and prefix counts are the stable grouping of the assignment;
    the assignment is a nearest stored centroid.  Returns [(centroids, assign)]
    per (sequence, version) as float64 / int64 arrays."""
    cents, offs, mem, cnt, asg = (idx[n].cpu() for n in ("centroids", "offsets", "members", "counts", "assign"))
    B, n_v, m = cents.shape[0], cents.shape[1], cents.shape[2]
    n_k = k.shape[1]
    out = []
    for b in range(B):
        row = []
        for v in range(n_v):
            u = v + 1
            win = min((u + 1) * R, n_k)
            a = asg[b, v].numpy().astype(np.int64)
            assert (a[win:] == -1).all() and (a[:win] >= 0).all() and (a[:win] < m).all(), what
            o = offs[b, v].numpy()
            assert o[0] == 0 and o[m] == win and (np.diff(o) >= 0).all(), what
            me = mem[b, v].numpy()
            for c in range(m):
                assert me[o[c]:o[c + 1]].tolist() == np.nonzero(a[:win] == c)[0].tolist(), f"{what} list {c}"
            nt = -(-win // TILE)
            onehot = np.zeros((win, m), dtype=np.int64)
            onehot[np.arange(win), a[:win]] = 1
            pre = np.concatenate([np.zeros((1, m), np.int64), np.cumsum(onehot, axis=0)])
            assert np.array_equal(cnt[b, v, : nt + 1].numpy(), pre[np.minimum(np.arange(nt + 1) * TILE, win)]), \
                f"{what} counts b={b} v={v}"
            # nearest stored centroid, exact distances on the GPU's own centroids
            C = to64(cents[b, v])
            kk = k[b, :win]
            d2 = (kk * kk).sum(1)[:, None] - 2.0 * kk @ C.T + (C * C).sum(1)[None, :]
            best = d2.min(axis=1)
            cn = np.sqrt((C * C).sum(1)).max()
            tol = 2e-5 * (cn * cn + 2.0 * np.sqrt((kk * kk).sum(1)) * cn) + 1e-30
            chosen = d2[np.arange(win), a[:win]]
            assert (chosen - best <= tol).all(), f"{what}: a key assigned beyond the rounding of its distance"
            srt = np.sort(d2, axis=1)
            clear = (srt[:, 1] - srt[:, 0]) > 2 * tol if m > 1 else np.ones(win, bool)
            assert (a[:win][clear] == d2.argmin(axis=1)[clear]).all(), f"{what}: a clear nearest centroid missed"
            row.append((C, a))
        out.append(row)
    return out


def means_of(k, a, n, prev, k_fmt, what):
    """Stored means of keys [0, n) grouped by a[:n]; empty clusters keep prev."""
    ref = prev.copy()
    for c in range(prev.shape[0]):
        sel = a[:n] == c
        if sel.any():
            ref[c] = stored(k[:n][sel].mean(axis=0), k_fmt)
    return ref


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_ivf_build_parity(case):
    wl, m, R, T, b_ins, C = case
    dev = cuda()
    print(f"\n[ivf build] {wl.name} m={m} R={R} T={T}", flush=True)
    inp = make_inputs(wl, dev)
    _, k, _ = real_inputs(inp)
    scale = np.abs(k).max()
    builds = {}
    for t in sorted({0, 1, min(T, 2)}):
        builds[t] = S.ivf_build(inp["k"], m, R, t, k_scale=inp["k_scale"], return_assign=True)
    torch.cuda.synchronize()
    n_v = wl.n_k // R
    views = {t: check_index(idx, k, R, f"{wl.name} T={t}") for t, idx in builds.items()}
    for b in range(wl.batch if n_v >= 1 else 0):
        init = stored(k[b][(np.arange(m) * R) // m], wl.k_fmt)
        for v in range(n_v):  # no iteration: every version keeps the initial keys
            close_stored(views[0][b][v][0], init, wl.k_fmt, scale, f"{wl.name} T=0 v={v}")
        # one iteration: version 1 from the assignment to the initial keys (the
        # T = 0 build's version-1 lists), version u from version u-1's lists
        prev, prev_a = views[0][b][0][0], views[0][b][0][1]
        for v in range(n_v):
            ref = means_of(k[b], prev_a, (v + 1) * R, prev, wl.k_fmt, wl.name)
            close_stored(views[1][b][v][0], ref, wl.k_fmt, scale, f"{wl.name} T=1 v={v}")
            prev, prev_a = views[1][b][v]
        if 2 in views:  # second iteration of version 1: from the T = 1 build's version-1 lists
            C1, a1 = views[1][b][0]
            ref = means_of(k[b], a1, R, C1, wl.k_fmt, wl.name)
            close_stored(views[2][b][0][0], ref, wl.k_fmt, scale, f"{wl.name} T=2 v=0")


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_ivf_route_parity(case):
    wl, m, R, T, b_ins, C = case
    dev = cuda()
    print(f"\n[ivf route] {wl.name} m={m} R={R} T={T} b={b_ins} C={C}", flush=True)
    inp = make_inputs(wl, dev)
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    G = wl.group
    idx = S.ivf_build(inp["k"], m, R, T, k_scale=inp["k_scale"], return_assign=True)
    cand, sc, pq, pw = S.ivf_route(inp["q"], inp["k"], inp["w"], idx, G, b_ins, C, return_scores=True,
                                   return_proxy=True, **a)
    cand_ws = S.ivf_route(inp["q"], inp["k"], inp["w"], idx, G, b_ins, C, **a)
    ridx = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, wl.topk, **a)
    torch.cuda.synchronize()
    assert torch.equal(cand, cand_ws)  # dump path and workspace path agree
    q, k, w = real_inputs(inp)
    views = check_index(idx, k, R, wl.name)
    pq_f, pw_f = to64(pq), pw.cpu().numpy().astype(np.float64)
    cand, sc, ridx = cand.cpu().numpy(), sc.cpu().numpy(), ridx.cpu().numpy()
    lim = O.proxy_limits(wl.n_q, G, wl.q_pos0)
    for b in range(wl.batch):
        qb, wb = O.proxy_means(q[b], w[b], G)
        qfmt = "f32" if wl.q_fmt == "f32" else "bf16"
        check_stored_mean(pq_f[b], O.round_proxy(qb, wb, qfmt)[0], q[b], O.group_bounds(wl.n_q, G), qfmt,
                          f"proxy b={b}")
        # cluster scores on the GPU's own proxy and centroids
        S_ref = np.full((lim.size, m), -np.inf)
        for g in range(lim.size):
            u = (int(lim[g]) + 1) // R
            if u >= 1:
                S_ref[g] = np.maximum(views[b][u - 1][0] @ pq_f[b, g].T, 0.0) @ pw_f[b, g]
        check_scores(sc[b], S_ref, f"{wl.name} cluster scores b={b}")
        # the walk on the GPU's own scores and lists: exact (as sets)
        c_own, _, _ = O.ivf_route(pq_f[b], pw_f[b], views[b], lim, R, b_ins, C, scores=sc[b])
        assert_same_sets(cand[b], c_own, f"{wl.name} candidates b={b}")
        check_rows_valid(cand[b], lim, C)
        # Refine over the routed candidates: causal, distinct, -1 padded, within the candidates
        check_rows_valid(ridx[b], wl.q_pos0 + np.arange(wl.n_q), wl.topk)
        for t in range(wl.n_q):
            assert sets(ridx[b, t : t + 1])[0] <= sets(cand[b, t // G : t // G + 1])[0]


CLUSTERED = Workload("ivf_clustered_bf16_L768_G8", 1, 768, 768, 64, 128, "bf16", "bf16", "ar1", "clustered",
                     rho=0.95, topk=48, group=8, seed=46, clusters=16, spread=0.05, seed_stride=16)


def test_ivf_end_to_end_on_scattered_groups():
    """Similarity groups scattered over positions, the first version's initial
    centroids one per group: no assignment or ranking is near a tie, so the
    GPU's index and candidates equal the oracle's own, and its Refine output
    agrees with the oracle's outside float near-ties."""
    wl, m, R, T, b_ins, C = CLUSTERED, 16, 256, 2, 128, 384
    dev = cuda()
    inp = make_inputs(wl, dev)
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    idx = S.ivf_build(inp["k"], m, R, T, return_assign=True)
    cand = S.ivf_route(inp["q"], inp["k"], inp["w"], idx, wl.group, b_ins, C, **a)
    ridx = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, wl.group, wl.topk, **a)
    torch.cuda.synchronize()
    q, k, w = real_inputs(inp)
    out, c_ora, _, versions = O.ivf_reference(q[0], k[0], w[0], wl.q_pos0, wl.group, m, R, T, b_ins, C, wl.topk,
                                              "bf16", "bf16")
    asg = idx["assign"].cpu().numpy()
    for v, (cent, a_ora) in enumerate(versions):
        assert np.array_equal(asg[0, v], a_ora), f"version {v + 1}: assignment differs"
        close_stored(to64(idx["centroids"][0, v]), cent, "bf16", np.abs(k).max(), f"version {v + 1}")
    assert_same_sets(cand.cpu().numpy()[0], c_ora, "candidates vs oracle")
    I = O.dense_scores(q[0], k[0], w[0], wl.q_pos0)
    assert band_agreement(ridx.cpu().numpy()[0], out, I) >= AGREEMENT


def test_ivf_whole_prefix_budget_equals_dense():
    wl = Workload("ivf_all_bf16_L640_G20", 1, 640, 640, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
                  topk=24, group=20, seed=47)
    dev = cuda()
    inp = make_inputs(wl, dev)
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    idx = S.ivf_build(inp["k"], 24, 128, 2)
    cand = S.ivf_route(inp["q"], inp["k"], inp["w"], idx, wl.group, 128, 640, **a)
    refine = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, wl.group, wl.topk, **a)
    dense = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    torch.cuda.synchronize()
    lim = O.proxy_limits(wl.n_q, wl.group, 0)
    assert sets(cand.cpu().numpy()[0]) == [frozenset(range(int(p) + 1)) for p in lim]
    assert_same_sets(refine.cpu().numpy()[0], dense.cpu().numpy()[0], "refine(all clusters) vs dense")


def test_ivf_build_is_deterministic():
    wl, m, R, T, _, _ = CASES[0]
    dev = cuda()
    inp = make_inputs(wl, dev)
    x = S.ivf_build(inp["k"], m, R, T, return_assign=True)
    y = S.ivf_build(inp["k"], m, R, T, return_assign=True)
    torch.cuda.synchronize()
    for n in ("centroids", "offsets", "assign"):
        assert torch.equal(x[n], y[n]), n
    for v in range(wl.n_k // R):  # members: only the version's window is written
        win = min((v + 2) * R, wl.n_k)
        assert torch.equal(x["members"][:, v, :win], y["members"][:, v, :win]), v
        nt = -(-win // TILE)
        assert torch.equal(x["counts"][:, v, : nt + 1], y["counts"][:, v, : nt + 1]), v
