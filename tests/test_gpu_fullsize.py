"""GPU vs oracle parity at the full workload sizes, on sampled outputs.

Every output row is checked for the invariants that hold at any size (distinct
causal indices, -1 padding at the end, the expected count); sampled rows and
groups are checked against the oracle, which computes them one by one:
scores within tolerance, the select bit-exact on the GPU's own scores, and
banded set agreement with the oracle's own top-k.  The grouped workloads also
run the dense scan at their full size (262144 and 131072 tokens) in the timed
configuration, check the proxy, the candidate select and Reuse exactly, check
that Refine equals dense wherever a group's whole prefix fits the candidate
budget, and report recall of the GPU dense top-k over every query (a
measurement, not a parity bar).
"""

import gc

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.calibrate import recall
from sparse_attention_token_causal_amd.synth import WORKLOADS, make_inputs

from parity import (AGREEMENT, ATOL, RTOL, assert_same_sets, band_agreement, check_rows_valid, check_scores,
                    cuda, real_rows)

pytestmark = pytest.mark.gpu


def sample_rows(n, count):
    """First, last and evenly spaced rows."""
    return sorted(set([0, n - 1] + list(np.linspace(0, n - 1, count).astype(int))))


def free():
    gc.collect()
    torch.cuda.empty_cache()


def args(inp, wl):
    return dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)


def check_dense_rows(inp, wl, b, idx_b, rows, scores_b=None):
    """Oracle checks of sampled rows of sequence b: D1/D2 when scores are given, D3 always."""
    q, k, w = real_rows(inp, b, rows)
    lim = wl.q_pos0 + np.asarray(rows)
    I = O.causal_scores(q, k, w, lim)
    if scores_b is not None:
        check_scores(scores_b, I, f"{wl.name} b={b} sampled scores")
        own = [O.select_topk(scores_b[i, : lim[i] + 1].astype(np.float64), np.arange(lim[i] + 1), wl.topk)
               for i in range(len(rows))]
        assert_same_sets(idx_b, own, f"{wl.name} b={b} select on own scores")
    ora = [O.select_topk(I[i, : lim[i] + 1], np.arange(lim[i] + 1), wl.topk) for i in range(len(rows))]
    ora = np.array([np.pad(r, (0, wl.topk - len(r)), constant_values=-1) for r in ora])
    agr = band_agreement(idx_b, ora, I)
    assert agr >= AGREEMENT, f"{wl.name}: set agreement {agr}"
    return I, ora


def all_rows_valid(idx, wl):
    """Vectorized invariants over every row: distinct, causal, padded, count."""
    idx = idx.reshape(-1, idx.shape[-1])
    n_q = wl.n_q
    lim = np.tile(wl.q_pos0 + np.arange(n_q), idx.shape[0] // n_q)
    valid = idx >= 0
    cnt = valid.sum(1)
    assert (cnt == np.minimum(wl.topk, lim + 1)).all(), "wrong counts"
    # valid entries first, then padding
    assert (valid[:, :-1] | ~valid[:, 1:]).all(), "padding not at the end"
    assert (np.where(valid, idx, -1) <= lim[:, None]).all(), "index beyond the causal limit"
    srt = np.sort(np.where(valid, idx, -1), axis=1)
    dup = (srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] >= 0)
    assert not dup.any(), "duplicate indices"


def same_sets_every_row(a, b):
    """Number of rows whose index sets differ between two [rows, k] GPU outputs."""
    sa, sb = torch.sort(a, dim=-1)[0], torch.sort(b, dim=-1)[0]
    return int((sa != sb).any(dim=-1).sum())


def test_prefill_bf16_L32768():
    dev = cuda()
    wl = WORKLOADS["prefill_bf16_L32768_H64_d128_k2048"]
    print(f"\n[full] {wl.name}", flush=True)
    inp = make_inputs(wl, dev)
    a = args(inp, wl)
    # the timed configuration: the library's own workspace size (bounded
    # candidate lists, rescans for rows that overflow them)
    idx = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    torch.cuda.synchronize()
    free()
    idx_np = idx.cpu().numpy()
    all_rows_valid(idx_np, wl)
    rows = sample_rows(wl.n_q, 96)
    # the score dump path on the same inputs (the same scores, every row's
    # top-k selected from its full score row): scores for D1/D2 on the
    # sampled rows, and every row's set equal to the timed path's
    idx_d, sc = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **a)
    torch.cuda.synchronize()
    n_diff = same_sets_every_row(idx[0], idx_d[0])
    assert n_diff == 0, f"timed path vs dump path: {n_diff} of {wl.n_q} rows differ"
    rows_t = torch.as_tensor(rows, device=dev)
    sc_rows = sc[0].index_select(0, rows_t).cpu().numpy()
    idx_d = idx_d[0].index_select(0, rows_t).cpu().numpy()
    del sc
    free()
    check_dense_rows(inp, wl, 0, idx_d, rows, sc_rows)
    print(f"  timed path = dump path on all {wl.n_q} rows", flush=True)


def test_decode_fp8k_B8_n131072():
    dev = cuda()
    wl = WORKLOADS["decode_fp8k_B8_mtp2_n131072_H64_d128_k2048"]
    print(f"\n[full] {wl.name}", flush=True)
    inp = make_inputs(wl, dev)
    a = args(inp, wl)
    idx_ws = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    idx, sc = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **a)
    torch.cuda.synchronize()
    idx, sc, idx_ws = idx.cpu().numpy(), sc.cpu().numpy(), idx_ws.cpu().numpy()
    assert np.array_equal(np.sort(idx, -1), np.sort(idx_ws, -1))
    all_rows_valid(idx, wl)
    for b in range(wl.batch):
        check_dense_rows(inp, wl, b, idx[b], list(range(wl.n_q)), sc[b])
    # decode grouping: the MTP step's queries form one group
    G, C, K = wl.group, wl.n_cand, wl.topk
    cand, pq, pw, ps = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, C, return_proxy=True,
                                          return_scores=True, **a)
    ridx, rsc = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, K, return_scores=True, **a)
    ptop = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, K, **a)
    uidx = S.reuse_topk(ptop, G, wl.n_q, wl.n_k, q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    cand, ps, ridx, rsc = cand.cpu().numpy(), ps.cpu().numpy(), ridx.cpu().numpy(), rsc.cpu().numpy()
    pq_f, pw_f = pq.float().cpu().numpy().astype(np.float64), pw.cpu().numpy().astype(np.float64)
    ptop, uidx = ptop.cpu().numpy(), uidx.cpu().numpy()
    lim = O.proxy_limits(wl.n_q, G, wl.q_pos0)
    recalls = []
    for b in range(wl.batch):
        q, k, w = real_rows(inp, b, list(range(wl.n_q)))
        P = O.proxy_scores(pq_f[b], pw_f[b], k, lim)
        check_scores(ps[b], P, f"decode proxy scores b={b}")
        assert_same_sets(cand[b], O.proxy_candidates(ps[b].astype(np.float64), lim, C), "decode candidates")
        own = O.refine_topk(q, k, w, cand[b], G, wl.q_pos0, K, scores=rsc[b].astype(np.float64))
        assert_same_sets(ridx[b], own, f"decode refine select b={b}")
        assert np.array_equal(uidx[b], O.reuse_topk(ptop[b], G, wl.q_pos0, wl.n_q, K))
        recalls.append(O.recall(ridx[b], idx[b]).mean())
    print(f"  decode-group Refine recall vs dense: {np.mean(recalls):.4f}", flush=True)


def default_starts(wl, m=32):
    """A middle and the last run of m queries (starts aligned to 8), prefill shapes only."""
    if wl.q_pos0 != 0 or wl.n_q < 2 * m:
        return []
    return sorted({(wl.n_q // 2) // 8 * 8, (wl.n_q - m) // 8 * 8})


def dense_fullsize(wl, inp, starts, m=32, every_row_dump=False):
    """The dense scan at full size as timed (the library's own workspace:
    bounded candidate lists, several chunks): the invariants on every row;
    for each sampled run of m consecutive queries, the score-dump path on a
    sub-problem (those queries against the keys up to the last of them: the
    same kernel arithmetic), whose scores are checked against the oracle
    (D1), whose select is bit-exact on its own scores (D2), whose sets equal
    the timed path's, and band agreement with the oracle's top-k (D3)."""
    a = args(inp, wl)
    idx = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    all_rows_valid(idx_np, wl)
    if every_row_dump:
        # the score dump path on the whole problem (every score row written,
        # each row's top-k selected from it): the same sets on every row
        idx_d, sc = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **a)
        torch.cuda.synchronize()
        del sc
        free()
        n_diff = same_sets_every_row(idx[0], idx_d[0])
        del idx_d
        free()
        assert n_diff == 0, f"{wl.name}: timed path vs dump path: {n_diff} of {wl.n_q} rows differ"
        print(f"  dense timed path = dump path on all {wl.n_q} rows", flush=True)
    k_full = real_rows(inp, 0, [0])[1]
    for t0 in starts:
        assert t0 % 8 == 0 and wl.q_pos0 == 0 and t0 + m <= wl.n_q
        sl = slice(t0, t0 + m)
        sub = lambda x, s2: None if x is None else x[:, s2].contiguous()
        idx_d, sc = S.score_topk(sub(inp["q"], sl), sub(inp["k"], slice(0, t0 + m)), sub(inp["w"], sl), wl.topk,
                                 q_scale=sub(inp["q_scale"], sl), k_scale=sub(inp["k_scale"], slice(0, t0 + m)),
                                 q_pos0=t0, return_scores=True)
        torch.cuda.synchronize()
        idx_d, sc = idx_d[0].cpu().numpy(), sc[0].cpu().numpy()
        rows = list(range(t0, t0 + m))
        q, _, w = real_rows(inp, 0, rows)
        lim = np.asarray(rows)
        I = O.causal_scores(q, k_full[: t0 + m], w, lim)
        check_scores(sc, I, f"{wl.name} dense scores t0={t0}")
        own = [O.select_topk(sc[i, : lim[i] + 1].astype(np.float64), np.arange(lim[i] + 1), wl.topk) for i in range(m)]
        assert_same_sets(idx_d, own, f"{wl.name} select on own scores t0={t0}")
        assert_same_sets(idx_np[0, sl], idx_d, f"{wl.name} timed path vs dump path t0={t0}")
        ora = [O.select_topk(I[i, : lim[i] + 1], np.arange(lim[i] + 1), wl.topk) for i in range(m)]
        ora = np.array([np.pad(r, (0, wl.topk - len(r)), constant_values=-1) for r in ora])
        agr = band_agreement(idx_np[0, sl], ora, I)
        assert agr >= AGREEMENT, f"{wl.name}: dense set agreement {agr} at t0={t0}"
    print(f"  dense at full size: every row valid, {len(starts)} x {m} sampled rows match the dump path "
          f"and the oracle", flush=True)
    return idx


def grouped_fullsize(wl, sample_groups, dense_queries, dense_starts=None, every_row_dump=False):
    dev = cuda()
    print(f"\n[full] {wl.name}", flush=True)
    inp = make_inputs(wl, dev)
    free()
    a = args(inp, wl)
    dense_gpu = dense_fullsize(wl, inp, default_starts(wl) if dense_starts is None else dense_starts,
                               every_row_dump=every_row_dump)
    free()
    G, C, K = wl.group, wl.n_cand, wl.topk
    n_g = -(-wl.n_q // G)
    lim = O.proxy_limits(wl.n_q, G, wl.q_pos0)
    # Refine, as timed: proxy scan to C candidates then the per-query re-score
    cand, pq, pw, ps = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, C, return_proxy=True,
                                          return_scores=True, **a)
    torch.cuda.synchronize()
    g_t = torch.as_tensor(sample_groups, device=dev)
    ps_s = ps[0].index_select(0, g_t).cpu().numpy()
    del ps
    free()
    ridx, rsc = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, K, return_scores=True, **a)
    torch.cuda.synchronize()
    qrows = [t for g in sample_groups for t in range(g * G, min((g + 1) * G, wl.n_q))]
    q_t = torch.as_tensor(qrows, device=dev)
    rsc_s = rsc[0].index_select(0, q_t).cpu().numpy()
    del rsc
    free()
    ptop = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, K, **a)
    uidx = S.reuse_topk(ptop, G, wl.n_q, wl.n_k, q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    # recall of the GPU dense top-k over every query (a measurement), and an
    # exact identity: where a group's whole prefix fits the candidate budget
    # its candidates are that prefix, so Refine (the same scores) is dense
    rec_r = recall(ridx, dense_gpu)
    rec_u = recall(uidx, dense_gpu)
    full_prefix = (torch.as_tensor(lim, device=dev) + 1 <= C).repeat_interleave(G)[: wl.n_q]
    n_exact = int(full_prefix.sum())
    srt = lambda x: torch.sort(x[0][full_prefix], dim=-1)[0]
    assert n_exact == 0 or torch.equal(srt(ridx), srt(dense_gpu)), "Refine over a whole prefix is not dense"
    print(f"  all {wl.n_q} queries vs the GPU dense top-k: Refine recall mean {float(rec_r.mean()):.4f} "
          f"min {float(rec_r.min()):.4f}; Reuse recall mean {float(rec_u.mean()):.4f} min {float(rec_u.min()):.4f}; "
          f"{n_exact} queries with the whole prefix as candidates: Refine = dense", flush=True)
    del dense_gpu
    cand_np, ptop_np = cand.cpu().numpy()[0], ptop.cpu().numpy()[0]
    ridx_np, uidx_np = ridx.cpu().numpy(), uidx.cpu().numpy()
    pq_s = pq[0].index_select(0, g_t).float().cpu().numpy().astype(np.float64)
    pw_s = pw[0].index_select(0, g_t).cpu().numpy().astype(np.float64)
    del ridx, uidx, ptop
    free()
    # invariants on every row
    check_rows_valid(cand_np, lim, C, np.minimum(C, lim + 1))
    assert (ridx_np[0] <= (wl.q_pos0 + np.arange(wl.n_q))[:, None]).all(), "refine index beyond the limit"
    # C >= k + G - 1 here, so every Refine row holds min(k, pos + 1) entries
    assert ((ridx_np[0] >= 0).sum(1) == np.minimum(K, wl.q_pos0 + np.arange(wl.n_q) + 1)).all()
    # Reuse is integer work: exact for every row
    assert np.array_equal(uidx_np[0], O.reuse_topk(ptop_np, G, wl.q_pos0, wl.n_q, K))
    # sampled groups against the oracle
    k_full = real_rows(inp, 0, [0])[1]
    for j, g in enumerate(sample_groups):
        P = O.proxy_scores(pq_s[j:j + 1], pw_s[j:j + 1], k_full, lim[g:g + 1])
        check_scores(ps_s[j:j + 1], P, f"{wl.name} proxy scores g={g}")
        own = O.proxy_candidates(ps_s[j:j + 1].astype(np.float64), lim[g:g + 1], C)
        assert_same_sets(cand_np[g:g + 1], own, f"{wl.name} candidates g={g}")
        members = list(range(g * G, min((g + 1) * G, wl.n_q)))
        q, k, w = real_rows(inp, 0, members)
        # candidate scores: oracle on the GPU's candidates, member by member
        sl = slice(qrows.index(members[0]), qrows.index(members[-1]) + 1)
        ref_sc = np.full((len(members), C), -np.inf)
        c = cand_np[g]
        for i, t in enumerate(members):
            ok = (c >= 0) & (c <= wl.q_pos0 + t)
            ref_sc[i, ok] = np.maximum(k[c[ok]] @ q[i].T, 0.0) @ w[i]
        check_scores(rsc_s[sl], ref_sc, f"{wl.name} refine scores g={g}")
        # refine select on the GPU's own scores, for these members (one group)
        own = O.refine_topk(q, k, w, cand_np[g:g + 1], len(members), wl.q_pos0 + members[0], K,
                            scores=rsc_s[sl].astype(np.float64))
        assert_same_sets(ridx_np[0, members], own, f"{wl.name} refine select g={g}")
    # recall of the grouped selections against the dense top-k (sampled queries)
    q, k, w = real_rows(inp, 0, dense_queries)
    dl = wl.q_pos0 + np.asarray(dense_queries)
    I = O.causal_scores(q, k, w, dl)
    dense = []
    for i in range(len(dense_queries)):
        r = O.select_topk(I[i, : dl[i] + 1], np.arange(dl[i] + 1), K)
        dense.append(np.pad(r, (0, K - len(r)), constant_values=-1))
    dense = np.array(dense)
    rec_ref = O.recall(ridx_np[0, dense_queries], dense)
    rec_reu = O.recall(uidx_np[0, dense_queries], dense)
    # Refine keeps every dense member that is a candidate (the candidate-coverage
    # identity), except where float32 and float64 order near-ties at the k-th
    # score differently: a member it misses lies within twice the score
    # tolerance of the k-th dense score (with every score within tolerance, K
    # candidates outscoring it on the GPU would otherwise all be dense members
    # besides it, one too many)
    dev_id = 0.0
    for i, t in enumerate(dense_queries):
        d_i = [int(x) for x in dense[i] if x >= 0]
        D = set(d_i)
        V = set(int(x) for x in cand_np[t // G] if 0 <= x <= wl.q_pos0 + t)
        Rf = set(int(x) for x in ridx_np[0, t] if x >= 0)
        tau = I[i, d_i[-1]]
        for s in (D & V) - Rf:
            assert abs(I[i, s] - tau) <= 2 * (ATOL + RTOL * abs(tau)), \
                f"query {t}: dense member {s} (score {I[i, s]}, k-th {tau}) is a candidate Refine missed"
        dev_id = max(dev_id, abs(rec_ref[i] - len(D & V) / len(D)))
    print(f"  Refine recall vs dense: mean {rec_ref.mean():.4f} min {rec_ref.min():.4f}; "
          f"Reuse recall: mean {rec_reu.mean():.4f}; identity deviation {dev_id:.2e}", flush=True)


def test_grouped_refine_bf16_L131072():
    wl = WORKLOADS["grouped_refine_bf16_L131072_G64_C8192_k2048"]
    n_g = wl.n_q // wl.group
    # (the full score dump of 131072 x 131072 float32 scores is 69 GB; at
    # 262144 tokens it would not fit beside the inputs)
    grouped_fullsize(wl, [0, 100, n_g // 2, n_g - 1],
                     [int(x) for x in np.linspace(wl.n_q // 8, wl.n_q - 1, 12)],
                     [4096, wl.n_q // 2, wl.n_q - 32], every_row_dump=True)


def test_grouped_fp8_L262144():
    wl = WORKLOADS["grouped_fp8_L262144_G128_C8192_k2048"]
    n_g = wl.n_q // wl.group
    grouped_fullsize(wl, [0, 50, n_g // 2, n_g - 1],
                     [int(x) for x in np.linspace(wl.n_q // 8, wl.n_q - 1, 8)],
                     [8192, wl.n_q // 2, wl.n_q - 32])
