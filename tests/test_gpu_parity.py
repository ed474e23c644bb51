"""GPU vs oracle parity on small workloads (every row checked), through the C ABI.

Sizes span several key tiles and query blocks and end on ragged tails; the
five storage/shape combinations of the kernels are all exercised, plus the
degenerate cases (one token, k = 1, k above the prefix, group size 1, group
larger than the sequence, decode positions).
"""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.synth import Workload, WORKLOADS, make_inputs

from parity import (AGREEMENT, assert_same_sets, band_agreement, check_rows_valid, check_scores, check_stored_mean,
                    cuda, real_inputs, score_magnitudes)

pytestmark = pytest.mark.gpu

DENSE = [
    WORKLOADS["prefill_f32_L1024_H16_d64_k128"],
    Workload("bf16_B2_L700_H64_d128", 2, 700, 700, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98, topk=128),
    Workload("bf16_L333_H32_d64", 1, 333, 333, 32, 64, "bf16", "bf16", "normal8", "normal8", topk=50, seed=1),
    Workload("f32_L200_H16_d128_k300", 1, 200, 200, 16, 128, "f32", "f32", "normal8", "normal8", topk=300, seed=2),
    Workload("decode_bf16q_fp8k_B3", 3, 2, 5000, 64, 128, "bf16", "fp8", "ar1", "heavy", rho=0.98, topk=256, seed=3),
    Workload("fp8_L600_H64_d128", 1, 600, 600, 64, 128, "fp8", "fp8", "ar1", "heavy", rho=0.99, topk=100, seed=4),
    Workload("decode_bf16_B2_nq4_H16_d64", 2, 4, 777, 16, 64, "bf16", "bf16", "normal8", "normal8", topk=33, seed=5),
    Workload("f32_nq150_nk300_H64_d64", 1, 150, 300, 64, 64, "f32", "f32", "normal8", "heavy", topk=16, seed=6),
    Workload("bf16_L1_k4", 1, 1, 1, 64, 128, "bf16", "bf16", "normal8", "normal8", topk=4, seed=7),
    Workload("bf16_L90_k1", 1, 90, 90, 32, 128, "bf16", "bf16", "normal8", "heavy", topk=1, seed=8),
    # tie-heavy rows: every score of a query equal (boundary bin beyond the LDS list
    # for prefixes above 2048 -> radix fallback), and small integers (many exact ties)
    Workload("ties_const_keys_L3000_k1000", 1, 3000, 3000, 32, 64, "bf16", "bf16", "normal8", "const",
             topk=1000, seed=9),
    Workload("ties_int_L2500_k300", 1, 2500, 2500, 16, 64, "bf16", "bf16", "int", "int", topk=300, seed=10,
             w_dist="int"),
    Workload("ties_int_f32_decode_B2_k700", 2, 3, 9000, 16, 64, "f32", "f32", "int", "int", topk=700,
             seed=11, w_dist="int"),
    # 64 heads take the candidate-filtering path: ties, and negative scores (signed weights)
    Workload("filter_ties_int_H64_L1500_k200", 1, 1500, 1500, 64, 128, "bf16", "bf16", "int", "int",
             topk=200, seed=12, w_dist="int"),
    Workload("filter_signed_w_H64_L1200_k150", 1, 1200, 1200, 64, 128, "bf16", "bf16", "ar1", "heavy",
             rho=0.98, topk=150, seed=13, w_dist="signed"),
    Workload("filter_fp8_B2_L900_H64_k64", 2, 900, 900, 64, 128, "fp8", "fp8", "ar1", "heavy", rho=0.99,
             topk=64, seed=14),
    # rows with more candidates than their list holds (scores growing along
    # the key axis; every score of a query tied): the overflowed row blocks
    # are rescanned, narrowing the boundary interval digit by digit, and a
    # tied class is cut to its lowest key indices
    Workload("filter_overflow_ramp_H64_L6000_k100", 1, 6000, 6000, 64, 128, "bf16", "bf16", "normal8", "ramp",
             topk=100, seed=21),
    Workload("filter_overflow_ramp_fp8_B2_L4000_k64", 2, 4000, 4000, 64, 128, "fp8", "fp8", "ar1", "ramp",
             rho=0.99, topk=64, seed=22),
    Workload("filter_overflow_tied_H64_L5000_k300", 1, 5000, 5000, 64, 128, "bf16", "bf16", "normal8", "const",
             topk=300, seed=23),
    Workload("filter_overflow_int_H64_L4500_k40", 1, 4500, 4500, 64, 64, "bf16", "bf16", "int", "int",
             topk=40, seed=24, w_dist="int"),
    # every 16th key 2^20 times larger: the first tile's spikes place the
    # histogram window far above the other keys, which are all clamped into
    # its lowest bin; rows of up to about 270 keys record that edge bin as
    # their boundary (the one-wave select's open-ended lower bin), longer
    # rows take the general select
    Workload("filter_spikes_H64_L600_k50", 1, 600, 600, 64, 128, "bf16", "bf16", "normal8", "spikes",
             topk=50, seed=27),
    # at most 4 rows per sequence take the split-key scan + histogram compaction:
    # fp8 x fp8 with a partly empty row-wave, d = 64, ties, k near the prefix
    Workload("split_fp8_B2_nq3_H32_d128", 2, 3, 4099, 32, 128, "fp8", "fp8", "ar1", "heavy", rho=0.99,
             topk=300, seed=15),
    Workload("split_bf16q_fp8k_nq1_H64_d64", 1, 1, 3001, 64, 64, "bf16", "fp8", "normal8", "heavy", topk=5,
             seed=16),
    Workload("split_ties_int_B2_nq2_H64_k700", 2, 2, 9000, 64, 128, "bf16", "bf16", "int", "int", topk=700,
             seed=17, w_dist="int"),
    Workload("split_fp8_nq4_H16_d64_k2000", 1, 4, 2500, 16, 64, "fp8", "fp8", "normal8", "normal8",
             topk=2000, seed=18),
    # long candidate lists (k 1500 of 12000); then the split select's general
    # path: every score of a query ties (the threshold bin holds more entries
    # than the lean path keeps), and keys whose scores spread over more octaves
    # above the threshold than a chunk's histogram window covers (more than k
    # entries above the bin)
    Workload("split_lists_nq2_n12000_k1500", 1, 2, 12000, 64, 128, "bf16", "bf16", "normal8", "heavy",
             topk=1500, seed=19),
    Workload("split_ties_const_keys_nq2_n20000_k1100", 1, 2, 20000, 64, 128, "bf16", "bf16", "normal8", "const",
             topk=1100, seed=20),
    Workload("split_spikes_nq2_n20000_k2000", 1, 2, 20000, 64, 128, "bf16", "bf16", "normal8", "spikes",
             topk=2000, seed=21),
    Workload("split_spikes_fp8_B2_nq1_n9000_k700", 2, 1, 9000, 64, 128, "fp8", "fp8", "ar1", "spikes",
             rho=0.99, topk=700, seed=22),
    # rows longer than 32768 keys take the streaming select (rows re-read
    # from global memory): a spread row, tie-heavy rows, a row of equal
    # keys, and k beyond the row
    Workload("stream_nq8_n40000_H16_k1000", 1, 8, 40000, 16, 64, "bf16", "bf16", "normal8", "heavy",
             topk=1000, seed=23),
    Workload("stream_ties_int_nq6_n36000_H16_k3000", 1, 6, 36000, 16, 64, "bf16", "bf16", "int", "int",
             topk=3000, seed=24, w_dist="int"),
    Workload("stream_const_keys_nq5_n34000_H32_k700", 1, 5, 34000, 32, 64, "bf16", "bf16", "normal8", "const",
             topk=700, seed=25),
    Workload("stream_f32_nq5_n33000_H16_k40000", 1, 5, 33000, 16, 64, "f32", "f32", "normal8", "normal8",
             topk=40000, seed=26),
]


def args(inp, wl):
    return dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)


@pytest.mark.parametrize("wl", DENSE, ids=[w.name for w in DENSE])
def test_dense_parity(wl):
    dev = cuda()
    print(f"\n[dense] {wl.name}", flush=True)
    inp = make_inputs(wl, dev)
    idx, sc = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **args(inp, wl))
    idx_ws = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **args(inp, wl))
    torch.cuda.synchronize()
    idx, sc, idx_ws = idx.cpu().numpy(), sc.cpu().numpy(), idx_ws.cpu().numpy()
    # the timed path (workspace; candidate filtering for 64 heads) and the dump
    # path select the same sets (rows are sets: their order is unspecified)
    assert np.array_equal(np.sort(idx, axis=-1), np.sort(idx_ws, axis=-1))
    q, k, w = real_inputs(inp)
    worst = 0.0
    for b in range(wl.batch):
        I = O.dense_scores(q[b], k[b], w[b], wl.q_pos0)
        M = score_magnitudes(q[b], k[b], w[b]) if (w[b] < 0).any() else None
        worst = max(worst, check_scores(sc[b], I, f"{wl.name} b={b}", mag=M))
        # select on the GPU's own scores: bit-exact
        own = _select_rows(sc[b], wl.q_pos0, wl.topk)
        assert_same_sets(idx[b], own, f"{wl.name} b={b} select on own scores")
        lim = wl.q_pos0 + np.arange(wl.n_q)
        check_rows_valid(idx[b], lim, wl.topk, np.minimum(wl.topk, lim + 1))
        ora = O.dense_topk(q[b], k[b], w[b], wl.q_pos0, wl.topk, scores=I)
        agr = band_agreement(idx[b], ora, I, mag_rows=None if M is None else M.max(axis=1))
        assert agr >= AGREEMENT, f"{wl.name}: set agreement {agr}"
    print(f"  worst err/tol {worst:.3g}", flush=True)


def _select_rows(scores, q_pos0, topk):
    rows = []
    for t in range(scores.shape[0]):
        p = q_pos0 + t
        rows.append(O.select_topk(scores[t, : p + 1].astype(np.float64), np.arange(p + 1), topk))
    out = np.full((scores.shape[0], topk), -1, dtype=np.int64)
    for t, r in enumerate(rows):
        out[t, : len(r)] = r
    return out


def test_dense_is_deterministic():
    dev = cuda()
    wl = DENSE[1]
    inp = make_inputs(wl, dev)
    a = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **args(inp, wl))
    b = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **args(inp, wl))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_split_scan_is_deterministic():
    """The split-key path's scores are bit-reproducible and its sets stable
    (candidate lists are gathered with atomics, so only the order may vary)."""
    dev = cuda()
    wl = WORKLOADS["decode_fp8k_B8_mtp2_n131072_H64_d128_k2048"].scaled(n_k=20000, batch=2)
    inp = make_inputs(wl, dev)
    a = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **args(inp, wl))
    b = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **args(inp, wl))
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1])
    assert torch.equal(torch.sort(a[0], dim=-1)[0], torch.sort(b[0], dim=-1)[0])


GROUPED = [
    Workload("g_bf16_L777_G16_C200", 1, 777, 777, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
             topk=64, group=16, n_cand=200, seed=11),
    Workload("g_fp8_L500_G32_C150", 1, 500, 500, 64, 128, "fp8", "fp8", "ar1", "heavy", rho=0.99,
             topk=40, group=32, n_cand=150, seed=12),
    Workload("g_f32_B2_L300_H16_d64_G5_C37", 2, 300, 300, 16, 64, "f32", "f32", "normal8", "normal8",
             topk=11, group=5, n_cand=37, seed=13),
    Workload("g_decode_bf16q_fp8k_B3_G2", 3, 2, 5000, 64, 128, "bf16", "fp8", "ar1", "heavy", rho=0.98,
             topk=256, group=2, n_cand=512, seed=14),
    Workload("g_bf16_L30_G100", 1, 30, 30, 32, 64, "bf16", "bf16", "normal8", "heavy", topk=8, group=100,
             n_cand=12, seed=15),
    Workload("g_ties_int_L600_G8_C300", 1, 600, 600, 16, 64, "bf16", "bf16", "int", "int", topk=100, group=8,
             n_cand=300, seed=16, w_dist="int"),
    # two-query groups of 64 heads take 256-column key tiles; with 512 groups
    # the Refine scan gets one workgroup per group, and 6000 candidates'
    # indices beside those tiles would overflow the LDS: the columns are split
    Workload("g_G2_n1024_k7000_C6000", 1, 1024, 7000, 64, 128, "bf16", "bf16", "normal8", "heavy", topk=100,
             group=2, n_cand=6000, seed=17),
]


@pytest.mark.parametrize("wl", GROUPED, ids=[w.name for w in GROUPED])
def test_grouped_parity(wl):
    dev = cuda()
    print(f"\n[grouped] {wl.name}", flush=True)
    inp = make_inputs(wl, dev)
    a = args(inp, wl)
    G, C, K = wl.group, wl.n_cand, wl.topk
    cand, pq, pw, ps = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, C, return_proxy=True,
                                          return_scores=True, **a)
    ridx, rsc = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, K, return_scores=True, **a)
    ridx_ws = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, K, **a)
    cand_ws = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, C, **a)
    ptop = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], G, K, **a)
    uidx = S.reuse_topk(ptop, G, wl.n_q, wl.n_k, q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    # rows are sets (the split-key path gathers candidates with atomics, so
    # their order may differ between calls)
    srt = lambda x: torch.sort(x, dim=-1)[0]
    assert torch.equal(srt(ridx), srt(ridx_ws)) and torch.equal(srt(cand), srt(cand_ws))
    q, k, w = real_inputs(inp)
    pq_f = pq.float().cpu().numpy().astype(np.float64)
    pw_f = pw.cpu().numpy().astype(np.float64)
    cand, ps, ridx, rsc = cand.cpu().numpy(), ps.cpu().numpy(), ridx.cpu().numpy(), rsc.cpu().numpy()
    ptop, uidx = ptop.cpu().numpy(), uidx.cpu().numpy()
    n_g = -(-wl.n_q // G)
    lim = O.proxy_limits(wl.n_q, G, wl.q_pos0)
    for b in range(wl.batch):
        # G1: the stored proxy is the rounded mean
        qb, wb = O.proxy_means(q[b], w[b], G)
        qr, wr = O.round_proxy(qb, wb, synth_fmt(wl))
        gb = O.group_bounds(wl.n_q, G)
        check_stored_mean(pq_f[b], qr, q[b], gb, "f32" if wl.q_fmt == "f32" else "bf16", f"{wl.name} proxy q b={b}")
        check_stored_mean(pw_f[b], wr, w[b], gb, "f32", f"{wl.name} proxy w b={b}")
        # G2: proxy scores on the GPU's own proxy
        P = O.proxy_scores(pq_f[b], pw_f[b], k[b], lim)
        signed = (w[b] < 0).any()
        check_scores(ps[b], P, f"{wl.name} proxy scores b={b}",
                     mag=score_magnitudes(pq_f[b], k[b], pw_f[b]) if signed else None)
        # G3: candidates = oracle select on the GPU's proxy scores
        own = O.proxy_candidates(ps[b].astype(np.float64), lim, C)
        assert_same_sets(cand[b], own, f"{wl.name} candidates b={b}")
        check_rows_valid(cand[b], lim, C, np.minimum(C, lim + 1))
        # G4: refine scores per candidate slot
        I = O.dense_scores(q[b], k[b], w[b], wl.q_pos0)
        M = score_magnitudes(q[b], k[b], w[b]) if signed else None
        ref_sc = np.full((wl.n_q, C), -np.inf)
        ref_mag = np.zeros((wl.n_q, C))
        for t in range(wl.n_q):
            c = cand[b, t // G]
            ok = (c >= 0) & (c <= wl.q_pos0 + t)
            ref_sc[t, ok] = I[t, c[ok]]
            if signed:
                ref_mag[t, ok] = M[t, c[ok]]
        check_scores(rsc[b], ref_sc, f"{wl.name} refine scores b={b}", mag=ref_mag if signed else None)
        # G5: refine select on the GPU's own scores
        own = O.refine_topk(q[b], k[b], w[b], cand[b], G, wl.q_pos0, K, scores=rsc[b].astype(np.float64))
        assert_same_sets(ridx[b], own, f"{wl.name} refine select b={b}")
        check_rows_valid(ridx[b], wl.q_pos0 + np.arange(wl.n_q), K)
        # G6: agreement with the oracle's refine on oracle scores
        ora = O.refine_topk(q[b], k[b], w[b], cand[b], G, wl.q_pos0, K)
        agr = band_agreement(ridx[b], ora, I, mag_rows=M.max(axis=1) if signed else None)
        assert agr >= AGREEMENT, f"{wl.name}: refine agreement {agr}"
        # G7: reuse is integer work: exact, in the proxy's order
        ora_u = O.reuse_topk(ptop[b], G, wl.q_pos0, wl.n_q, K)
        assert np.array_equal(uidx[b], ora_u), f"{wl.name}: reuse differs"
        assert n_g == cand.shape[1]


def synth_fmt(wl):
    return wl.q_fmt


def test_group_size_one_matches_dense():
    dev = cuda()
    wl = Workload("g1_bf16_L300", 1, 300, 300, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98, topk=24,
                  seed=21)
    inp = make_inputs(wl, dev)
    a = args(inp, wl)
    dense = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    ptop = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], 1, wl.topk, **a)
    reuse = S.reuse_topk(ptop, 1, wl.n_q, wl.n_k, q_pos0=wl.q_pos0)
    cand = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], 1, 100, **a)
    refine = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, 1, wl.topk, **a)
    torch.cuda.synchronize()
    d, u, r = dense.cpu().numpy()[0], reuse.cpu().numpy()[0], refine.cpu().numpy()[0]
    # a bf16 query is its own bf16 proxy, so the proxy scan is the dense scan
    assert_same_sets(u, d, "reuse vs dense")
    assert_same_sets(r, d, "refine vs dense")


def test_refine_whole_prefix_equals_dense():
    dev = cuda()
    wl = Workload("wp_bf16_L256_G32", 1, 256, 256, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
                  topk=20, seed=22)
    inp = make_inputs(wl, dev)
    a = args(inp, wl)
    cand = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], 32, 256, **a)
    refine = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, 32, wl.topk, **a)
    dense = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    torch.cuda.synchronize()
    assert_same_sets(refine.cpu().numpy()[0], dense.cpu().numpy()[0], "refine(whole prefix) vs dense")


def test_refine_candidates_split_over_column_chunks():
    """A long caller-supplied candidate list (16700 slots, some empty) for one
    group of 64 queries: with so few query blocks the Refine scan splits the
    candidate columns over many workgroups, each staging its own slice of the
    key indices in LDS.  Scores per slot within tolerance of the oracle, the
    select bit-exact on the GPU's own scores, agreement with the oracle's
    Refine on its own scores."""
    dev = cuda()
    wl = Workload("refine_C16700_H16_d64", 1, 64, 17000, 16, 64, "bf16", "bf16", "normal8", "heavy",
                  topk=100, seed=23)
    print(f"\n[refine] {wl.name}", flush=True)
    inp = make_inputs(wl, dev)
    G, C, K = 64, 16700, wl.topk
    gen = torch.Generator(device="cpu").manual_seed(23)
    cand = torch.randperm(wl.n_k, generator=gen)[:C].to(torch.int32)
    cand[::97] = -1  # some empty slots
    cand = cand.view(1, 1, C).to(dev)
    ridx, rsc = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, K, return_scores=True, **args(inp, wl))
    torch.cuda.synchronize()
    ridx, rsc, c = ridx.cpu().numpy()[0], rsc.cpu().numpy()[0], cand.cpu().numpy()[0, 0].astype(np.int64)
    q, k, w = real_inputs(inp)
    ref_sc = np.full((wl.n_q, C), -np.inf)
    for t in range(wl.n_q):
        ok = (c >= 0) & (c <= wl.q_pos0 + t)
        ref_sc[t, ok] = np.maximum(k[0][c[ok]] @ q[0][t].T, 0.0) @ w[0][t]
    check_scores(rsc, ref_sc, f"{wl.name} refine scores")
    own = O.refine_topk(q[0], k[0], w[0], c[None], G, wl.q_pos0, K, scores=rsc.astype(np.float64))
    assert_same_sets(ridx, own, f"{wl.name} refine select on own scores")
    check_rows_valid(ridx, wl.q_pos0 + np.arange(wl.n_q), K)
    ora = O.refine_topk(q[0], k[0], w[0], c[None], G, wl.q_pos0, K)
    I = np.full((wl.n_q, wl.n_k), -np.inf)
    for t in range(wl.n_q):
        ok = (c >= 0) & (c <= wl.q_pos0 + t)
        I[t, c[ok]] = ref_sc[t, ok]
    agr = band_agreement(ridx, ora, I)
    assert agr >= AGREEMENT, f"{wl.name}: refine agreement {agr}"
