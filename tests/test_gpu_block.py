"""GPU vs oracle parity of block-mean candidate routing (through the C ABI).

Chain, as for the proxy scan: the stored proxy and block means are the
rounded means; the block scores on the GPU's own proxy and means match the
oracle within the score tolerance; the routed candidates equal the oracle's
routing on the GPU's own block scores (exact, as sets); Refine over them is
valid and, with every block kept, equals the dense path.  Shapes cover the
tiled scan (many groups) and the split-key scan (at most four groups per
sequence), FP8 and float32 keys, blocks of 1 and ragged last blocks.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.synth import Workload, make_inputs

from parity import assert_same_sets, check_rows_valid, check_scores, check_stored_mean, cuda, real_inputs, sets

pytestmark = pytest.mark.gpu

# (workload, block, blocks kept)
CASES = [
    (Workload("blk_bf16_L1000_G16", 1, 1000, 1000, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
              topk=64, group=16, seed=31), 32, 6),
    (Workload("blk_fp8_L777_G64", 1, 777, 777, 64, 128, "fp8", "fp8", "ar1", "heavy", rho=0.99,
              topk=40, group=64, seed=32), 48, 4),
    (Workload("blk_f32_B2_L300_H16_d64_G5", 2, 300, 300, 16, 64, "f32", "f32", "normal8", "normal8",
              topk=11, group=5, seed=33), 7, 3),
    (Workload("blk_decode_bf16q_fp8k_B3_G2", 3, 2, 5000, 64, 128, "bf16", "fp8", "ar1", "heavy", rho=0.98,
              topk=100, group=2, seed=34), 64, 8),
    (Workload("blk_bf16_L400_G32_block1", 1, 400, 400, 32, 64, "bf16", "bf16", "normal8", "heavy",
              topk=20, group=32, seed=35), 1, 50),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_block_route_parity(case):
    wl, S_blk, n_sel = case
    dev = cuda()
    print(f"\n[block] {wl.name} block {S_blk} keep {n_sel}", flush=True)
    inp = make_inputs(wl, dev)
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    G = wl.group
    cand, km, bsc, pq, pw = S.block_route(inp["q"], inp["k"], inp["w"], G, S_blk, n_sel, return_means=True,
                                         return_scores=True, return_proxy=True, **a)
    cand_ws = S.block_route(inp["q"], inp["k"], inp["w"], G, S_blk, n_sel, **a)
    ridx = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, G, wl.topk, **a)
    torch.cuda.synchronize()
    srt = lambda x: torch.sort(x, dim=-1)[0]
    assert torch.equal(srt(cand), srt(cand_ws))  # dump path and workspace path agree
    q, k, w = real_inputs(inp)
    km_f = km.float().cpu().numpy().astype(np.float64)
    pq_f = pq.float().cpu().numpy().astype(np.float64)
    pw_f = pw.cpu().numpy().astype(np.float64)
    cand, bsc, ridx = cand.cpu().numpy(), bsc.cpu().numpy(), ridx.cpu().numpy()
    lim = O.proxy_limits(wl.n_q, G, wl.q_pos0)
    for b in range(wl.batch):
        # block means and proxy: the rounded means
        mean = O.block_means(k[b], S_blk)
        qb, wb = O.proxy_means(q[b], w[b], G)
        kfmt = "f32" if wl.k_fmt == "f32" else "bf16"
        qfmt = "f32" if wl.q_fmt == "f32" else "bf16"
        bb = [(j, min(j + S_blk, wl.n_k)) for j in range(0, wl.n_k, S_blk)]
        check_stored_mean(km_f[b], O.round_proxy(mean, wb, kfmt)[0], k[b], bb, kfmt, f"block means b={b}")
        check_stored_mean(pq_f[b], O.round_proxy(qb, wb, qfmt)[0], q[b], O.group_bounds(wl.n_q, G), qfmt,
                          f"proxy b={b}")
        # block scores on the GPU's own proxy and block means
        c_ora, B_ora, _ = O.block_route(pq_f[b], pw_f[b], km_f[b], lim, wl.n_k, S_blk, n_sel)
        check_scores(bsc[b], B_ora, f"{wl.name} block scores b={b}")
        # routing on the GPU's own block scores: exact (as sets)
        c_own = []
        n_full = (lim + 1) // S_blk
        for g in range(cand.shape[1]):
            f = int(n_full[g])
            top = O.select_topk(bsc[b, g, :f].astype(np.float64), np.arange(f), n_sel)
            keys = [np.arange(j * S_blk, (j + 1) * S_blk) for j in top]
            keys.append(np.arange(f * S_blk, int(lim[g]) + 1))
            c_own.append(np.concatenate(keys))
        assert_same_sets(cand[b], c_own, f"{wl.name} candidates b={b}")
        # Refine over the routed candidates: causal, distinct, -1 padded
        check_rows_valid(ridx[b], wl.q_pos0 + np.arange(wl.n_q), wl.topk)
        for t in range(wl.n_q):
            got = sets(ridx[b, t : t + 1])[0]
            assert got <= sets(cand[b, t // G : t // G + 1])[0]


def test_all_blocks_kept_equals_dense():
    dev = cuda()
    wl = Workload("blk_all_bf16_L300_G20", 1, 300, 300, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
                  topk=24, group=20, seed=36)
    inp = make_inputs(wl, dev)
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    cand = S.block_route(inp["q"], inp["k"], inp["w"], wl.group, 16, 300 // 16, **a)
    refine = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, wl.group, wl.topk, **a)
    dense = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    torch.cuda.synchronize()
    assert_same_sets(refine.cpu().numpy()[0], dense.cpu().numpy()[0], "refine(all blocks) vs dense")


def test_calibration_sweep_small():
    """The (G, C) / block / IVF sweep runs end to end: dense recall 1, every recall in [0, 1],
    and a budget that covers the whole prefix recovers the dense top-k exactly."""
    from sparse_attention_token_causal_amd.calibrate import choose, sweep
    cuda()
    L = 1024
    rows = sweep(L, [(16, 256), (16, L)], [(16, 32, 8), (16, 32, L // 32)],
                 [(16, 32, 256, 2, 128, 512), (16, 32, 256, 2, 128, L)], reps=1)
    assert rows[0]["path"] == "dense" and rows[0]["recall_mean"] == 1.0
    for r in rows:
        assert 0.0 <= r["recall_min"] <= r["recall_mean"] <= 1.0 and r["ms"] > 0
    full = [r for r in rows if r["budget"] >= L and r["path"] != "dense"]
    assert full and all(r["recall_min"] == 1.0 for r in full)
    assert choose(rows, 1.0) is not None
    assert any(r["path"] == "ivf-refine" and r["build_ms"] > 0 for r in rows)
