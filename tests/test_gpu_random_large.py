"""GPU vs oracle parity on seeded random shapes at large sizes.

The shapes are drawn from a seeded generator: decode positions (1-4 queries
at the end of 40K-300K keys, up to 16 sequences: the split-key path and the
segmented list select) or prefill (3K-40K queries: the tiled scan with the
candidate filter), every storage combination, 16/32/64 heads, d = 64/128,
smooth, heavy-tailed or small-integer (tie-heavy) values, signed head
weights, and k from 1 to 20000 (every select length class).  Work per call
is capped so that each case runs in seconds.  Every output row is checked
for the invariants; sampled rows of the first and last sequence against the
oracle: scores within tolerance, the select bit-exact on the GPU's own
scores, banded set agreement with the oracle's own top-k, and the timed
(no score dump) path equal to the dump path.

Grouped shapes (PIVOT: proxy scan, Refine, Reuse) are drawn the same way,
with group sizes 1-256 or the decode grouping (the few queries at the end
of the keys as one group), candidate budgets from k + G - 1 to 4k + G, and
clustered keys besides; they run the full-size grouped checks (every row's
invariants, Reuse exact, sampled groups' proxy scores, candidates, Refine
scores and select against the oracle, the Refine candidate-coverage
identity up to near-ties).
"""

import gc

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.synth import Workload, make_inputs

from parity import (AGREEMENT, assert_same_sets, band_agreement, check_scores, cuda, real_rows,
                    score_magnitudes)
from test_gpu_fullsize import all_rows_valid, grouped_fullsize, sample_rows

pytestmark = pytest.mark.gpu

COMBOS = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")]


def _draw(rng, i):
    qf, kf = COMBOS[int(rng.integers(len(COMBOS)))]
    H = int(rng.choice([16, 32, 64]))
    d = int(rng.choice([64, 128]))
    if rng.random() < 0.5:  # decode positions
        B, n_q, n_k = int(rng.integers(1, 17)), int(rng.integers(1, 5)), int(rng.integers(40000, 300001))
    else:
        B, n_q = int(rng.integers(1, 3)), int(rng.integers(3000, 40001))
        n_k = n_q if rng.random() < 0.7 else int(rng.integers(n_q, n_q + 20000))
    pairs = (1e12 if qf == "f32" else 2e13) / (2 * H * d * B)  # causal pairs per call
    if n_q < 5:
        n_k = min(n_k, int(pairs / n_q))
    elif n_q * (n_k - n_q / 2) > pairs:
        n_q = n_k = int((2 * pairs) ** 0.5)
    kd = str(rng.choice(["normal8", "heavy", "int"]))
    qd = "int" if kd == "int" else str(rng.choice(["normal8", "ar1"]))
    wd = "int" if kd == "int" else str(rng.choice(["uniform", "uniform", "signed"]))
    r = rng.random()
    topk = int(rng.integers(1, 64) if r < 0.15 else rng.integers(64, 4097) if r < 0.85 else rng.integers(4097, 20001))
    name = f"rl{i}_B{B}_q{n_q}_k{n_k}_H{H}_d{d}_{qf}{kf}_{qd}-{kd}-{wd}_k{topk}"
    return Workload(name, B, n_q, n_k, H, d, qf, kf, qd, kd, rho=0.98 if qd == "ar1" else 0.0, topk=topk,
                    seed=23000 + i, w_dist=wd)


_RNG = np.random.default_rng(20261207)  # a draw that covers every class listed above
LARGE = [_draw(_RNG, i) for i in range(8)]


@pytest.mark.parametrize("wl", LARGE, ids=[w.name for w in LARGE])
def test_large_random_shape(wl):
    dev = cuda()
    print(f"\n[large] {wl.name}", flush=True)
    inp = make_inputs(wl, dev)
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    idx = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **a)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    del idx
    all_rows_valid(idx_np, wl)
    idx_d, sc = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, return_scores=True, **a)
    torch.cuda.synchronize()
    signed = wl.w_dist == "signed"
    rows = sample_rows(wl.n_q, 12) if wl.n_q > 4 else list(range(wl.n_q))
    rt = torch.as_tensor(rows, device=dev)
    for b in sorted({0, wl.batch - 1}):
        sc_b = sc[b].index_select(0, rt).cpu().numpy()
        idd = idx_d[b].index_select(0, rt).cpu().numpy()
        assert_same_sets(idx_np[b, rows], idd, f"{wl.name} b={b}: timed path vs dump path")
        q, k, w = real_rows(inp, b, rows)
        lim = wl.q_pos0 + np.asarray(rows)
        I = O.causal_scores(q, k, w, lim)
        M = score_magnitudes(q, k, w) if signed else None
        check_scores(sc_b, I, f"{wl.name} b={b}", mag=M)
        own = [O.select_topk(sc_b[i, : lim[i] + 1].astype(np.float64), np.arange(lim[i] + 1), wl.topk)
               for i in range(len(rows))]
        assert_same_sets(idd, own, f"{wl.name} b={b}: select on own scores")
        ora = [O.select_topk(I[i, : lim[i] + 1], np.arange(lim[i] + 1), wl.topk) for i in range(len(rows))]
        ora = np.array([np.pad(r, (0, wl.topk - len(r)), constant_values=-1) for r in ora])
        agr = band_agreement(idd, ora, I, mag_rows=M.max(axis=1) if signed else None)
        assert agr >= AGREEMENT, f"{wl.name} b={b}: set agreement {agr}"
    del sc, idx_d, inp
    gc.collect()
    torch.cuda.empty_cache()


def _draw_grouped(rng, i):
    qf, kf = COMBOS[int(rng.integers(len(COMBOS)))]
    H = int(rng.choice([16, 32, 64]))
    d = int(rng.choice([64, 128]))
    if rng.random() < 0.3:  # decode grouping
        n_q = int(rng.integers(1, 5))
        n_k, G = int(rng.integers(40000, 300001)), n_q
    else:
        n_q = int(rng.integers(3000, 70001))
        n_k = n_q if rng.random() < 0.7 else int(rng.integers(n_q, n_q + 20000))
        G = int(rng.choice([1, 2, 7, 16, 33, 64, 128, 256]))
    pairs = (1e12 if qf == "f32" else 2e13) / (2 * H * d)  # proxy-scan pairs per call
    if n_q >= 5 and n_q * (n_k - n_q / 2) / G > pairs:
        n_q = n_k = int((2 * pairs * G) ** 0.5)
    kd = str(rng.choice(["normal8", "heavy", "int", "clustered"]))
    qd = "int" if kd == "int" else str(rng.choice(["normal8", "ar1"]))
    K = int(rng.integers(1, 64) if rng.random() < 0.2 else rng.integers(64, 4097))
    C = int(rng.integers(K + G - 1, 4 * K + G + 1))
    kw = dict(rho=0.98 if qd == "ar1" else 0.0, topk=K, seed=24000 + i, w_dist="int" if kd == "int" else "uniform",
              group=G, n_cand=C)
    if kd == "clustered":
        kw.update(clusters=int(rng.integers(2, 512)), seed_stride=0)
    name = f"rlg{i}_q{n_q}_k{n_k}_H{H}_d{d}_{qf}{kf}_{qd}-{kd}_k{K}_G{G}_C{C}"
    return Workload(name, 1, n_q, n_k, H, d, qf, kf, qd, kd, **kw)


_RNG_G = np.random.default_rng(20261206)  # a draw that covers every class listed above
LARGE_GROUPED = [_draw_grouped(_RNG_G, i) for i in range(6)]


@pytest.mark.parametrize("wl", LARGE_GROUPED, ids=[w.name for w in LARGE_GROUPED])
def test_large_random_grouped_shape(wl):
    n_g = -(-wl.n_q // wl.group)
    groups = sorted({0, n_g // 3, n_g - 1})
    queries = sorted({int(x) for x in np.linspace(wl.n_q // 4, wl.n_q - 1, 5)})
    grouped_fullsize(wl, groups, queries)
    gc.collect()
    torch.cuda.empty_cache()
