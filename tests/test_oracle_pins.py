"""Pins for the CPU oracle: values and identities fixed by the definitions and by
mathematics, not by the oracle itself.

* a hand-worked four-token example (tests/golden/hand_L4_H2_d2.json);
* a literal pure-Python brute force on tiny integer inputs (exact in float64,
  with frequent ties, so the tie rule is exercised);
* closed forms (recency, all-ties, all-zero, one head, positive scaling);
* a special case that reduces to library routines (non-negative q and k:
  ReLU is the identity, the score is one matmul and a stable argsort is the
  select);
* invariants (causal, distinct, counts, order, Refine with the whole prefix =
  dense, Reuse = Refine = dense at group size 1, Refine recall identity,
  recall monotone in the candidate budget);
* format decoders against torch's own conversions and the OCP FP8 table;
* mutation checks: plausible mistakes planted in a copy of the oracle's
  steps are caught by these pins.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# literal brute force (pure Python)


def bf_score(q, k, w, t, s):
    total = 0.0
    for h in range(len(q[t])):
        dot = 0.0
        for j in range(len(k[s])):
            dot += q[t][h][j] * k[s][j]
        total += w[t][h] * (dot if dot > 0 else 0.0)
    return total


def bf_select(pairs, kk):
    """pairs: list of (score, index)."""
    return [s for (_, s) in sorted(pairs, key=lambda p: (-p[0], p[1]))[:kk]]


def bf_dense(q, k, w, q_pos0, kk):
    out = []
    for t in range(len(q)):
        pairs = [(bf_score(q, k, w, t, s), s) for s in range(q_pos0 + t + 1)]
        out.append(bf_select(pairs, kk))
    return out


def bf_groups(n_q, G):
    return [list(range(a, min(a + G, n_q))) for a in range(0, n_q, G)]


def bf_proxy(q, w, members):
    H, d = len(q[0]), len(q[0][0])
    n = len(members)
    qb = [[sum(q[t][h][j] for t in members) / n for j in range(d)] for h in range(H)]
    wb = [sum(w[t][h] for t in members) / n for h in range(H)]
    return qb, wb


def bf_grouped(q, k, w, q_pos0, G, C, kk, variant):
    out = [None] * len(q)
    for members in bf_groups(len(q), G):
        qb, wb = bf_proxy(q, w, members)
        lim = q_pos0 + members[-1]
        pairs = [(bf_score([qb], k, [wb], 0, s), s) for s in range(lim + 1)]
        if variant == "refine":
            cand = bf_select(pairs, C)
            for t in members:
                v = [c for c in cand if c <= q_pos0 + t]
                out[t] = bf_select([(bf_score(q, k, w, t, c), c) for c in v], kk)
        else:
            top = bf_select(pairs, kk)
            for t in members:
                out[t] = [c for c in top if c <= q_pos0 + t]
    return out


def as_sets(rows):
    return [sorted(int(x) for x in r if x >= 0) for r in rows]


def tiny_int_case(rng, n_q, n_k, H, d, lo=-2, hi=3):
    q = rng.integers(lo, hi, size=(n_q, H, d)).astype(np.float64)
    k = rng.integers(lo, hi, size=(n_k, d)).astype(np.float64)
    w = rng.integers(0, 3, size=(n_q, H)).astype(np.float64)
    return q, k, w


# ----------------------------------------------------------------------------
# the hand-worked example


@pytest.fixture(scope="module")
def hand():
    with open(os.path.join(GOLDEN, "hand_L4_H2_d2.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)
    k = np.array(g["k"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    return g, q, k, w


def test_hand_scores(hand):
    g, q, k, w = hand
    I = O.dense_scores(q, k, w, 0)
    for t, row in enumerate(g["scores"]):
        for s, v in enumerate(row):
            if v is None:
                assert I[t, s] == -np.inf
            else:
                assert I[t, s] == v


@pytest.mark.parametrize("kk", [1, 2, 3])
def test_hand_dense_topk(hand, kk):
    g, q, k, w = hand
    out = O.dense_topk(q, k, w, 0, kk)
    exp = g["dense_topk"][str(kk)]
    for t in range(4):
        assert [int(x) for x in out[t] if x >= 0] == exp[t]  # rank order too


def test_hand_decode_positions(hand):
    g, q, k, w = hand
    out = O.dense_topk(q[2:], k, w[2:], 2, 2)
    assert out.tolist() == g["decode_q_pos0_2"]["topk_2"]


def test_hand_grouped(hand):
    g, q, k, w = hand
    G = g["group"]
    qb, wb = O.proxy_means(q, w, G)
    assert np.array_equal(qb, np.array(g["proxy_q"]))
    assert np.array_equal(wb, np.array(g["proxy_w"]))
    lim = O.proxy_limits(4, G, 0)
    assert lim.tolist() == [1, 3]
    P = O.proxy_scores(qb, wb, k, lim)
    for r, row in enumerate(g["proxy_scores"]):
        for s, v in enumerate(row):
            assert (P[r, s] == -np.inf) if v is None else (P[r, s] == v)
    for C in (2, 3):
        assert O.proxy_candidates(P, lim, C).tolist() == g["candidates"][str(C)]
    cand2 = O.proxy_candidates(P, lim, 2)
    cand3 = O.proxy_candidates(P, lim, 3)
    for key, cand, kk in (("C2_k1", cand2, 1), ("C2_k2", cand2, 2), ("C3_k2", cand3, 2)):
        out = O.refine_topk(q, k, w, cand, G, 0, kk)
        assert [[int(x) for x in r if x >= 0] for r in out] == g["refine"][key]
    out = O.reuse_topk(cand2, G, 0, 4, 2)
    assert [[int(x) for x in r if x >= 0] for r in out] == g["reuse_k2"]
    # the whole pipeline (proxy values are exact in bf16 here)
    for fmt in ("f32", "bf16"):
        o, c, _, _ = O.grouped_reference(q, k, w, 0, G, 3, 2, "refine", fmt)
        assert [[int(x) for x in r if x >= 0] for r in o] == g["refine"]["C3_k2"]
        o, c, _, _ = O.grouped_reference(q, k, w, 0, G, 0, 2, "reuse", fmt)
        assert [[int(x) for x in r if x >= 0] for r in o] == g["reuse_k2"]


# ----------------------------------------------------------------------------
# brute force on tiny integer inputs


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_dense(seed):
    rng = np.random.default_rng(seed)
    n_k = int(rng.integers(1, 48))
    n_q = int(rng.integers(1, n_k + 1))
    H, d = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    q, k, w = tiny_int_case(rng, n_q, n_k, H, d)
    for q_pos0 in sorted({0, n_k - n_q}):
        if q_pos0 + n_q > n_k:
            continue
        I = O.dense_scores(q, k, w, q_pos0)
        for t in range(n_q):
            for s in range(n_k):
                if s <= q_pos0 + t:
                    assert I[t, s] == bf_score(q.tolist(), k.tolist(), w.tolist(), t, s)
                else:
                    assert I[t, s] == -np.inf
        for kk in sorted({1, 3, 7, n_k}):
            got = O.dense_topk(q, k, w, q_pos0, kk)
            exp = bf_dense(q.tolist(), k.tolist(), w.tolist(), q_pos0, kk)
            assert [[int(x) for x in r if x >= 0] for r in got] == exp


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("variant", ["refine", "reuse"])
def test_brute_force_grouped(seed, variant):
    rng = np.random.default_rng(100 + seed)
    n_q = int(rng.integers(1, 40))
    n_k = n_q + int(rng.integers(0, 8))
    H, d = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    q, k, w = tiny_int_case(rng, n_q, n_k, H, d)
    q_pos0 = n_k - n_q
    # group sizes 1, 2, 4 (partial groups of 1..3): with q in multiples of 12 and
    # w in multiples of 12 every proxy mean is an exact float32, so the stored
    # proxy equals the brute force's exact mean
    q, w = q * 12.0, w * 12.0
    for G in (1, 2, 4):
        for kk in (1, 3, 7):
            for C in sorted({kk, kk + G - 1, n_k}):
                out, _, _, _ = O.grouped_reference(q, k, w, q_pos0, G, C, kk, variant, "f32")
                exp = bf_grouped(q.tolist(), k.tolist(), w.tolist(), q_pos0, G, C, kk, variant)
                assert [[int(x) for x in r if x >= 0] for r in out] == exp


# ----------------------------------------------------------------------------
# closed forms


def test_recency_closed_form():
    L = 37
    q = np.ones((L, 1, 1))
    k = np.arange(L, dtype=np.float64).reshape(L, 1)
    w = np.ones((L, 1))
    for kk in (1, 5, L):
        out = O.dense_topk(q, k, w, 0, kk)
        for t in range(L):
            e = min(kk, t + 1)
            assert sorted(out[t][:e].tolist()) == list(range(t + 1 - e, t + 1))
            assert (out[t][e:] == -1).all()


@pytest.mark.parametrize("how", ["equal_keys", "zero_query", "negated"])
def test_all_ties_closed_form(how):
    rng = np.random.default_rng(7)
    L, H, d = 29, 3, 5
    q = rng.normal(size=(L, H, d))
    k = np.tile(rng.normal(size=(1, d)), (L, 1))
    w = rng.uniform(size=(L, H))
    if how == "zero_query":
        q[:] = 0.0
        k = rng.normal(size=(L, d))
    if how == "negated":
        q = np.abs(q)
        k = -np.abs(rng.normal(size=(L, d)))  # every q.k < 0 -> every score is 0
    for kk in (1, 4, L):
        out = O.dense_topk(q, k, w, 0, kk)
        for t in range(L):
            assert out[t][: min(kk, t + 1)].tolist() == list(range(min(kk, t + 1)))
    if how == "negated":
        assert (O.dense_scores(q, k, w, 0)[np.tril_indices(L)] == 0).all()


def test_single_head_weight():
    rng = np.random.default_rng(3)
    L, H, d = 20, 4, 6
    q, k = rng.normal(size=(L, H, d)), rng.normal(size=(L, d))
    w = np.zeros((L, H))
    w[:, 2] = 1.7
    I = O.dense_scores(q, k, w, 0)
    for t in range(L):
        exp = 1.7 * np.maximum(k[: t + 1] @ q[t, 2], 0.0)
        assert np.allclose(I[t, : t + 1], exp, rtol=1e-14, atol=0)


def test_positive_scaling():
    rng = np.random.default_rng(4)
    L, H, d = 40, 3, 5
    q, k, w = rng.normal(size=(L, H, d)), rng.normal(size=(L, d)), rng.uniform(size=(L, H))
    c = 4.0  # a power of two keeps every product exact
    I1, I2 = O.dense_scores(q, k, w, 0), O.dense_scores(q, c * k, w, 0)
    assert np.array_equal(I2, c * I1)
    assert np.array_equal(O.dense_topk(q, k, w, 0, 9), O.dense_topk(q, c * k, w, 0, 9))


def test_nonnegative_reduces_to_matmul_and_stable_argsort():
    rng = np.random.default_rng(5)
    L, H, d = 64, 4, 8
    q = rng.integers(0, 3, size=(L, H, d)).astype(np.float64)
    k = rng.integers(0, 3, size=(L, d)).astype(np.float64)
    w = rng.integers(0, 4, size=(L, H)).astype(np.float64)
    qw = np.einsum("th,thd->td", w, q)  # sum_h w_h q_h (ReLU is the identity here)
    full = qw @ k.T
    I = O.dense_scores(q, k, w, 0)
    for kk in (1, 6, 64):
        out = O.dense_topk(q, k, w, 0, kk)
        for t in range(L):
            assert np.array_equal(I[t, : t + 1], full[t, : t + 1])
            ref = np.argsort(-full[t, : t + 1], kind="stable")[:kk]
            assert out[t][: len(ref)].tolist() == ref.tolist()


# ----------------------------------------------------------------------------
# invariants on random real-valued inputs


def random_case(seed, n_q, n_k, H=4, d=8):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(n_q, H, d)).astype(np.float32).astype(np.float64)
    k = rng.normal(size=(n_k, d)).astype(np.float32).astype(np.float64)
    w = rng.uniform(size=(n_q, H)).astype(np.float32).astype(np.float64)
    return q, k, w


@pytest.mark.parametrize("q_pos0", [0, 17])
def test_dense_invariants(q_pos0):
    n_q = 60
    q, k, w = random_case(11, n_q, n_q + q_pos0)
    kk = 13
    I = O.dense_scores(q, k, w, q_pos0)
    out = O.dense_topk(q, k, w, q_pos0, kk)
    for t in range(n_q):
        p = q_pos0 + t
        sel = out[t][out[t] >= 0]
        assert len(sel) == min(kk, p + 1)
        assert len(set(sel.tolist())) == len(sel)
        assert (sel <= p).all() and (sel >= 0).all()
        unsel = np.setdiff1d(np.arange(p + 1), sel)
        if unsel.size:
            # every selected entry precedes every unselected one in (-score, index) order
            worst_sel = min((I[t, s], -s) for s in sel)
            best_unsel = max((I[t, s], -s) for s in unsel)
            assert worst_sel > best_unsel


@pytest.mark.parametrize("G", [3, 8])
def test_refine_whole_prefix_equals_dense(G):
    n_q, kk = 50, 9
    q, k, w = random_case(12, n_q, n_q)
    dense = O.dense_topk(q, k, w, 0, kk)
    out, _, _, _ = O.grouped_reference(q, k, w, 0, G, n_q, kk, "refine", "f32")
    assert as_sets(out) == as_sets(dense)


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_group_size_one_reuse_refine_dense(fmt):
    n_q, kk = 45, 7
    q, k, w = random_case(13, n_q, n_q + 5)
    if fmt == "bf16":  # inputs representable in bf16 so the stored proxy equals the query
        q = O.bf16_bits_to_f64(O.f64_to_bf16_bits_rne(q))
    dense = O.dense_topk(q, k, w, 5, kk)
    ref, _, _, _ = O.grouped_reference(q, k, w, 5, 1, kk, kk, "refine", fmt)
    reu, _, _, _ = O.grouped_reference(q, k, w, 5, 1, kk, kk, "reuse", fmt)
    assert as_sets(ref) == as_sets(dense) == as_sets(reu)


def test_refine_recall_identity_and_monotone_in_C():
    n_q, kk, G = 64, 8, 8
    q, k, w = random_case(14, n_q, n_q)
    dense = O.dense_topk(q, k, w, 0, kk)
    prev = None
    for C in (8, 12, 20, 40, 64):
        out, cand, _, _ = O.grouped_reference(q, k, w, 0, G, C, kk, "refine", "f32")
        rec = O.recall(out, dense)
        for g, (a, b) in enumerate(O.group_bounds(n_q, G)):
            for t in range(a, b):
                V = set(int(c) for c in cand[g] if 0 <= c <= t)
                D = set(int(x) for x in dense[t] if x >= 0)
                assert rec[t] == len(D & V) / len(D)
                # counts: C >= k + G - 1 guarantees min(k, pos+1) survivors
                if C >= kk + G - 1:
                    assert (out[t] >= 0).sum() == min(kk, t + 1)
        if prev is not None:
            assert (rec >= prev).all()
        prev = rec
    assert (prev == 1.0).all()


def test_reuse_subset_of_proxy_topk():
    n_q, kk, G = 48, 6, 6
    q, k, w = random_case(15, n_q, n_q)
    out, top, _, _ = O.grouped_reference(q, k, w, 0, G, 0, kk, "reuse", "f32")
    for g, (a, b) in enumerate(O.group_bounds(n_q, G)):
        R = set(int(c) for c in top[g] if c >= 0)
        for t in range(a, b):
            sel = set(int(x) for x in out[t] if x >= 0)
            assert sel <= R and all(c <= t for c in sel)
            assert sel == set(c for c in R if c <= t)


def test_partial_last_group_and_short_prefix():
    n_q, kk, G, C = 23, 5, 4, 6  # 23 = 5 full groups + 3
    q, k, w = random_case(16, n_q, n_q)
    lim = O.proxy_limits(n_q, G, 0)
    assert lim.tolist() == [3, 7, 11, 15, 19, 22]
    out, cand, _, _ = O.grouped_reference(q, k, w, 0, G, C, kk, "refine", "f32")
    assert (cand[0] >= 0).sum() == 4  # C exceeds the first group's prefix
    assert out.shape == (n_q, kk)


# ----------------------------------------------------------------------------
# formats


def test_e4m3fn_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])


def test_e4m3fn_spot_values():
    # OCP 8-bit floating point specification, E4M3: bias 7, max normal 448, min subnormal 2^-9
    table = {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x3C: 1.5}
    vals = O.e4m3fn_bits_to_f64(np.array(list(table), dtype=np.uint8))
    assert vals.tolist() == list(table.values())
    assert np.isnan(O.e4m3fn_bits_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_bf16_decode_and_rne_against_torch():
    rng = np.random.default_rng(6)
    x = rng.normal(size=4096).astype(np.float32) * np.float32(3.0)
    # exact halfway cases in [1, 2) and [2^-100, 2^-99): low 16 bits 0x8000 under
    # every 7-bit retained mantissa (even and odd retained lsb)
    m7 = np.arange(128, dtype=np.uint32) << np.uint32(16)
    hw = (np.uint32(0x3F800000) | m7 | np.uint32(0x8000)).view(np.float32)
    hw_odd = (np.uint32(0x0D800000) | m7 | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, hw, hw_odd])
    ours = O.f64_to_bf16_bits_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = O.bf16_bits_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_real_values_scale():
    codes = np.array([[[0x38, 0x40]], [[0xB8, 0x00]]], dtype=np.uint8)  # [token=2, 1, d=2]
    scale = np.array([[0.5], [2.0]], dtype=np.float32)
    v = O.real_values(codes, "fp8", scale)
    assert v.tolist() == [[[0.5, 1.0]], [[-2.0, 0.0]]]


# ----------------------------------------------------------------------------
# block-mean routing ("AttentionIndex Architecture ...", "Why Positional Blocks
# Lose Recall" and its worked example)


def bf_block_route(q, k, w, q_pos0, G, S, n_sel, kk):
    """Literal loops: proxy, block means, routable complete blocks, top blocks
    by (-score, j), their keys plus the trailing partial block, then Refine."""
    n_k = len(k)
    out = [None] * len(q)
    cands = []
    for members in bf_groups(len(q), G):
        qb, wb = bf_proxy(q, w, members)
        lim = q_pos0 + members[-1]
        n_full = (lim + 1) // S
        pairs = []
        for j in range(n_full):
            rows = list(range(j * S, min(j * S + S, n_k)))
            mean = [sum(k[s][c] for s in rows) / len(rows) for c in range(len(k[0]))]
            pairs.append((bf_score([qb], [mean], [wb], 0, 0), j))
        blocks = bf_select(pairs, n_sel)
        cand = [s for j in blocks for s in range(j * S, j * S + S)] + list(range(n_full * S, lim + 1))
        cands.append(sorted(cand))
        for t in members:
            v = [c for c in cand if c <= q_pos0 + t]
            out[t] = bf_select([(bf_score(q, k, w, t, c), c) for c in v], kk)
    return out, cands


def block_case(q, k, w, q_pos0, G, S, n_sel, kk):
    out, cand, _, _ = O.block_reference(q, k, w, q_pos0, G, S, n_sel, kk, "f32", "f32")
    return as_sets(out), as_sets(cand)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_block_route(seed):
    rng = np.random.default_rng(200 + seed)
    n_q = int(rng.integers(1, 40))
    n_k = n_q + int(rng.integers(0, 9))
    H, d = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    q, k, w = tiny_int_case(rng, n_q, n_k, H, d)
    # multiples of 12 make every proxy mean and every block mean (blocks of 1,
    # 2, 3, 4; partial last blocks) exact in float32
    q, k, w = q * 12.0, k * 12.0, w * 12.0
    q_pos0 = n_k - n_q
    for G in (1, 2, 4):
        for S in (1, 2, 3, 4):
            for n_sel in (1, 2, 5):
                for kk in (1, 3):
                    got = block_case(q, k, w, q_pos0, G, S, n_sel, kk)
                    exp_out, exp_cand = bf_block_route(q.tolist(), k.tolist(), w.tolist(), q_pos0, G, S,
                                                       n_sel, kk)
                    assert got == (as_sets(exp_out), exp_cand)


def test_block_size_one_is_the_proxy_scan():
    """With one key per block every block is complete and its mean is the key:
    the routed candidates are the proxy's top-n_sel."""
    rng = np.random.default_rng(11)
    q, k, w = tiny_int_case(rng, 24, 30, 2, 3)
    q, w = q * 12.0, w * 12.0
    for G, n_sel in ((1, 4), (3, 5), (8, 7)):
        qb, wb = O.proxy_means(q, w, G)
        lim = O.proxy_limits(24, G, 6)
        ref = O.proxy_candidates(O.proxy_scores(qb, wb, k, lim), lim, n_sel)
        cand, _, _ = O.block_route(qb, wb, O.block_means(k, 1), lim, 30, 1, n_sel)
        assert as_sets(cand) == as_sets(ref)


def test_all_blocks_kept_is_dense():
    """Keeping every complete block (plus the partial tail) covers the whole
    prefix, so Refine over it equals the dense top-k."""
    rng = np.random.default_rng(12)
    q, k, w = tiny_int_case(rng, 30, 30, 2, 3)
    for S in (1, 4, 7):
        out, cand, _, _ = O.block_reference(q, k, w, 0, 6, S, 30, 5, "f32", "f32")
        assert as_sets(out) == as_sets(O.dense_topk(q, k, w, 0, 5))
        for g, (a, b) in enumerate(O.group_bounds(30, 6)):
            assert as_sets(cand[g : g + 1]) == [list(range(b))]


def test_block_mean_hides_a_strong_key():
    """The failure mode the pages describe: one high-scoring key in a block of
    low ones ranks the block low on its mean, so routing to one block drops it."""
    q = np.ones((1, 1, 1))
    w = np.ones((1, 1))
    k = np.array([[10.0], [-10.0], [-10.0], [-10.0], [1.0], [1.0], [1.0], [1.0]])
    out, cand, B, sel = O.block_reference(q, k, w, 7, 1, 4, 1, 1, "f32", "f32")
    assert B[0].tolist() == [0.0, 1.0]            # relu(-2.5) and relu(1.0)
    assert sel[0].tolist() == [1]
    assert as_sets(cand) == [[4, 5, 6, 7]]
    assert as_sets(O.dense_topk(q, k, w, 7, 1)) == [[0]]
    assert as_sets(out) == [[4]]


def test_partial_block_is_not_routable():
    """A block that reaches past the group's last member is not ranked (its mean
    would include future keys); its visible keys are candidates anyway."""
    q = np.ones((1, 1, 1))
    w = np.ones((1, 1))
    k = np.array([[1.0], [1.0], [1.0], [5.0], [100.0], [100.0]])  # the future keys are large
    _, cand, B, sel = O.block_reference(q, k, w, 4, 1, 3, 1, 1, "f32", "f32")
    assert np.isneginf(B[0, 1]) and sel[0].tolist() == [0]
    assert as_sets(cand) == [[0, 1, 2, 3, 4]]


# ----------------------------------------------------------------------------
# mutation checks: each plausible mistake below is caught by a pin above


def _mut_dense(q, k, w, q_pos0, kk, mistake):
    n_q = q.shape[0]
    rows = []
    for t in range(n_q):
        p = q_pos0 + t + (0 if mistake != "exclusive" else -1)
        if p < 0:
            rows.append([])
            continue
        x = k[: p + 1] @ q[t].T
        if mistake == "no_relu":
            v = x @ w[t]
        elif mistake == "abs":
            v = np.abs(x) @ w[t]
        elif mistake == "w_transposed":
            v = np.maximum(x, 0) @ w[(t + 1) % n_q]
        else:
            v = np.maximum(x, 0) @ w[t]
        idx = np.arange(p + 1)
        if mistake == "ties_high":
            order = np.lexsort((-idx, -v))
        elif mistake == "ascending":
            order = np.lexsort((idx, v))
        else:
            order = np.lexsort((idx, -v))
        rows.append(idx[order[:kk]].tolist())
    return rows


@pytest.mark.parametrize("mistake", ["exclusive", "no_relu", "abs", "w_transposed", "ties_high",
                                     "ascending"])
def test_pins_catch_planted_mistakes(mistake, hand):
    g, q, k, w = hand
    caught = False
    for kk in (1, 2, 3):
        if _mut_dense(q, k, w, 0, kk, mistake) != g["dense_topk"][str(kk)]:
            caught = True
    for seed in range(4):
        rng = np.random.default_rng(seed)
        qq, kk_, ww = tiny_int_case(rng, 20, 20, 2, 3)
        exp = bf_dense(qq.tolist(), kk_.tolist(), ww.tolist(), 0, 5)
        if _mut_dense(qq, kk_, ww, 0, 5, mistake) != exp:
            caught = True
    assert caught, mistake
