"""Pins for the oracle's IVF routing with causal index versions.

Source: "AttentionIndex Architecture ..." (globaltechdigest.blogspot.com),
"KEY FINDINGS", "An Inverted File With Causal Versions" and "Worked Example:
Blocks Lose, Clusters Win".  The oracle's readings are listed in its IVF
section; these tests fix them without going through its code:

* a literal pure-Python brute force (k-means by loops, version windows, insert
  batches, the budget walk, then Refine) on tiny integer inputs, where every
  distance and score is exact in float64, so ties are frequent and decided by
  the tie rules;
* identities: one cluster per key (the first version's k-means keeps every key
  as its own centroid) reduces routing to the proxy scan over the refit
  window; a budget that holds the whole prefix makes Refine the dense top-k;
  with no version every prefix key is a candidate;
* causality: a version does not change when keys outside its window change,
  and no group ever receives a key beyond its last member;
* k-means itself: on well-separated groups one Lloyd iteration recovers the
  groups and their means; the objective never increases over iterations;
* the failure mode the page contrasts: on similarity groups scattered over
  positions, cluster routing at the budget of two groups keeps the query's
  group whole where block routing at the same budget does not;
* mutation checks: plausible mistakes planted in a copy of the routing and
  build steps are caught by the brute force.
"""

import numpy as np
import pytest

import oracle as O

from test_oracle_pins import as_sets, bf_groups, bf_proxy, bf_score, bf_select, tiny_int_case


def f32(x):
    return float(np.float32(x))


# ----------------------------------------------------------------------------
# literal brute force (pure Python lists; centroids stored as float32)


def bf_nearest(x, cents):
    def dist(a, b):
        return sum((u - v) * (u - v) for u, v in zip(a, b))
    best = 0
    for c in range(1, len(cents)):
        if dist(x, cents[c]) < dist(x, cents[best]):
            best = c
    return best


def bf_versions(k, m, R, T, mistake=None):
    """[(centroids, lists)] per version; lists[c] = keys of the version's window
    nearest to centroid c, in key order."""
    n_k, d = len(k), len(k[0])
    cents = [[f32(x) for x in k[(c * R) // m]] for c in range(m)]
    out = []
    for u in range(1, n_k // R + 1):
        for _ in range(T):
            groups = [[] for _ in range(m)]
            for s in range(u * R + (1 if mistake == "refit_window" and u * R < n_k else 0)):
                groups[bf_nearest(k[s], cents)].append(s)
            for c in range(m):
                if groups[c]:
                    cents[c] = [f32(sum(k[s][j] for s in groups[c]) / len(groups[c])) for j in range(d)]
                elif mistake == "empty_zero":
                    cents[c] = [0.0] * d
        end = min((u + 1) * R, n_k)
        lists = [[] for _ in range(m)]
        for s in range(end):
            lists[bf_nearest(k[s], cents)].append(s)
        out.append(([list(c) for c in cents], lists))
    return out


def bf_route(qb, wb, versions, last, R, b, C, mistake=None):
    u = (last + 1) // R if mistake != "version_late" else last // R
    e = u * R + b * ((last + 1 - u * R) // b) if mistake != "batch_ignored" else u * R
    if u == 0 and mistake != "batches_without_version":
        e = 0
    cand = list(range(e, last + 1))
    room = C - len(cand)
    if u >= 1:
        cents, lists = versions[u - 1]
        pairs = [(bf_score([qb], [cents[c]], [wb], 0, 0), c) for c in range(len(cents))]
        if mistake == "ties_high":
            order = [c for (_, c) in sorted(pairs, key=lambda p: (-p[0], -p[1]))]
        else:
            order = bf_select(pairs, len(cents))
        for c in order:
            vis = [s for s in lists[c] if s < e]
            if len(vis) > room:
                if mistake == "skip_not_stop":
                    continue
                break
            cand += vis
            room -= len(vis)
    return sorted(cand)


def bf_ivf(q, k, w, q_pos0, G, m, R, T, b, C, kk, mistake=None):
    versions = bf_versions(k, m, R, T, mistake)
    out = [None] * len(q)
    cands = []
    for members in bf_groups(len(q), G):
        qb, wb = bf_proxy(q, w, members)
        cand = bf_route(qb, wb, versions, q_pos0 + members[-1], R, b, C, mistake)
        cands.append(cand)
        for t in members:
            v = [c for c in cand if c <= q_pos0 + t]
            out[t] = bf_select([(bf_score(q, k, w, t, c), c) for c in v], kk)
    return out, cands


def ivf_case(q, k, w, q_pos0, G, m, R, T, b, C, kk):
    out, cand, _, _ = O.ivf_reference(q, k, w, q_pos0, G, m, R, T, b, C, kk, "f32", "f32")
    return as_sets(out), as_sets(cand)


@pytest.mark.parametrize("seed", range(5))
def test_brute_force_ivf(seed):
    rng = np.random.default_rng(300 + seed)
    n_q = int(rng.integers(6, 30))
    n_k = n_q + int(rng.integers(0, 10))
    H, d = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    q, k, w = tiny_int_case(rng, n_q, n_k, H, d)
    q, w = q * 12.0, w * 12.0  # exact proxy means for groups of 1, 2, 3, 4
    q_pos0 = n_k - n_q
    for G in (1, 3, 4):
        for m, R in ((1, 3), (2, 4), (3, 5), (4, 4)):
            for T in (0, 1, 2):
                for b in sorted({1, 2, R}):
                    for C in (R, R + 3, n_k):
                        got = ivf_case(q, k, w, q_pos0, G, m, R, T, b, C, 2)
                        exp_out, exp_cand = bf_ivf(q.tolist(), k.tolist(), w.tolist(), q_pos0, G, m, R, T, b,
                                                   C, 2)
                        assert got == (as_sets(exp_out), exp_cand), (G, m, R, T, b, C)


def test_brute_force_lists_and_centroids():
    """The versions themselves (not only what routing makes of them)."""
    rng = np.random.default_rng(310)
    _, k, _ = tiny_int_case(rng, 1, 23, 1, 3)
    for m, R, T in ((3, 5, 1), (4, 6, 2), (2, 7, 3)):
        ora = O.ivf_build(k, m, R, T, "f32")
        bf = bf_versions(k.tolist(), m, R, T)
        assert len(ora) == len(bf) == 23 // R
        for (cent, a), (bc, lists) in zip(ora, bf):
            assert cent.tolist() == bc
            for c in range(m):
                assert np.nonzero(a == c)[0].tolist() == lists[c]


# ----------------------------------------------------------------------------
# identities and invariants


def test_one_cluster_per_key_is_the_proxy_scan():
    """m = R: the first version starts from every key of its window as its own
    centroid, so (distinct keys) each list holds one key and ranking clusters
    ranks those keys by the proxy's score.  With insert batches of R, the keys
    after the window are always candidates and the rest of the budget is the
    proxy's top keys of the window."""
    rng = np.random.default_rng(320)
    R, n_k = 16, 28
    k = rng.permutation(np.arange(-40, 40))[: n_k * 2].reshape(n_k, 2).astype(np.float64)
    q = rng.integers(-3, 4, size=(12, 2, 2)).astype(np.float64) * 12.0
    w = rng.integers(0, 3, size=(12, 2)).astype(np.float64) * 12.0
    q_pos0 = n_k - 12
    for G, C in ((1, 17), (4, 20), (12, 25)):
        qb, wb = O.round_proxy(*O.proxy_means(q, w, G), "f32")
        lim = O.proxy_limits(12, G, q_pos0)
        versions = O.ivf_build(k, R, R, 2, "f32")
        assert len(versions) == 1 and (versions[0][0] == k[:R]).all()
        cand, _, _ = O.ivf_route(qb, wb, versions, lim, R, R, C)
        P = O.proxy_scores(qb, wb, k, lim)
        for g in range(lim.size):
            tail = list(range(R, int(lim[g]) + 1))
            top = O.select_topk(P[g, :R], np.arange(R), C - len(tail))
            assert as_sets(cand[g : g + 1]) == [sorted(tail + top.tolist())]


@pytest.mark.parametrize("b", [1, 4, 8])
def test_whole_prefix_budget_is_dense(b):
    rng = np.random.default_rng(321)
    q, k, w = tiny_int_case(rng, 40, 40, 2, 3)
    out, cand, _, _ = O.ivf_reference(q, k, w, 0, 5, 3, 8, 2, b, 40, 4, "bf16", "bf16")
    assert as_sets(out) == as_sets(O.dense_topk(q, k, w, 0, 4))
    for g, (_, e) in enumerate(O.group_bounds(40, 5)):
        assert as_sets(cand[g : g + 1]) == [list(range(e))]


def test_no_version_routes_the_whole_prefix():
    rng = np.random.default_rng(322)
    q, k, w = tiny_int_case(rng, 9, 9, 2, 3)
    out, cand, S, versions = O.ivf_reference(q, k, w, 0, 2, 2, 10, 1, 1, 10, 3, "f32", "f32")
    assert versions == [] and np.isneginf(S).all()
    assert as_sets(out) == as_sets(O.dense_topk(q, k, w, 0, 3))
    assert as_sets(cand) == [list(range(e)) for (_, e) in O.group_bounds(9, 2)]


def test_versions_are_causal():
    """Version u reads keys [0, uR) to refit and lists keys [0, (u + 1) R):
    changing keys from position p on leaves every version whose window ends at
    or before p unchanged, and routing never hands a group a future key."""
    rng = np.random.default_rng(323)
    k = rng.standard_normal((70, 4))
    R, p = 10, 40
    base = O.ivf_build(k, 4, R, 2, "bf16")
    k2 = k.copy()
    k2[p:] = rng.standard_normal((70 - p, 4)) * 5.0
    changed = O.ivf_build(k2, 4, R, 2, "bf16")
    for u in range(1, p // R):  # windows [0, (u + 1) R) within [0, p)
        assert (base[u - 1][0] == changed[u - 1][0]).all()
        assert (base[u - 1][1] == changed[u - 1][1]).all()
    assert (base[p // R - 1][0] == changed[p // R - 1][0]).all()  # refit keys [0, p) unchanged
    q = rng.standard_normal((70, 2, 4))
    w = rng.random((70, 2))
    for G, b in ((1, 1), (7, 3), (16, 10)):
        _, cand, _, _ = O.ivf_reference(q, k, w, 0, G, 4, R, 1, b, 24, 5, "bf16", "bf16")
        lim = O.proxy_limits(70, G, 0)
        for g in range(lim.size):
            row = cand[g][cand[g] >= 0]
            assert row.size == np.unique(row).size and (row <= lim[g]).all()


def scattered_groups(rng, n_groups, size, d, spread=0.05):
    """Tight similarity groups whose members are scattered over positions; the
    keys at positions floor(c R / m) (the first version's initial centroids,
    R = n_groups * size, m = n_groups) come one from each group."""
    centers = rng.standard_normal((n_groups, d)) * 3.0
    owner = np.repeat(np.arange(n_groups), size)
    rng.shuffle(owner)
    seeds = np.arange(n_groups) * size
    # put group c's first member at the seed position c * size
    for c in range(n_groups):
        j = int(np.nonzero(owner == c)[0][0])
        owner[j], owner[seeds[c]] = owner[seeds[c]], owner[j]
    k = centers[owner] + spread * rng.standard_normal((owner.size, d))
    return k, owner, centers


def test_one_iteration_recovers_separated_groups():
    rng = np.random.default_rng(324)
    k, owner, _ = scattered_groups(rng, 8, 12, 6)
    for fmt in ("f32", "bf16"):
        (cent, a), = O.ivf_build(k, 8, 96, 1, fmt)
        for c in range(8):
            assert (a == c).tolist() == (owner == owner[c * 12]).tolist()
            assert np.allclose(cent[c], k[owner == owner[c * 12]].mean(axis=0), rtol=2 ** -7, atol=1e-6)


def test_lloyd_objective_does_not_increase():
    rng = np.random.default_rng(325)
    k = rng.standard_normal((150, 5))
    prev = np.inf
    for T in range(6):
        (cent, a), = O.ivf_build(k[:100], 7, 100, T, "f32")
        J = float(((k[:100] - cent[a]) ** 2).sum())
        assert J <= prev * (1 + 1e-6)
        prev = J
    # and each key sits at its nearest centroid
    d2 = ((k[:100, None, :] - cent[None]) ** 2).sum(axis=2)
    assert (d2[np.arange(100), a] == d2.min(axis=1)).all()


def test_clusters_keep_what_blocks_lose():
    """Similarity groups scattered over positions; a query close to one group.
    At a budget of two groups, cluster routing keeps all of that group's keys;
    block routing (blocks of one group's size, two kept) loses some."""
    rng = np.random.default_rng(326)
    k, owner, centers = scattered_groups(rng, 8, 12, 6)
    target = owner[0]
    q = (centers[target] + 0.2 * rng.standard_normal(6)).reshape(1, 1, 6)
    w = np.ones((1, 1))
    want = set(np.nonzero(owner == target)[0].tolist())
    _, cand, _, _ = O.ivf_reference(q, k, w, 95, 1, 8, 96, 1, 96, 24, 12, "f32", "f32")
    assert want <= set(as_sets(cand)[0])
    _, bcand, _, _ = O.block_reference(q, k, w, 95, 1, 12, 2, 12, "f32", "f32")
    assert not want <= set(as_sets(bcand)[0])


# ----------------------------------------------------------------------------
# mutation checks


@pytest.mark.parametrize("mistake", ["ties_high", "skip_not_stop", "version_late", "batch_ignored",
                                     "empty_zero", "refit_window", "batches_without_version"])
def test_ivf_pins_catch_planted_mistakes(mistake):
    """Each mistake, planted in the brute force's steps, changes some result on
    the brute-force grid: the pins would catch it in the oracle."""
    caught = False
    for seed in range(5):
        rng = np.random.default_rng(300 + seed)
        n_q = int(rng.integers(6, 30))
        n_k = n_q + int(rng.integers(0, 10))
        H, d = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        q, k, w = tiny_int_case(rng, n_q, n_k, H, d)
        q, w = q * 12.0, w * 12.0
        for G in (1, 3):
            for m, R in ((2, 4), (3, 5), (4, 4)):
                for T in (1, 2):
                    for b in (1, 2):
                        for C in (R, R + 3):
                            args = (q.tolist(), k.tolist(), w.tolist(), n_k - n_q, G, m, R, T, b, C, 2)
                            if bf_ivf(*args, mistake=mistake) != bf_ivf(*args):
                                caught = True
                                break
                        if caught:
                            break
                    if caught:
                        break
                if caught:
                    break
            if caught:
                break
        if caught:
            break
    assert caught, mistake
