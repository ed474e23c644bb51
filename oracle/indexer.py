"""Plain float64 definition of the causal lightning indexer, dense and group-shared.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: one
query or one group at a time, one library matmul per step, no blocking or
fusion, so that each function can be checked by eye against what it cites.

Sources (web pages; cited by title and section):

* "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention"
  (aiqbench.com), Abstract: the indexer scores every preceding token of each
  query and keeps a per-query top-k; PIVOT forms fixed-size groups of
  consecutive queries, aggregates each group into one proxy query, does one
  shared full-prefix scan to a candidate set, and then either re-scores the
  candidates with each member's own indexer and selects each member's own
  top-k (Refine) or shares the proxy's top-k with the whole group (Reuse).
* "IndexCache: Accelerating Sparse Attention via Cross-Layer Index Reuse"
  (wispaper.ai), "The Quadratic Tax of Sparse Attention": the lightning
  indexer scores all preceding tokens to pick the top-k.
* "ADIndex Restructures Sparse-Attention Indexing with Group-Level
  Distillation" (zicq.com), "Why the Indexer Becomes the Bottleneck": the
  scan covers the whole causal prefix of every query, in prefill and decode.
* "MLI Restructures DeepSeek Sparse Attention ..." (zicq.com), "Core Idea":
  k = 2048 positions are kept per query.
* "AttentionIndex Architecture ..." (globaltechdigest.blogspot.com), "KEY
  FINDINGS": recall is measured against the exhaustive top-k.

Readings where the pages are silent (each is also listed in the design notes):

* Score.  No page prints the indexer's formula.  The reading is the DeepSeek
  lightning-indexer form I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]),
  with no extra constant (a positive constant would change no top-k).
* Causality.  "Preceding" is read inclusively: key s is visible to query t
  iff s <= pos(t) = q_pos0 + t (q_pos0 = 0 in prefill, n_k - n_q in decode,
  where the cache already holds the new tokens' keys).
* Ties.  Order by (score descending, key index ascending); equal means exact
  equality, so -0.0 == +0.0.  Output rows are sets (padded with -1).
* Fewer candidates than k.  Keep all of them.
* Proxy.  "Aggregates" is read as the arithmetic mean of the members' real
  (dequantised) q and of their head weights w; the proxy scan covers the
  prefix of the group's last member.  The proxy is stored for the scan in
  bfloat16 (round to nearest even) for bf16 and fp8 inputs and in float32
  for float32 inputs; see ``round_proxy``.
* Causality inside a group.  Refine and Reuse drop candidates beyond the
  member's own position; Reuse does not refill the dropped slots.
"""

import numpy as np

from .formats import f64_to_bf16_bits_rne, bf16_bits_to_f64


# ----------------------------------------------------------------------------
# scoring


def causal_scores(q, k, w, limits):
    """Score rows with a per-row causal limit.

    q : [R, H, d] float64 real query values (R rows), k : [n_k, d] float64,
    w : [R, H] float64, limits : [R] int, row r sees keys 0..limits[r].
    Returns [R, n_k] float64; entries beyond a row's limit are -inf (excluded).
    """
    R = q.shape[0]
    n_k = k.shape[0]
    out = np.full((R, n_k), -np.inf)
    for r in range(R):
        p = int(limits[r])
        if p < 0:
            continue
        x = k[: p + 1] @ q[r].T  # [p+1, H]: q[r,h,:] . k[s,:]
        out[r, : p + 1] = np.maximum(x, 0.0) @ w[r]  # sum_h w[r,h] * relu(x[s,h])
    return out


def dense_scores(q, k, w, q_pos0):
    """I[t, s] for one sequence: query t sees keys s <= pos(t) = q_pos0 + t."""
    n_q = q.shape[0]
    return causal_scores(q, k, w, q_pos0 + np.arange(n_q))


# ----------------------------------------------------------------------------
# selection


def select_topk(values, index, k):
    """The first min(k, n) of ``index`` ordered by (value descending, index ascending)."""
    values = np.asarray(values, dtype=np.float64)
    index = np.asarray(index, dtype=np.int64)
    order = np.lexsort((index, -values))
    return index[order[: min(k, index.size)]]


def _pad(rows, width):
    out = np.full((len(rows), width), -1, dtype=np.int64)
    for i, r in enumerate(rows):
        out[i, : len(r)] = r
    return out


def dense_topk(q, k, w, q_pos0, topk, scores=None):
    """Per-query top-k over the causal prefix, one sequence; [n_q, topk] padded with -1.

    ``scores`` may supply precomputed rows (e.g. a GPU dump, to check a select
    bit-exactly on the same values); masked entries are never selected.
    """
    I = dense_scores(q, k, w, q_pos0) if scores is None else np.asarray(scores, np.float64)
    rows = []
    for t in range(I.shape[0]):
        p = q_pos0 + t
        rows.append(select_topk(I[t, : p + 1], np.arange(p + 1), topk))
    return _pad(rows, topk)


# ----------------------------------------------------------------------------
# group-shared (PIVOT) indexing


def group_bounds(n_q, group):
    """Fixed-size groups of consecutive queries: [(first, last_exclusive), ...]."""
    return [(g0, min(g0 + group, n_q)) for g0 in range(0, n_q, group)]


def proxy_limits(n_q, group, q_pos0):
    """Each group's scan covers the prefix of its last member: pos(t_last)."""
    return np.array([q_pos0 + e - 1 for (_, e) in group_bounds(n_q, group)], dtype=np.int64)


def proxy_means(q, w, group):
    """Proxy query and weights: the mean over the group's members (float64)."""
    gb = group_bounds(q.shape[0], group)
    qbar = np.stack([q[a:b].mean(axis=0) for (a, b) in gb])
    wbar = np.stack([w[a:b].mean(axis=0) for (a, b) in gb])
    return qbar, wbar


def round_proxy(qbar, wbar, q_fmt):
    """The proxy's storage format for the scan (a reading, see module docstring).

    q: float32 for float32 inputs, bfloat16 (nearest, ties to even) otherwise;
    w: float32.  Returns float64 values of the stored proxy.
    """
    if q_fmt == "f32":
        qs = qbar.astype(np.float32).astype(np.float64)
    else:
        qs = bf16_bits_to_f64(f64_to_bf16_bits_rne(qbar))
    return qs, wbar.astype(np.float32).astype(np.float64)


def proxy_scores(qbar, wbar, k, limits):
    """P[g, s] = sum_h wbar[g,h] relu(qbar[g,h,:] . k[s,:]) for s <= limits[g]."""
    return causal_scores(qbar, k, wbar, limits)


def proxy_candidates(P, limits, n_cand):
    """cand[g] = top min(C, limit+1) of the group's prefix by (-P, s); padded with -1."""
    rows = []
    for g in range(P.shape[0]):
        p = int(limits[g])
        rows.append(select_topk(P[g, : p + 1], np.arange(p + 1), n_cand))
    return _pad(rows, n_cand)


def refine_topk(q, k, w, cand, group, q_pos0, topk, scores=None):
    """PIVOT-Refine: each member re-scores its group's candidates with its own
    indexer and keeps its own top min(k, |V_t|), V_t = cand(g) within [0, pos(t)].

    cand : [n_g, C] int, -1 (or any negative) = empty slot.  ``scores`` may
    supply [n_q, C] per-candidate values to select from instead of computing
    them (to check a select on a GPU's own values).
    """
    n_q = q.shape[0]
    rows = []
    for g, (a, b) in enumerate(group_bounds(n_q, group)):
        c = np.asarray(cand[g], dtype=np.int64)
        for t in range(a, b):
            p = q_pos0 + t
            keep = (c >= 0) & (c <= p)
            v = c[keep]
            if scores is None:
                vals = np.maximum(k[v] @ q[t].T, 0.0) @ w[t] if v.size else np.zeros(0)
            else:
                vals = np.asarray(scores[t], np.float64)[keep]
            rows.append(select_topk(vals, v, topk))
    return _pad(rows, topk)


def reuse_topk(proxy_top, group, q_pos0, n_q, topk):
    """PIVOT-Reuse: member t keeps the proxy's top-k entries that are <= pos(t), no refill."""
    rows = []
    for g, (a, b) in enumerate(group_bounds(n_q, group)):
        r = np.asarray(proxy_top[g], dtype=np.int64)
        r = r[r >= 0][:topk]
        for t in range(a, b):
            rows.append(r[r <= q_pos0 + t])
    return _pad(rows, topk)


def grouped_reference(q, k, w, q_pos0, group, n_cand, topk, variant, q_fmt):
    """Whole group-shared pipeline for one sequence, entirely in the oracle.

    variant "refine": proxy -> scan -> top-C candidates -> per-member re-score
    and top-k.  variant "reuse": proxy -> scan -> top-k shared by the group.
    Returns (out [n_q, topk], cand [n_g, C or topk], proxy q, proxy w).
    """
    n_q = q.shape[0]
    qbar, wbar = round_proxy(*proxy_means(q, w, group), q_fmt)
    lim = proxy_limits(n_q, group, q_pos0)
    P = proxy_scores(qbar, wbar, k, lim)
    if variant == "refine":
        cand = proxy_candidates(P, lim, n_cand)
        out = refine_topk(q, k, w, cand, group, q_pos0, topk)
    elif variant == "reuse":
        cand = proxy_candidates(P, lim, topk)
        out = reuse_topk(cand, group, q_pos0, n_q, topk)
    else:
        raise ValueError(variant)
    return out, cand, qbar, wbar


# ----------------------------------------------------------------------------
# block-mean routing (a second candidate generator for Refine)
#
# "AttentionIndex Architecture ...", "Why Positional Blocks Lose Recall" and
# "Worked Example: Blocks Lose, Clusters Win": two-stage selection that routes
# a query to contiguous blocks of keys ranked by a mean-pooled representative
# of each block, keeps the best blocks, and runs the native indexer only on
# the keys of the kept blocks.  Readings (the pages leave them open):
#   * the router of a group is its PIVOT proxy, the block score is the native
#     indexer form applied to the block mean;
#   * a block is routable for a group only when all its keys lie in the
#     prefix of the group's last member; the keys of the trailing partial
#     block are always candidates;
#   * the block mean is stored for the scan like the proxy (``round_proxy``).


def block_means(k, block):
    """kbar[j] = mean of the real keys of block j = [j*block, min((j+1)*block, n_k))."""
    n_k = k.shape[0]
    return np.stack([k[j : min(j + block, n_k)].mean(axis=0) for j in range(0, n_k, block)])


def block_limits(n_q, group, q_pos0, block):
    """Complete blocks in each group's prefix: floor((pos(t_last) + 1) / block)."""
    return (proxy_limits(n_q, group, q_pos0) + 1) // block


def block_route(qbar, wbar, kbar, k_lim, n_k, block, n_sel):
    """Candidates of each group: the keys of its top min(n_sel, n_full) complete
    blocks by (-B, j), B[g, j] = sum_h wbar relu(qbar_h . kbar_j), plus the
    keys of the trailing partial block up to pos(t_last).

    qbar, wbar: stored proxies; kbar: stored block means; k_lim: pos(t_last)
    per group.  Returns (cand [n_g, (n_sel + 1) * block] ascending, -1 padded;
    block scores [n_g, n_b] with -inf for blocks that are not routable; the
    selected blocks [n_g, n_sel], -1 padded).
    """
    n_g, n_b = qbar.shape[0], kbar.shape[0]
    width = (n_sel + 1) * block
    n_full = (np.asarray(k_lim) + 1) // block
    B = np.full((n_g, n_b), -np.inf)
    rows, sel = [], []
    for g in range(n_g):
        f = int(n_full[g])
        if f > 0:
            B[g, :f] = np.maximum(kbar[:f] @ qbar[g].T, 0.0) @ wbar[g]
        top = select_topk(B[g, :f], np.arange(f), n_sel)
        sel.append(top)
        keys = [np.arange(j * block, (j + 1) * block) for j in top]
        keys.append(np.arange(f * block, int(k_lim[g]) + 1))
        rows.append(np.sort(np.concatenate(keys)))
    return _pad(rows, width), B, _pad(sel, n_sel)


def block_reference(q, k, w, q_pos0, group, block, n_sel, topk, q_fmt, k_fmt):
    """Block routing then Refine, entirely in the oracle, for one sequence."""
    n_q = q.shape[0]
    qbar, wbar = round_proxy(*proxy_means(q, w, group), q_fmt)
    kbar, _ = round_proxy(block_means(k, block), np.zeros((1, 1)), k_fmt)
    lim = proxy_limits(n_q, group, q_pos0)
    cand, B, sel = block_route(qbar, wbar, kbar, lim, k.shape[0], block, n_sel)
    return refine_topk(q, k, w, cand, group, q_pos0, topk), cand, B, sel


# ----------------------------------------------------------------------------
# IVF routing with causal index versions (a third candidate generator)
#
# "AttentionIndex Architecture ...", "KEY FINDINGS", "An Inverted File With
# Causal Versions" and "Worked Example: Blocks Lose, Clusters Win": keys are
# grouped by similarity into inverted lists, a query is routed to the lists
# whose representatives score highest and the native indexer re-scores their
# members.  Arriving keys are candidates right away and join existing lists
# batch by batch; now and then a refit reclusters all keys so far, seeded with
# the previous clustering, giving a new version of lists and representatives;
# causality holds per version: a group may use a version only when all of the
# keys behind it precede the group's last member.  Readings (the pages leave them open; no trained encoder here,
# so representatives are plain means):
#   * refits happen every R keys: version u (u = 1, 2, ...) is refit on keys
#     [0, u R) by T Lloyd iterations of k-means with m centroids, starting
#     from version u-1's centroids (version 1: the keys at positions
#     floor(c R / m), c < m); one iteration assigns every key to its nearest
#     stored centroid (squared L2, ties to the lower centroid) and replaces
#     each centroid by the mean of its members (an empty cluster keeps its
#     centroid);
#   * centroids are stored like the proxy (``round_proxy``: bfloat16, float32
#     for float32 keys) and assignment and routing both use the stored values;
#   * between refits, new keys are added to version u's lists (nearest stored
#     centroid, same rule) in batches of b keys counted from u R: a key
#     becomes routable through its list once its batch is complete within the
#     query's prefix; until then it is a candidate outright;
#   * group g (prefix [0, p], p = pos of its last member) uses version
#     u = floor((p + 1) / R); the keys [e, p] with e = u R + b floor((p + 1 - u R) / b)
#     are always candidates (with no version, u = 0, e = 0: the whole prefix);
#   * clusters are ranked by the indexer form of the group proxy against the
#     stored centroid, ties to the lower centroid, and their visible members
#     (keys < e) taken in that order while they fit in the budget C left next
#     to the always-candidates; the first cluster that does not fit ends the walk.


def ivf_store(x, k_fmt):
    """A centroid as stored: float32 for float32 keys, bfloat16 (nearest even) otherwise."""
    return round_proxy(x, np.zeros((1, 1)), k_fmt)[0]


def ivf_assign(keys, cent):
    """Index of the nearest centroid (squared L2) of each key; ties to the lower index."""
    d2 = ((keys[:, None, :] - cent[None, :, :]) ** 2).sum(axis=2)
    return np.argmin(d2, axis=1)


def ivf_update(keys, assign, cent, k_fmt):
    """One k-means update: each centroid becomes the stored mean of its members."""
    new = cent.copy()
    for c in range(cent.shape[0]):
        members = keys[assign == c]
        if members.shape[0] > 0:
            new[c] = ivf_store(members.mean(axis=0), k_fmt)
    return new


def ivf_build(k, m, R, T, k_fmt):
    """Versions u = 1..floor(n_k / R) of the index over one sequence's real keys k.

    Returns a list of (centroids [m, d] as stored, assignment [n_k]) per
    version: the nearest stored centroid of every key of the version's window
    [0, min((u + 1) R, n_k)) - its refit keys and the keys added to its lists
    until the next refit - and -1 beyond the window.
    """
    n_k = k.shape[0]
    assert 1 <= m <= R
    cent = ivf_store(np.stack([k[(c * R) // m] for c in range(m)]), k_fmt)
    versions = []
    for u in range(1, n_k // R + 1):
        keys = k[: u * R]
        for _ in range(T):
            cent = ivf_update(keys, ivf_assign(keys, cent), cent, k_fmt)
        end = min((u + 1) * R, n_k)
        a = np.full(n_k, -1, dtype=np.int64)
        a[:end] = ivf_assign(k[:end], cent)
        versions.append((cent.copy(), a))
    return versions


def ivf_visible_end(last, R, b):
    """Version used by a group whose last member sits at `last`, and the end e of its
    routable keys: u = floor((last + 1) / R), e = u R + b floor((last + 1 - u R) / b)
    (e = 0 without a version: there are no lists to add keys to)."""
    u = (last + 1) // R
    return u, (u * R + b * ((last + 1 - u * R) // b) if u >= 1 else 0)


def ivf_route(qbar, wbar, versions, k_lim, R, b, n_cand, scores=None):
    """Candidates of each group ([n_g, n_cand] ascending, -1 padded), the cluster
    scores [n_g, m] (-inf where the group has no version) and the clusters taken
    ([n_g, m] in walk order, -1 padded).

    qbar, wbar: stored proxies; versions: as ``ivf_build``; k_lim: pos(t_last) per group.
    ``scores`` may supply precomputed cluster score rows (e.g. a GPU dump, to
    check the walk exactly on the same values).
    """
    n_g = qbar.shape[0]
    m = versions[0][0].shape[0] if versions else 1
    S = np.full((n_g, m), -np.inf)
    rows, taken = [], []
    for g in range(n_g):
        last = int(k_lim[g])
        u, e = ivf_visible_end(last, R, b)
        keys = [np.arange(e, last + 1)]
        room = n_cand - keys[0].size
        assert room >= 0, "budget below the always-candidate keys"
        took = []
        if u >= 1:
            cent, a = versions[u - 1]
            if scores is None:
                S[g] = np.maximum(cent @ qbar[g].T, 0.0) @ wbar[g]
            else:
                S[g] = np.asarray(scores[g], dtype=np.float64)
            for c in select_topk(S[g], np.arange(m), m):
                members = np.nonzero(a[:e] == c)[0]
                if members.size > room:
                    break
                keys.append(members)
                took.append(c)
                room -= members.size
        rows.append(np.sort(np.concatenate(keys)))
        taken.append(np.array(took, dtype=np.int64))
    return _pad(rows, n_cand), S, _pad(taken, m)


def ivf_reference(q, k, w, q_pos0, group, m, R, T, b, n_cand, topk, q_fmt, k_fmt):
    """IVF index build, routing and Refine, entirely in the oracle, for one sequence."""
    n_q = q.shape[0]
    qbar, wbar = round_proxy(*proxy_means(q, w, group), q_fmt)
    versions = ivf_build(k, m, R, T, k_fmt)
    lim = proxy_limits(n_q, group, q_pos0)
    cand, S, taken = ivf_route(qbar, wbar, versions, lim, R, b, n_cand)
    return refine_topk(q, k, w, cand, group, q_pos0, topk), cand, S, versions


# ----------------------------------------------------------------------------
# measurement


def recall(approx, exact):
    """recall_t = |approx_t & exact_t| / |exact_t| per query (-1 entries ignored)."""
    out = np.empty(exact.shape[0])
    for t in range(exact.shape[0]):
        e = set(int(x) for x in exact[t] if x >= 0)
        a = set(int(x) for x in approx[t] if x >= 0)
        out[t] = len(a & e) / len(e) if e else 1.0
    return out
