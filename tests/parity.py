"""Shared helpers for the GPU-vs-oracle parity tests.

Criteria (written here once, used by every parity test):

* scores: |gpu - oracle| <= ATOL + RTOL * |oracle| per eligible entry, with
  the oracle in float64 on the exact input bytes; excluded entries are -inf
  on both sides;
* select: the GPU's top-k set equals the oracle's select run on the GPU's
  own float32 scores (bit-exact: same values, same tie rule);
* set agreement against the oracle's own top-k, ignoring entries whose
  oracle score lies within the score tolerance of the oracle's k-th score
  (near-ties that float32 and float64 may order differently); required >=
  AGREEMENT.

With head weights of both signs a score can be a small residual of large
terms w_h relu(q_h . k), and any float32 evaluation then errs in proportion
to the terms, not to the result: there the tolerance (and the near-tie band)
gains MAG_RTOL times M = sum_h |w_h| sum_d |q_hd| |k_d|, the float32
accumulation bound of a d <= 128 dot product (d 2^-24 = 2^-17) with a
factor 2 of margin.
"""

import numpy as np
import torch

import oracle as O
from sparse_attention_token_causal_amd import synth

ATOL, RTOL = 1e-3, 2e-3
AGREEMENT = 0.999
MAG_RTOL = 2.0 ** -16


def score_magnitudes(q, k, w):
    """M[t, s] = sum_h |w[t,h]| sum_d |q[t,h,d]| |k[s,d]| (float64)."""
    qa = np.einsum("th,thd->td", np.abs(w), np.abs(q))
    return qa @ np.abs(k).T


def cuda():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def real_inputs(inp):
    """Decode the raw storage the GPU consumed into float64 (oracle side)."""
    qs = None if inp["q_scale"] is None else inp["q_scale"].cpu().numpy()
    ks = None if inp["k_scale"] is None else inp["k_scale"].cpu().numpy()
    q = O.real_values(synth.raw_numpy(inp["q"]), synth.fmt_of(inp["q"]), qs)
    k = O.real_values(synth.raw_numpy(inp["k"]), synth.fmt_of(inp["k"]), ks)
    w = inp["w"].cpu().numpy().astype(np.float64)
    return q, k, w


def real_rows(inp, b, rows):
    """Like real_inputs but only sequence b's listed query rows (for big workloads)."""
    rows = torch.as_tensor(np.asarray(rows), device=inp["q"].device, dtype=torch.long)
    qb = inp["q"][b].index_select(0, rows)
    qs = None if inp["q_scale"] is None else inp["q_scale"][b].index_select(0, rows).cpu().numpy()
    q = O.real_values(synth.raw_numpy(qb), synth.fmt_of(qb), qs)
    w = inp["w"][b].index_select(0, rows).cpu().numpy().astype(np.float64)
    ks = None if inp["k_scale"] is None else inp["k_scale"][b].cpu().numpy()
    k = O.real_values(synth.raw_numpy(inp["k"][b]), synth.fmt_of(inp["k"]), ks)
    return q, k, w


def check_scores(gpu, ref, what="", mag=None):
    """mag: the term magnitudes M of each entry (signed weights), or None."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), m_ref), f"{what}: excluded entries differ"
    e = ~m_ref
    err = np.abs(gpu[e] - ref[e])
    lim = ATOL + RTOL * np.abs(ref[e]) + (0.0 if mag is None else MAG_RTOL * np.asarray(mag, np.float64)[e])
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {e.sum()} scores outside tolerance, "
                           f"worst err/tol {np.max(err / lim):.3g}")
    return float(np.max(err / lim)) if e.any() else 0.0


def ulp_bf16(x):
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 7)


def run_absmax(x, bounds):
    """Per run [a, b) of consecutive rows: the largest magnitude of each element."""
    return np.stack([np.abs(x[a:b]).max(axis=0) for (a, b) in bounds])


def check_stored_mean(gpu, ref, x, bounds, fmt, what):
    """A mean over runs of rows of x, averaged in float32 and stored in `fmt`
    (bf16 or f32), against the float64 mean rounded to that format.

    Bound: one unit of the stored format at the larger of the two values,
    plus the float32 accumulation error of a run of n members, each
    conversion (scale product) and each of the n additions rounding once:
    (n + 2) 2^-24 max|member|.  That second term governs when the members
    cancel and the mean is near zero, where one unit of the stored format is
    tiny."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.array([b - a for (a, b) in bounds], np.float64).reshape((-1,) + (1,) * (ref.ndim - 1))
    acc = (n + 2) * 2.0 ** -24 * run_absmax(np.asarray(x, np.float64), bounds)
    top = np.maximum(np.abs(gpu), np.abs(ref))
    unit = ulp_bf16(top) if fmt == "bf16" else np.exp2(np.floor(np.log2(np.maximum(top, 1e-30))) - 23)
    lim = unit * 1.0001 + acc
    bad = np.abs(gpu - ref) > lim
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the stored-mean bound"


def sets(rows):
    return [frozenset(int(x) for x in np.asarray(r).ravel() if x >= 0) for r in rows]


def assert_same_sets(a, b, what=""):
    sa, sb = sets(a), sets(b)
    bad = [i for i in range(len(sa)) if sa[i] != sb[i]]
    assert not bad, f"{what}: {len(bad)} rows differ, first row {bad[0]}: " \
                    f"only-a {sorted(sa[bad[0]] - sb[bad[0]])[:8]} only-b {sorted(sb[bad[0]] - sa[bad[0]])[:8]}"


def check_rows_valid(idx, limits, topk, expect_counts=None):
    """Distinct, causal, -1 padded at the end, and (optionally) the expected counts."""
    idx = np.asarray(idx)
    for t in range(idx.shape[0]):
        row = idx[t]
        n = int((row >= 0).sum())
        assert (row[:n] >= 0).all() and (row[n:] == -1).all(), f"row {t}: padding not at the end"
        assert len(set(row[:n].tolist())) == n, f"row {t}: duplicate indices"
        assert (row[:n] <= limits[t]).all(), f"row {t}: index beyond the causal limit"
        if expect_counts is not None:
            assert n == expect_counts[t], f"row {t}: {n} entries, expected {expect_counts[t]}"


def band_agreement(gpu_idx, ora_idx, ora_values, keys=None, mag_rows=None):
    """1 - |symmetric difference outside the near-tie band| / (2 * sum k_eff).

    ora_values[t] maps each eligible key of query t to its oracle score (an
    array indexed by key when keys is None, else aligned with keys[t]).
    mag_rows[t]: the largest term magnitude M of row t (signed weights; the
    band widens by twice MAG_RTOL times it), or None.
    """
    num = 0
    den = 0
    for t in range(len(ora_idx)):
        o = [int(x) for x in ora_idx[t] if x >= 0]
        g = [int(x) for x in gpu_idx[t] if x >= 0]
        den += 2 * len(o)
        if not o:
            continue
        if keys is None:
            val = lambda s: ora_values[t][s]
        else:
            lut = dict(zip((int(x) for x in keys[t]), ora_values[t]))
            val = lambda s: lut[s]
        tau = min(val(s) for s in o)
        band = ATOL + RTOL * abs(tau) + (0.0 if mag_rows is None else 2 * MAG_RTOL * float(mag_rows[t]))
        for s in set(o) ^ set(g):
            if abs(val(s) - tau) > band:
                num += 1
    return 1.0 - num / max(den, 1)
