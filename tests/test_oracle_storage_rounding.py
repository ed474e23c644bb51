"""Pins for the oracle's storage rounding of means: the PIVOT proxy query, block
means and IVF centroids.

"PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention",
Abstract: a group of queries is aggregated into one proxy query that does the
shared scan.  "AttentionIndex Architecture ...", "Why Positional Blocks Lose
Recall" and "An Inverted File With Causal Versions": blocks and clusters are
ranked through a mean representative.  The pages do not give a storage format;
the reading is that these means are stored in bfloat16 (round to nearest,
ties to the even significand) for bfloat16 and FP8 inputs and in float32 for
float32 inputs, head weights always in float32, and that the stored values are
what the scan uses.

The expected stored values below are worked out by hand, not computed by the
oracle's own rounding helper.  bfloat16 keeps 8 significant bits, so values in
[1, 2) are spaced 2^-7 and values in [1/2, 1) are spaced 2^-8; float32 keeps
24, spacing 2^-23 in [1, 2).  The means are chosen so that each plausible
mistake gives a different value:

* 1 + 2^-8 lies exactly halfway between 1 (even significand) and 1 + 2^-7
  (odd): ties-to-even gives 1, rounding half up gives 1 + 2^-7;
* 1 + 3 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even):
  ties-to-even gives 1 + 2^-6, truncation gives 1 + 2^-7;
* 3/4 + 3 2^-10 = (192 + 3/4) 2^-8 is not a tie: nearest gives 193 2^-8,
  truncation 192 2^-8;
* (1 + 9/8 + 9/8) / 3 = 13/12 = 138.67 2^-7 (not dyadic): nearest gives
  139 2^-7, truncation 138 2^-7;
* the negatives of the above round symmetrically.

Every member value used is representable in bfloat16 and in OCP FP8 E4M3
(2, 2^-7, 3/2, 3 2^-9, 1, 9/8, or their bfloat16-only variants where noted), so
the same groups are valid bf16 or FP8 inputs.

A mutation test then plants the mistakes (no rounding, truncation, FP8 inputs
left unrounded, ties rounded away from zero) in the oracle's rounding step and
shows that each one fails every one of these pins.
"""

import numpy as np
import pytest

import oracle as O
import oracle.indexer as OI

# (members of one group along the first axis, hand-derived stored bfloat16 mean)
HALF_DOWN = ([2.0, 2.0 ** -7], 1.0)                                    # tie -> even (down)
HALF_UP = ([1.0 + 2.0 ** -7, 1.0 + 2.0 ** -6], 1.0 + 2.0 ** -6)       # tie -> even (up); bf16-only members
ABOVE_HALF = ([1.5, 3 * 2.0 ** -9], 193 * 2.0 ** -8)                   # not a tie: nearest is up
THIRDS = ([1.0, 1.125, 1.125], 139 * 2.0 ** -7)                        # 13/12, not dyadic

# float32 storage (float32 inputs) and float32 head weights
F32_HALF_DOWN = ([2.0, 2.0 ** -23], 1.0)
F32_HALF_UP = ([1.0 + 2.0 ** -23, 1.0 + 2.0 ** -22], 1.0 + 2.0 ** -22)


def _hand_cases(fp8_members_only=False):
    cases = [HALF_DOWN, ABOVE_HALF, THIRDS]
    if not fp8_members_only:
        cases.append(HALF_UP)
    out = []
    for members, stored in cases:
        out.append((members, stored))
        out.append(([-m for m in members], -stored))
    return out


def _assert_bits_equal(got, want, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, what
    bad = got != want
    assert not bad.any(), f"{what}: stored {got[bad][:4]} expected {want[bad][:4]}"


# ----------------------------------------------------------------------------
# the pins (each raises AssertionError when the oracle's rounding is wrong)


def pin_round_proxy_direct():
    """round_proxy on float64 means whose stored values are known by hand."""
    for fmt in ("bf16", "fp8"):
        cases = _hand_cases()
        means = np.array([np.mean(m) for m, _ in cases])
        qs, ws = OI.round_proxy(means.reshape(1, 1, -1), np.array([[1.0 + 2.0 ** -24]]), fmt)
        _assert_bits_equal(qs.ravel(), [s for _, s in cases], f"round_proxy {fmt}")
        # a stored value differs from the unrounded mean in every case
        assert (qs.ravel() != means).all(), f"round_proxy {fmt} left a mean unrounded"
        _assert_bits_equal(ws, [[1.0]], f"round_proxy {fmt} weight (float32 tie)")
    for members, stored in (F32_HALF_DOWN, F32_HALF_UP):
        qs, ws = OI.round_proxy(np.array([[[np.mean(members)]]]), np.array([[np.mean(members)]]), "f32")
        _assert_bits_equal(qs.ravel(), [stored], "round_proxy f32")
        _assert_bits_equal(ws.ravel(), [stored], "round_proxy f32 weight")


def _group_inputs(cases):
    """One group per case, heads = 1, d = 1: q[t, 0, 0] = member value, w = 1.
    Groups have the size of the largest case; shorter cases repeat their
    members so that the mean is unchanged (a multiple of the member list)."""
    G = 6  # common multiple of 2 and 3
    q = []
    for members, _ in cases:
        q += list(members) * (G // len(members))
    q = np.array(q, np.float64).reshape(-1, 1, 1)
    return q, G


def pin_grouped_proxy():
    """The proxy the whole grouped pipeline stores, for bfloat16 and FP8 inputs."""
    for fmt, fp8_only in (("bf16", False), ("fp8", True)):
        cases = _hand_cases(fp8_members_only=fp8_only)
        q, G = _group_inputs(cases)
        n = q.shape[0]
        k = np.ones((n, 1))
        w = np.ones((n, 1))
        _, _, qbar, wbar = O.grouped_reference(q, k, w, 0, G, 4, 2, "refine", fmt)
        _assert_bits_equal(qbar.ravel(), [s for _, s in cases], f"grouped proxy {fmt}")
        _assert_bits_equal(wbar.ravel(), np.ones(len(cases)), f"grouped weights {fmt}")


def pin_block_means():
    """Stored block means, read back through the block scores: one head, the
    proxy is (1, 0) (exact) and w = 1, so score(j) = relu(stored mean_j[0])."""
    for fmt, fp8_only in (("bf16", False), ("fp8", True)):
        cases = [c for c in _hand_cases(fp8_members_only=fp8_only) if c[1] > 0]
        S = 6
        k = []
        for members, _ in cases:
            for m in list(members) * (S // len(members)):
                k.append([m, 0.0])
        k = np.array(k, np.float64)
        n = k.shape[0]
        q = np.tile(np.array([[[1.0, 0.0]]]), (n, 1, 1))
        w = np.ones((n, 1))
        _, _, B, _ = O.block_reference(q, k, w, 0, n, S, len(cases), 4, fmt, fmt)
        _assert_bits_equal(B[0], [s for _, s in cases], f"block means {fmt}")


def pin_ivf_centroids():
    """One cluster refit on one window: its centroid is the stored mean of the window."""
    for fmt, fp8_only in (("bf16", False), ("fp8", True)):
        for members, stored in _hand_cases(fp8_members_only=fp8_only):
            k = np.array([[m, 0.0] for m in members], np.float64)
            versions = O.ivf_build(k, 1, k.shape[0], 1, fmt)
            _assert_bits_equal(versions[0][0][0], [stored, 0.0], f"IVF centroid {fmt} {members}")
            _assert_bits_equal(O.ivf_store(np.array([np.mean(members)]), fmt), [stored], f"ivf_store {fmt}")
    for members, stored in (F32_HALF_DOWN, F32_HALF_UP):
        k = np.array([[m] for m in members], np.float64)
        _assert_bits_equal(O.ivf_build(k, 1, 2, 1, "f32")[0][0], [[stored]], "IVF centroid f32")


PINS = [pin_round_proxy_direct, pin_grouped_proxy, pin_block_means, pin_ivf_centroids]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_storage_rounding_pins(pin):
    pin()


def test_torch_agrees_where_float32_is_exact():
    """Independent check of the hand values: every mean above except 13/12 is
    exact in float32, where torch's float32 -> bfloat16 conversion (round to
    nearest even) applies."""
    import torch
    for members, stored in _hand_cases():
        if len(members) == 3:
            continue
        mean = np.float32(np.mean(members))
        assert float(mean) == np.mean(members)
        assert float(torch.tensor(mean).to(torch.bfloat16).float()) == stored


# ----------------------------------------------------------------------------
# planted mistakes in the rounding step


def _bits_to_f64(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _mut_no_rounding(qbar, wbar, q_fmt):
    qs = qbar.astype(np.float32).astype(np.float64) if q_fmt == "f32" else np.asarray(qbar, np.float64)
    return qs, wbar.astype(np.float32).astype(np.float64)


def _mut_truncate(qbar, wbar, q_fmt):
    if q_fmt == "f32":
        return _mut_no_rounding(qbar, wbar, q_fmt)
    bits = np.asarray(qbar, np.float32).view(np.uint32) >> np.uint32(16)
    return _bits_to_f64(bits), wbar.astype(np.float32).astype(np.float64)


def _mut_fp8_unrounded(qbar, wbar, q_fmt):
    if q_fmt == "fp8":
        return np.asarray(qbar, np.float64), wbar.astype(np.float32).astype(np.float64)
    return ORIGINAL(qbar, wbar, q_fmt)


def _mut_ties_away(qbar, wbar, q_fmt):
    if q_fmt == "f32":
        return ORIGINAL(qbar, wbar, q_fmt)
    x = np.asarray(qbar, np.float64)
    _, e = np.frexp(x)
    quantum = np.exp2(e.astype(np.float64) - 8.0)
    r = np.sign(x) * np.floor(np.abs(x) / quantum + 0.5) * quantum
    return r, wbar.astype(np.float32).astype(np.float64)


ORIGINAL = OI.round_proxy
MUTANTS = {"no_rounding": _mut_no_rounding, "truncation": _mut_truncate, "fp8_unrounded": _mut_fp8_unrounded,
           "ties_away_from_zero": _mut_ties_away}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_rounding_mistakes(name, monkeypatch):
    monkeypatch.setattr(OI, "round_proxy", MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
    # each path that stores a mean catches it on its own
    assert set(failed) == {p.__name__ for p in PINS}, (name, failed)
