"""GPU vs oracle parity on seeded random shapes.

The fixed cases in test_gpu_parity.py pick shapes by hand; these draw them
from a seeded generator over everything the library accepts: batch 1-2,
prefill or decode positions (at most four queries at the end of up to 6000
keys, the split-key path), 16/32/64 heads, d = 64/128, every storage
combination, smooth, heavy-tailed or small-integer (tie-heavy) values,
k from 1 to 400, and for the grouped path group sizes 1-64 and candidate
budgets below and above k.  Each case runs the same checks as the fixed
ones.
"""

import numpy as np
import pytest

from sparse_attention_token_causal_amd.synth import Workload

import test_gpu_parity as P

pytestmark = pytest.mark.gpu

COMBOS = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")]


def _draw(rng, i, prefix, grouped):
    qf, kf = COMBOS[int(rng.integers(len(COMBOS)))]
    H = int(rng.choice([16, 32, 64]))
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    if rng.random() < 0.35:  # decode positions
        n_q = int(rng.integers(1, 5))
        n_k = int(rng.integers(n_q, 6001))
    else:
        n_q = int(rng.integers(1, 701))
        n_k = n_q if rng.random() < 0.7 else int(rng.integers(n_q, 1501))
    kd = str(rng.choice(["normal8", "heavy", "int"]))
    qd = "int" if kd == "int" else str(rng.choice(["normal8", "ar1"]))
    wd = "int" if kd == "int" else str(rng.choice(["uniform", "uniform", "signed"]))
    topk = int(rng.integers(1, 401))
    kw = dict(rho=0.98 if qd == "ar1" else 0.0, topk=topk, seed=7000 + i, w_dist=wd)
    if grouped:
        kw["group"] = int(rng.integers(1, 65))
        kw["n_cand"] = int(rng.integers(max(1, topk // 2), 3 * topk + 2))
    name = (f"{prefix}{i}_B{B}_q{n_q}_k{n_k}_H{H}_d{d}_{qf}{kf}_{qd}-{kd}_k{topk}"
            + (f"_G{kw['group']}_C{kw['n_cand']}" if grouped else ""))
    return Workload(name, B, n_q, n_k, H, d, qf, kf, qd, kd, **kw)


def _shapes(seed, n, prefix, grouped):
    rng = np.random.default_rng(seed)
    return [_draw(rng, i, prefix, grouped) for i in range(n)]


DENSE_RND = _shapes(20261203, 24, "rd", False)
GROUPED_RND = _shapes(20261204, 12, "rg", True)


@pytest.mark.parametrize("wl", DENSE_RND, ids=[w.name for w in DENSE_RND])
def test_dense_random_shape(wl):
    P.test_dense_parity(wl)


@pytest.mark.parametrize("wl", GROUPED_RND, ids=[w.name for w in GROUPED_RND])
def test_grouped_random_shape(wl):
    P.test_grouped_parity(wl)
