"""The library's stored means, bit for bit: PIVOT proxies and block means.

"PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention",
Abstract (a group is aggregated into one proxy query); "AttentionIndex
Architecture ...", "Why Positional Blocks Lose Recall" (mean-pooled block
representatives).  The library averages in float32 and stores bfloat16, round
to nearest with ties to even (float32 head weights).  When every member is a
dyadic number of limited range and the member count is a power of two, the
float32 sum and the division are exact, so the stored value must be exactly
the oracle's rounding of the exact mean: no tolerance.  A quarter of the
means of four 8-bit significands fall exactly halfway between two bfloat16
values, so the tie rule is exercised on every run.
"""

import numpy as np
import pytest
import torch

import oracle as O

from parity import cuda

pytestmark = pytest.mark.gpu


def dyadic(rng, shape, fmt):
    """Random values exactly representable in `fmt` with exponents in a range
    narrow enough that sums of up to 16 of them are exact in float32 (bf16:
    granularity 2^-13 and magnitude below 2^11 for 16 members)."""
    if fmt == "bf16":
        m = rng.integers(0, 128, size=shape) / 128.0
        e = rng.integers(-6, 7, size=shape)
    else:  # OCP FP8 E4M3 normals below its largest binade
        m = rng.integers(0, 8, size=shape) / 8.0
        e = rng.integers(-6, 8, size=shape)
    s = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    return (s * (1.0 + m) * np.exp2(e)).astype(np.float32)


def make(fmt, n_q, n_k, H, d, seed, dev):
    rng = np.random.default_rng(seed)
    qv = dyadic(rng, (1, n_q, H, d), fmt)
    kv = dyadic(rng, (1, n_k, d), fmt)
    w = (rng.integers(0, 256, size=(1, n_q, H)) / 256.0).astype(np.float32)
    if fmt == "bf16":
        q = torch.from_numpy(qv).to(torch.bfloat16)
        k = torch.from_numpy(kv).to(torch.bfloat16)
        qs = ks = None
        q_real, k_real = qv.astype(np.float64), kv.astype(np.float64)
    else:
        q = torch.from_numpy(qv).to(torch.float8_e4m3fn)
        k = torch.from_numpy(kv).to(torch.float8_e4m3fn)
        # powers of two: the real values code * scale stay exact, and with
        # exponents in [-7, 8] a sum of up to 16 of them needs at most 23 bits
        qs_np = np.exp2(rng.integers(-1, 2, size=(1, n_q))).astype(np.float32)
        ks_np = np.exp2(rng.integers(-1, 2, size=(1, n_k))).astype(np.float32)
        qs, ks = torch.from_numpy(qs_np).to(dev), torch.from_numpy(ks_np).to(dev)
        q_real = qv.astype(np.float64) * qs_np[..., None, None]
        k_real = kv.astype(np.float64) * ks_np[..., None]
    # the conversions above are exact by construction
    assert np.array_equal(q.float().numpy(), qv) and np.array_equal(k.float().numpy(), kv)
    return (q.to(dev), k.to(dev), torch.from_numpy(w).to(dev), qs, ks), q_real, k_real, w.astype(np.float64)


def stored(t):
    """float64 values of a GPU bfloat16 or float32 tensor."""
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [2, 4, 16])
def test_proxy_is_round_to_nearest_even_of_exact_mean(fmt, G):
    import sparse_attention_token_causal_amd as S
    dev = cuda()
    n_q, H, d = 64, 64, 128
    print(f"\n[rounding] proxy {fmt} G={G}", flush=True)
    (q, k, w, qs, ks), q_real, _, w_real = make(fmt, n_q, n_q, H, d, 100 + G, dev)
    _, pq, pw = S.group_proxy_scan(q, k, w, G, 8, q_scale=qs, k_scale=ks, return_proxy=True)
    torch.cuda.synchronize()
    qbar, wbar = O.proxy_means(q_real[0], w_real[0], G)
    want_q, want_w = O.round_proxy(qbar, wbar, fmt)
    got_q, got_w = stored(pq[0]), stored(pw[0])
    ties = (np.abs(qbar - want_q) == 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(want_q), 1e-30))) - 7))
    assert np.array_equal(got_q, want_q), f"{int((got_q != want_q).sum())} stored proxy elements differ"
    assert np.array_equal(got_w, want_w), "stored proxy weights differ"
    print(f"  {qbar.size} means, {int(ties.sum())} exact ties, all stored values equal", flush=True)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_block_means_are_round_to_nearest_even_of_exact_mean(fmt):
    import sparse_attention_token_causal_amd as S
    dev = cuda()
    n_q, H, d, block = 64, 64, 128, 4
    print(f"\n[rounding] block means {fmt}", flush=True)
    (q, k, w, qs, ks), _, k_real, _ = make(fmt, n_q, n_q, H, d, 7, dev)
    _, km = S.block_route(q, k, w, 4, block, 4, q_scale=qs, k_scale=ks, return_means=True)
    torch.cuda.synchronize()
    want, _ = O.round_proxy(O.block_means(k_real[0], block), np.zeros((1, 1)), fmt)
    got = stored(km[0])
    assert np.array_equal(got, want), f"{int((got != want).sum())} stored block-mean elements differ"
