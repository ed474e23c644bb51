"""Seeded synthetic indexer inputs, shaped like the pages' workloads.

This module holds no part of the indexer's arithmetic: it draws random
numbers, shapes them and stores them (float32, bfloat16 or OCP FP8 E4M3 with
a per-token float32 scale).  Both the HIP library's tests and the CPU oracle
consume the exact bytes it returns.

Structure mimicked (PIVOT, Abstract: nearby queries select highly overlapping
top-k tokens and scores are long-tailed along the key axis):

* queries: either i.i.d. N(0,1)/8, or an AR(1) process along the token axis,
  q_t = rho * q_{t-1} + eps_t with eps ~ N(0,1) i.i.d. per (head, dim) and
  q_0 drawn from the stationary N(0, 1/(1-rho^2));
* keys: either i.i.d. N(0,1)/8, or N(0,1) with floor(n_k/100) randomly
  chosen rows scaled by 4 (heavy-tailed keys), or similarity groups
  scattered over positions ("clustered": `clusters` centers ~ N(0,1), each
  key = its group's center + spread * N(0,1), groups drawn uniformly per
  position; with seed_stride > 0 the key at position c * seed_stride belongs
  to group c, for c < clusters);
* head weights: U(0,1).

Two further structures exist only to exercise the select's tie handling:
small-integer queries, keys and weights ("int": values in {-2..2}, weights
in {0, 1, 2}), where many scores are exactly equal, and identical keys
("const": every key row is the same N(0,1) vector), where every score of a
query ties.  A third exists to defeat a running top-k threshold: "ramp"
keys k_s = (s + 1) / n_k * |v| for one N(0,1) vector v, so that every
query's scores grow with the key position (up to storage rounding) and
nearly every key beats the best ones seen before it.

Draw order per call: query noise, keys, heavy-row choice, weights, all from
one torch generator seeded with ``seed`` on the target device.
"""

from dataclasses import dataclass, replace
import math

import torch

FP8_MAX = 448.0  # largest finite OCP E4M3 magnitude


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q: int
    n_k: int
    heads: int
    dim: int
    q_fmt: str          # "f32" | "bf16" | "fp8"
    k_fmt: str
    q_dist: str         # "normal8" | "ar1" | "int"
    k_dist: str         # "normal8" | "heavy" | "int" | "const" | "ramp" | "spikes" | "clustered"
    rho: float = 0.0
    topk: int = 2048
    group: int = 0      # 0: dense only
    n_cand: int = 0
    seed: int = 0
    w_dist: str = "uniform"  # "uniform" | "int" | "signed" (U(-1, 1): scores can be negative)
    clusters: int = 0        # "clustered" keys: number of groups
    spread: float = 0.1      # "clustered" keys: within-group noise
    seed_stride: int = 0     # "clustered" keys: position c * seed_stride holds group c

    @property
    def q_pos0(self):
        return self.n_k - self.n_q

    def scaled(self, **kw):
        return replace(self, **kw)


# The five workloads the indexer is specified on.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("prefill_f32_L1024_H16_d64_k128", 1, 1024, 1024, 16, 64, "f32", "f32",
                 "normal8", "normal8", topk=128),
        Workload("prefill_bf16_L32768_H64_d128_k2048", 1, 32768, 32768, 64, 128, "bf16", "bf16",
                 "ar1", "heavy", rho=0.98, topk=2048),
        Workload("decode_fp8k_B8_mtp2_n131072_H64_d128_k2048", 8, 2, 131072, 64, 128, "bf16", "fp8",
                 "ar1", "heavy", rho=0.98, topk=2048, group=2, n_cand=8192),
        Workload("grouped_refine_bf16_L131072_G64_C8192_k2048", 1, 131072, 131072, 64, 128, "bf16",
                 "bf16", "ar1", "heavy", rho=0.98, topk=2048, group=64, n_cand=8192),
        Workload("grouped_fp8_L262144_G128_C8192_k2048", 1, 262144, 262144, 64, 128, "fp8", "fp8",
                 "ar1", "heavy", rho=0.99, topk=2048, group=128, n_cand=8192),
    ]
}


def _ar1(eps, rho):
    """AR(1) along dim 1 of eps [B, T, ...] by a log-depth doubling scan."""
    x = eps.clone()
    x[:, 0] *= 1.0 / math.sqrt(1.0 - rho * rho)
    off, a = 1, rho
    T = x.shape[1]
    while off < T:
        x[:, off:] += a * x[:, :-off]
        off *= 2
        a = a * a
    return x


def _store(x, fmt, payload_dims):
    """float32 values -> (raw storage tensor, per-token scale or None)."""
    if fmt == "f32":
        return x.contiguous(), None
    if fmt == "bf16":
        return x.to(torch.bfloat16).contiguous(), None
    if fmt == "fp8":
        amax = x.abs().amax(dim=payload_dims)
        scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
        shp = scale.shape + (1,) * len(payload_dims)
        codes = (x / scale.reshape(shp)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
        return codes.contiguous(), scale.contiguous()
    raise ValueError(fmt)


def make_inputs(wl: Workload, device="cpu"):
    """Returns dict(q, q_scale, k, k_scale, w) of raw storage tensors on ``device``.

    q [B, n_q, H, d], k [B, n_k, d], w [B, n_q, H] float32, scales [B, tokens]
    float32 for fp8 storage (else None).
    """
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed)
    B, nq, nk, H, d = wl.batch, wl.n_q, wl.n_k, wl.heads, wl.dim
    eps = torch.randn((B, nq, H, d), generator=g, device=device, dtype=torch.float32)
    if wl.q_dist == "normal8":
        q = eps / 8.0
    elif wl.q_dist == "ar1":
        q = _ar1(eps, wl.rho)
    elif wl.q_dist == "int":
        q = torch.clamp(torch.round(eps * 1.5), -2, 2)
    else:
        raise ValueError(wl.q_dist)
    del eps
    k = torch.randn((B, nk, d), generator=g, device=device, dtype=torch.float32)
    if wl.k_dist == "normal8":
        k = k / 8.0
    elif wl.k_dist == "int":
        k = torch.clamp(torch.round(k * 1.5), -2, 2)
    elif wl.k_dist == "const":
        k = k[:, :1].expand(B, nk, d).clone()
    elif wl.k_dist == "ramp":
        ramp = torch.arange(1, nk + 1, device=device, dtype=torch.float32).reshape(1, nk, 1) / nk
        k = ramp * k[:, :1].abs()
    elif wl.k_dist == "spikes":
        # every 16th key 2^20 times larger (exact in every storage format)
        k = k / 8.0
        k[:, ::16] *= float(2 ** 20)
    elif wl.k_dist == "heavy":
        n_heavy = nk // 100
        for b in range(B):
            rows = torch.randperm(nk, generator=g, device=device)[:n_heavy]
            k[b, rows] *= 4.0
    elif wl.k_dist == "clustered":
        C = wl.clusters
        centers = torch.randn((B, C, d), generator=g, device=device, dtype=torch.float32)
        owner = torch.randint(0, C, (B, nk), generator=g, device=device)
        if wl.seed_stride > 0:
            pos = torch.arange(C, device=device) * wl.seed_stride
            keep = pos < nk
            owner[:, pos[keep]] = torch.arange(C, device=device)[keep]
        k = torch.gather(centers, 1, owner[..., None].expand(B, nk, d)) + wl.spread * k
    else:
        raise ValueError(wl.k_dist)
    w = torch.rand((B, nq, H), generator=g, device=device, dtype=torch.float32)
    if wl.w_dist == "int":
        w = torch.floor(w * 3.0)
    elif wl.w_dist == "signed":
        w = 2.0 * w - 1.0
    qs, q_scale = _store(q, wl.q_fmt, (2, 3))
    del q
    ks, k_scale = _store(k, wl.k_fmt, (2,))
    return dict(q=qs, q_scale=q_scale, k=ks, k_scale=k_scale, w=w.contiguous())


def raw_numpy(t):
    """Raw storage as NumPy: float32 stays float32, bf16 -> uint16 bits, fp8 -> uint8 bits."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def fmt_of(t):
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}[t.dtype]
