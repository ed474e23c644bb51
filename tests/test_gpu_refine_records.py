"""PIVOT-Refine's one-pass select against its general path (GPU).

With a workspace the Refine scan leaves, per query, an exact record of the
boundary bin of its candidate scores, and the select then writes the bins
above it and ranks only that bin; asked for the candidate scores, the same
scan writes no records and the select runs its general path.  Both select
the exact top-k of the same float32 scores (ties to the lower key index), so
the two index sets must agree on every row: tie-heavy rows, rows whose keys
all rise with position, rows with fewer eligible candidates than k (also
rows of 8192 slots that are mostly empty), and rows longer than one
register tile of the select.

Source: "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse
Attention", Abstract (each query keeps the top-k of its re-scored
candidates).
"""

import pytest
import torch

import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.synth import Workload, make_inputs

from parity import assert_same_sets, cuda

CASES = [
    Workload("rec_fp8_L600_G32_C300_k100", 1, 600, 600, 64, 128, "fp8", "fp8", "ar1", "heavy", rho=0.99,
             topk=100, group=32, n_cand=300, seed=41),
    Workload("rec_bf16_B2_L700_G64_C512_k128", 2, 700, 700, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
             topk=128, group=64, n_cand=512, seed=42),
    # many exactly equal scores: boundary bins beyond the rankable size
    Workload("rec_int_L500_G16_C256_k40", 1, 500, 500, 64, 128, "bf16", "bf16", "int", "int", topk=40,
             group=16, n_cand=256, seed=43, w_dist="int"),
    # scores that rise with the key position
    Workload("rec_ramp_fp8_L800_G32_C400_k64", 1, 800, 800, 64, 128, "fp8", "fp8", "ar1", "ramp", rho=0.99,
             topk=64, group=32, n_cand=400, seed=44),
    # candidate rows longer than 8192 columns
    Workload("rec_bf16_L64_n12000_G64_C10000_k300", 1, 64, 12000, 64, 128, "bf16", "bf16", "ar1", "heavy",
             rho=0.98, topk=300, group=64, n_cand=10000, seed=45),
    # the longest candidate rows one workgroup holds (16384 columns): the
    # records' histograms are 16-bit counters
    Workload("rec_bf16_L64_n20000_G64_C16384_k700", 1, 64, 20000, 64, 128, "bf16", "bf16", "ar1", "heavy",
             rho=0.98, topk=700, group=64, n_cand=16384, seed=46),
    Workload("rec_fp8_L32_n18000_G32_C16384_k2048", 1, 32, 18000, 64, 128, "fp8", "fp8", "ar1", "heavy",
             rho=0.99, topk=2048, group=32, n_cand=16384, seed=47),
    # a budget beyond every prefix: rows of 8192 candidate slots, mostly
    # empty, and in the groups with fewer than k keys no record, so the
    # one-pass kernel's general path streams them with a sampled bin range
    # (most waves' samples hold no eligible key)
    Workload("rec_sparse_bf16_L2500_G64_C8192_k2048", 1, 2500, 2500, 64, 128, "bf16", "bf16", "ar1", "heavy",
             rho=0.98, topk=2048, group=64, n_cand=8192, seed=48),
]


@pytest.mark.gpu
@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_refine_records_match_general_path(wl):
    dev = cuda()
    inp = make_inputs(wl, dev)
    a = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"])
    cand = S.group_proxy_scan(inp["q"], inp["k"], inp["w"], wl.group, wl.n_cand, **a)
    one_pass = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, wl.group, wl.topk, **a)
    general, _ = S.refine_topk(inp["q"], inp["k"], inp["w"], cand, wl.group, wl.topk, return_scores=True, **a)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        assert_same_sets(one_pass[b].cpu().numpy(), general[b].cpu().numpy(), f"{wl.name} sequence {b}")
