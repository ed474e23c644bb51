"""The entry point that allocates nothing, idx_score_topk_static, against
idx_score_topk with a caller workspace, through the C ABI.

Calls in a row on one GPU, each a different problem sharing the library's
fixed scratch array (which keeps the previous call's contents): the decode
step of 8 sequences x 2 multi-token-prediction queries over 131072 FP8 keys
(split-key scan), then a smaller one (2 sequences over 20000 keys), then a
short 64-head prefill (the filtering dense scan, whose overflow counters are
cleared inside the same scratch) and one whose candidate lists overflow
(the rescan).  Index work is exact: every row must hold the same set.
"""

import ctypes

import pytest
import torch

import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd.synth import WORKLOADS, Workload, make_inputs

from parity import cuda

pytestmark = pytest.mark.gpu

DECODE = WORKLOADS["decode_fp8k_B8_mtp2_n131072_H64_d128_k2048"]
CASES = [
    DECODE,
    DECODE.scaled(name="decode_fp8k_B2_mtp2_n20000", batch=2, n_k=20000, seed=5),
    Workload("prefill_bf16_L2048_H64_k64", 1, 2048, 2048, 64, 128, "bf16", "bf16", "ar1", "heavy", rho=0.98,
             topk=64, seed=6),
    Workload("prefill_overflow_ramp_L3000_H64_k50", 1, 3000, 3000, 64, 128, "bf16", "bf16", "normal8", "ramp",
             topk=50, seed=7),
]


def both_entry_points(wl, inp):
    lib = S.load_library()
    p = S.make_problem(inp["q"], inp["k"], inp["w"], inp["q_scale"], inp["k_scale"], wl.q_pos0)
    dev = inp["q"].device
    out_static = torch.full((wl.batch, wl.n_q, wl.topk), -7, dtype=torch.int32, device=dev)
    out_ws = torch.full_like(out_static, -7)
    n = lib.idx_workspace_bytes(ctypes.byref(p), S.IDX_OP_SCORE_TOPK, 0, 0, wl.topk)
    assert 0 < n <= 64 << 20, n
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = lib.idx_score_topk_static(ctypes.byref(p), wl.topk, ctypes.c_void_p(out_static.data_ptr()), None, st)
    assert rc == 0, lib.idx_status_string(rc)
    rc = lib.idx_score_topk(ctypes.byref(p), wl.topk, ctypes.c_void_p(out_ws.data_ptr()), None,
                            ctypes.c_void_p(ws.data_ptr()), n, st)
    assert rc == 0, lib.idx_status_string(rc)
    torch.cuda.synchronize()
    return out_static, out_ws


def test_static_scratch_matches_workspace_entry_point():
    dev = cuda()
    for wl in CASES:
        print(f"\n[no-alloc] {wl.name}", flush=True)
        inp = make_inputs(wl, dev)
        a, b = both_entry_points(wl, inp)
        # rows are sets (the split-key path gathers its lists in parallel)
        assert torch.equal(torch.sort(a, dim=-1)[0], torch.sort(b, dim=-1)[0]), wl.name
        assert (a != -7).all(), "every output slot is written"


def test_static_scratch_binding_allocates_nothing_given_out():
    dev = cuda()
    wl = CASES[1]
    inp = make_inputs(wl, dev)
    out = torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.int32, device=dev)
    args = dict(q_scale=inp["q_scale"], k_scale=inp["k_scale"], q_pos0=wl.q_pos0)
    S.score_topk_static(inp["q"], inp["k"], inp["w"], wl.topk, out=out, **args)
    ref = S.score_topk(inp["q"], inp["k"], inp["w"], wl.topk, **args)
    torch.cuda.synchronize()
    assert torch.equal(torch.sort(out, dim=-1)[0], torch.sort(ref, dim=-1)[0])
