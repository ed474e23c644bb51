"""Host-side checks of the Python binding's caller-supplied tensors (no GPU needed).

The kernels write every element of an output row and carve the workspace by
byte offsets, so a wrong-shaped, wrong-typed, strided or misplaced ``out`` or
``workspace`` must be refused before any pointer reaches the library.
"""

import pytest
import torch

import sparse_attention_token_causal_amd as S
from sparse_attention_token_causal_amd import IndexerError

B, N, H, D, K = 1, 16, 64, 128, 4


def inputs(device="cpu"):
    q = torch.zeros((B, N, H, D), dtype=torch.bfloat16, device=device)
    k = torch.zeros((B, N, D), dtype=torch.bfloat16, device=device)
    w = torch.zeros((B, N, H), dtype=torch.float32, device=device)
    return q, k, w


BAD_OUTS = {
    "shape": lambda: torch.zeros((B, N, K + 1), dtype=torch.int32),
    "rank": lambda: torch.zeros((B * N, K), dtype=torch.int32),
    "dtype": lambda: torch.zeros((B, N, K), dtype=torch.int64),
    "strided": lambda: torch.zeros((B, K, N), dtype=torch.int32).transpose(1, 2),
    "not_a_tensor": lambda: [[0] * K] * N,
}


@pytest.mark.parametrize("bad", sorted(BAD_OUTS))
def test_score_topk_rejects_bad_out(bad):
    q, k, w = inputs()
    with pytest.raises(IndexerError, match="out must be"):
        S.score_topk(q, k, w, K, out=BAD_OUTS[bad]())


@pytest.mark.parametrize("bad", sorted(BAD_OUTS))
def test_refine_topk_rejects_bad_out(bad):
    q, k, w = inputs()
    cand = torch.zeros((B, N // 4, 8), dtype=torch.int32)
    with pytest.raises(IndexerError, match="out must be"):
        S.refine_topk(q, k, w, cand, 4, K, out=BAD_OUTS[bad]())


@pytest.mark.parametrize("bad", sorted(BAD_OUTS))
def test_reuse_topk_rejects_bad_out(bad):
    ptop = torch.zeros((B, N // 4, K), dtype=torch.int32)
    with pytest.raises(IndexerError, match="out must be"):
        S.reuse_topk(ptop, 4, N, N, out=BAD_OUTS[bad]())


BAD_WS = {
    "dtype": lambda: torch.zeros(1 << 12, dtype=torch.float32),
    "rank": lambda: torch.zeros((16, 256), dtype=torch.uint8),
    "strided": lambda: torch.zeros(1 << 13, dtype=torch.uint8)[::2],
}


@pytest.mark.parametrize("bad", sorted(BAD_WS))
@pytest.mark.parametrize("entry", ["score_topk", "group_proxy_scan", "refine_topk", "block_route"])
def test_entry_points_reject_bad_workspace(bad, entry):
    q, k, w = inputs()
    ws = BAD_WS[bad]()
    with pytest.raises(IndexerError, match="workspace must be"):
        if entry == "score_topk":
            S.score_topk(q, k, w, K, workspace=ws)
        elif entry == "group_proxy_scan":
            S.group_proxy_scan(q, k, w, 4, 8, workspace=ws)
        elif entry == "refine_topk":
            S.refine_topk(q, k, w, torch.zeros((B, N // 4, 8), dtype=torch.int32), 4, K, workspace=ws)
        else:
            S.block_route(q, k, w, 4, 4, 2, workspace=ws)


def test_out_and_workspace_must_share_the_inputs_device():
    # "meta" stands in for the GPU here: the check compares devices, not kinds
    q, k, w = inputs("meta")
    with pytest.raises(IndexerError, match="out must be on meta"):
        S.score_topk(q, k, w, K, out=torch.zeros((B, N, K), dtype=torch.int32))
    with pytest.raises(IndexerError, match="workspace must be on meta"):
        S.score_topk(q, k, w, K, workspace=torch.zeros(64, dtype=torch.uint8))


def test_candidates_must_be_contiguous_int32():
    q, k, w = inputs()
    for cand in (torch.zeros((B, N // 4, 8), dtype=torch.int64),
                 torch.zeros((B, 8, N // 4), dtype=torch.int32).transpose(1, 2)):
        with pytest.raises(IndexerError, match="cand must be"):
            S.refine_topk(q, k, w, cand, 4, K)


def test_cpu_inputs_are_refused():
    q, k, w = inputs()
    with pytest.raises(IndexerError, match="on the GPU"):
        S.score_topk(q, k, w, K, out=torch.zeros((B, N, K), dtype=torch.int32))
