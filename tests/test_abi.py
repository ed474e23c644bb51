"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before touching the device."""

import ctypes
import os
import re

import pytest

import sparse_attention_token_causal_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int32_t|size_t|const char\*)\s+(idx_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return S.load_library()


def test_header_declares_the_four_entry_points():
    fns = declared_functions()
    for f in ("idx_score_topk", "idx_group_proxy_scan", "idx_refine_topk", "idx_reuse_topk",
              "idx_block_route", "idx_ivf_build", "idx_ivf_route", "idx_workspace_bytes", "idx_status_string",
              "idx_version"):
        assert f in fns


def test_library_exports_every_declared_symbol(lib):
    for f in declared_functions():
        assert hasattr(lib, f), f


def test_status_strings(lib):
    assert lib.idx_status_string(0) == b"ok"
    assert b"workspace" in lib.idx_status_string(-3)
    assert lib.idx_version() >= 100


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def problem(**kw):
    d = dict(batch=1, n_q=64, n_k=64, q_pos0=0, heads=64, dim=128, q_dtype=1, k_dtype=1,
             q=FAKE, q_scale=None, k=FAKE, k_scale=None, w=FAKE)
    d.update(kw)
    return S._Problem(d["batch"], d["n_q"], d["n_k"], d["q_pos0"], d["heads"], d["dim"],
                      d["q_dtype"], d["k_dtype"], d["q"], d["q_scale"], d["k"], d["k_scale"], d["w"])


def score(lib, p, topk=8, out=FAKE, ws=None, ws_bytes=0):
    return lib.idx_score_topk(ctypes.byref(p), topk, out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("bad", [
    dict(batch=0), dict(n_q=0), dict(n_k=0), dict(heads=0), dict(dim=0),
    dict(q_pos0=-1), dict(n_q=65), dict(q_pos0=1), dict(q=None), dict(k=None), dict(w=None),
    dict(q_dtype=7), dict(q_dtype=2),                   # fp8 q without its scale
    dict(k_scale=FAKE),                                 # a scale for bf16 keys
])
def test_invalid_problem(lib, bad):
    assert score(lib, problem(**bad)) == -1


@pytest.mark.parametrize("bad", [dict(heads=8), dict(heads=128), dict(dim=96), dict(dim=256),
                                 dict(q_dtype=0, k_dtype=1), dict(q_dtype=2, k_dtype=1, q_scale=FAKE)])
def test_unsupported_combination(lib, bad):
    assert score(lib, problem(**bad)) == -2


def test_invalid_call_arguments(lib):
    p = problem()
    assert score(lib, p, topk=0) == -1
    assert score(lib, p, out=None) == -1
    assert lib.idx_group_proxy_scan(ctypes.byref(p), 0, 8, FAKE, None, None, None, None, 0, None) == -1
    assert lib.idx_group_proxy_scan(ctypes.byref(p), 4, 0, FAKE, None, None, None, None, 0, None) == -1
    assert lib.idx_refine_topk(ctypes.byref(p), 4, None, 8, 8, FAKE, None, None, 0, None) == -1
    assert lib.idx_refine_topk(ctypes.byref(p), 4, FAKE, 8, 0, FAKE, None, None, 0, None) == -1
    assert lib.idx_reuse_topk(ctypes.byref(p), 0, FAKE, 8, FAKE, None) == -1
    assert lib.idx_reuse_topk(ctypes.byref(p), 4, None, 8, FAKE, None) == -1
    assert lib.idx_reuse_topk(ctypes.byref(problem(n_q=65)), 4, FAKE, 8, FAKE, None) == -1
    # block routing: group, block, blocks kept, output, row width
    assert lib.idx_block_route(ctypes.byref(p), 0, 8, 2, FAKE, None, None, None, None, None, 0, None) == -1
    assert lib.idx_block_route(ctypes.byref(p), 4, 0, 2, FAKE, None, None, None, None, None, 0, None) == -1
    assert lib.idx_block_route(ctypes.byref(p), 4, 8, 0, FAKE, None, None, None, None, None, 0, None) == -1
    assert lib.idx_block_route(ctypes.byref(p), 4, 8, 2, None, None, None, None, None, None, 0, None) == -1
    assert lib.idx_block_route(ctypes.byref(p), 4, 1 << 20, 1 << 12, FAKE, None, None, None, None, None, 0,
                               None) == -1
    assert lib.idx_block_route(ctypes.byref(problem(q=None)), 4, 8, 2, FAKE, None, None, None, None, None, 0,
                               None) == -1


def ivf_build_call(lib, p, m=64, R=256, T=2, outs=(FAKE, FAKE, FAKE, FAKE), ws=FAKE, ws_bytes=1 << 40):
    return lib.idx_ivf_build(ctypes.byref(p), m, R, T, *outs, None, ws, ws_bytes, None)


def ivf_route_call(lib, p, G=4, m=64, R=256, b=128, C=512, index=(FAKE, FAKE, FAKE, FAKE), out=FAKE, ws=FAKE,
                   ws_bytes=1 << 40):
    return lib.idx_ivf_route(ctypes.byref(p), G, m, R, b, C, *index, out, None, None, None, ws, ws_bytes, None)


def test_ivf_invalid_arguments(lib):
    p = problem(n_q=512, n_k=512)
    # build: clusters in [1, 1024], refit >= clusters and a multiple of 128, iterations in [0, 64]
    for m, R, T in ((0, 256, 1), (1025, 2048, 1), (300, 256, 1), (64, 200, 1), (64, 256, -1), (64, 256, 65)):
        assert ivf_build_call(lib, p, m, R, T) == -1, (m, R, T)
    for i in range(4):
        outs = [FAKE] * 4
        outs[i] = None
        assert ivf_build_call(lib, p, outs=tuple(outs)) == -1
    assert ivf_build_call(lib, problem(n_q=512, n_k=512, k=None)) == -1
    assert ivf_build_call(lib, problem(n_q=512, n_k=512, dim=96)) == -2
    # the build reads only the keys: q and w may be absent
    assert ivf_build_call(lib, problem(n_q=512, n_k=512, q=None, w=None), ws=None, ws_bytes=0) == -3
    # route: group, batch a multiple of 128 within refit, budget >= refit, index present, output
    assert ivf_route_call(lib, p, G=0) == -1
    for b in (0, 64, 200, 384):
        assert ivf_route_call(lib, p, b=b) == -1, b
    assert ivf_route_call(lib, p, C=255) == -1
    assert ivf_route_call(lib, p, out=None) == -1
    for i in range(4):
        index = [FAKE] * 4
        index[i] = None
        assert ivf_route_call(lib, p, index=tuple(index)) == -1
    # no version inside the keys (n_k < refit): the index is not needed
    short = problem(n_q=100, n_k=100)
    assert ivf_route_call(lib, short, index=(None,) * 4, ws=None, ws_bytes=0) == -3
    assert ivf_build_call(lib, short, ws=None, ws_bytes=0) == 0  # nothing to build, nothing enqueued
    # ... and its outputs are empty, so they may be null (as empty tensors' pointers are)
    assert ivf_build_call(lib, short, outs=(None,) * 4, ws=None, ws_bytes=0) == 0


def test_ivf_workspace_sizes(lib):
    p = problem(n_q=1000, n_k=1000)
    nb = lib.idx_workspace_bytes(ctypes.byref(p), 5, 0, 64, 0)
    nt = -(-1000 // 128)
    # initial centroids (bf16), rank, assignment, tile counts, prefix counts, offsets, members
    assert nb >= 64 * 128 * 2 + 2 * 1000 * 4 + nt * 64 * 4 + (nt + 1) * 64 * 4 + 65 * 4 + 1000 * 4
    assert lib.idx_workspace_bytes(ctypes.byref(p), 5, 0, 0, 0) == 0
    assert lib.idx_workspace_bytes(ctypes.byref(p), 5, 0, 1025, 0) == 0
    nr = lib.idx_workspace_bytes(ctypes.byref(p), 6, 10, 64, 0)
    assert nr >= 100 * 64 * 128 * 2 + 100 * 64 * 4 + 100 * 64 * 4
    assert ivf_build_call(lib, p, m=64, R=256, ws_bytes=nb - 1) == -3
    assert ivf_route_call(lib, p, G=10, m=64, R=256, ws_bytes=nr - 1) == -3


def test_workspace_checks(lib):
    p = problem()
    need = lib.idx_workspace_bytes(ctypes.byref(p), 0, 0, 0, 8)
    assert need > 0
    assert score(lib, p, ws=None, ws_bytes=0) == -3
    assert score(lib, p, ws=FAKE, ws_bytes=need - 1) == -3
    need_g = lib.idx_workspace_bytes(ctypes.byref(p), 1, 4, 16, 0)
    assert lib.idx_group_proxy_scan(ctypes.byref(p), 4, 16, FAKE, None, None, None, FAKE,
                                    need_g - 1, None) == -3
    need_r = lib.idx_workspace_bytes(ctypes.byref(p), 2, 4, 16, 8)
    assert lib.idx_refine_topk(ctypes.byref(p), 4, FAKE, 16, 8, FAKE, None, FAKE, need_r - 1, None) == -3
    assert lib.idx_workspace_bytes(ctypes.byref(p), 3, 4, 16, 8) == 0
    need_b = lib.idx_workspace_bytes(ctypes.byref(p), 4, 4, 8, 2)
    assert need_b > 0
    assert lib.idx_block_route(ctypes.byref(p), 4, 8, 2, FAKE, None, None, None, None, FAKE, need_b - 1,
                               None) == -3


def test_workspace_sizes_follow_the_layout(lib):
    # dense: the score buffer holds whole rows of n_k float32, in whole row blocks
    p = problem(n_q=1000, n_k=1000)
    need = lib.idx_workspace_bytes(ctypes.byref(p), 0, 0, 0, 8)
    assert need >= 1000 * 1000 * 4 and need % 256 == 0
    # large, 64 heads: candidate lists of cap = 1.25 k (1 + ln(n / k)) + 1024 entries
    # (rounded up to 256) of a score and a key each, plus a 32-byte record, for
    # whole 8-row blocks within a 4 GiB budget, after two int slots per row block
    import math
    big = problem(n_q=131072, n_k=131072)
    nb = lib.idx_workspace_bytes(ctypes.byref(big), 0, 0, 0, 2048)
    cap = -(-math.ceil(1.25 * 2048 * (1 + math.log(131072 / 2048)) + 1024) // 256) * 256
    row = cap * 8 + 32
    rows = (4 << 30) // row // 8 * 8
    fixed = 2 * (-(-(131072 // 8) * 4 // 256) * 256)
    assert fixed + rows * row <= nb <= fixed + rows * row + 256
    big32 = problem(n_q=131072, n_k=131072, heads=32)
    nb32 = lib.idx_workspace_bytes(ctypes.byref(big32), 0, 0, 0, 2048)
    assert (2 << 30) <= nb32 <= (2 << 30) + 16 * 131072 * 4 + 256
    # proxy scan: proxy q (bf16) + proxy w + score rows
    g = lib.idx_workspace_bytes(ctypes.byref(p), 1, 10, 64, 0)
    assert g >= 100 * 64 * 128 * 2 + 100 * 64 * 4 + 100 * 1000 * 4
    # block routing: proxy q + w, block means (bf16), kept blocks, block-score rows
    br = lib.idx_workspace_bytes(ctypes.byref(p), 4, 10, 16, 3)
    n_b = -(-1000 // 16)
    assert br >= 100 * 64 * 128 * 2 + 100 * 64 * 4 + n_b * 128 * 2 + 100 * 3 * 4 + 100 * n_b * 4


def test_calibration_recall_matches_the_oracle_definition():
    """The sweep's recall (torch, batched search) equals the oracle's set definition."""
    import numpy as np
    import torch
    import oracle as O
    from sparse_attention_token_causal_amd.calibrate import choose, recall
    rng = np.random.default_rng(3)
    exact = np.full((40, 16), -1, dtype=np.int32)
    approx = np.full((40, 16), -1, dtype=np.int32)
    for t in range(40):
        n = int(rng.integers(1, 17))
        e = rng.choice(200, size=n, replace=False)
        exact[t, :n] = e
        m = int(rng.integers(0, 17))
        a = rng.choice(200, size=m, replace=False)
        a[: m // 2] = e[: min(m // 2, n)][: m // 2] if m // 2 <= n else a[: m // 2]
        a = np.unique(a)
        approx[t, : a.size] = a
    got = recall(torch.from_numpy(approx), torch.from_numpy(exact)).numpy()
    assert np.allclose(got, O.recall(approx, exact))
    rows = [dict(path="dense", recall_mean=1.0, ms=10.0), dict(path="a", recall_mean=0.95, ms=3.0),
            dict(path="b", recall_mean=0.99, ms=5.0), dict(path="c", recall_mean=0.80, ms=1.0)]
    assert choose(rows, 0.9)["path"] == "a" and choose(rows, 0.98)["path"] == "b"
    assert choose(rows, 0.999) is None


def test_dense_workspace_is_bounded_at_any_length(lib):
    """The dense scan's candidate lists hold a bounded number of entries per row
    (about 1.25 k (1 + ln(n / k))), and the workspace buffers whole row blocks up to
    a fixed budget: its size stops growing with the sequence length (beyond a
    few bytes per row block for the overflow bookkeeping)."""
    sizes = {}
    for n in (32768, 131072, 262144, 1 << 20):
        p = problem(n_q=n, n_k=n)
        sizes[n] = lib.idx_workspace_bytes(ctypes.byref(p), 0, 0, 0, 2048)
    budget = (4 << 30) + 2 * ((1 << 20) // 8) * 4 + 4096
    for n, b in sizes.items():
        assert 0 < b <= budget, (n, b)
    # far below one float per (query, key) pair: 4 n^2 bytes would be 4 GiB at 32K, 4 TiB at 1M
    assert sizes[1 << 20] < sizes[32768] * 2
    # decode shapes (at most four queries per sequence) take the split-key scan
    p = problem(batch=8, n_q=2, n_k=131072, q_pos0=131070, k_dtype=2, k_scale=FAKE)
    assert 0 < lib.idx_workspace_bytes(ctypes.byref(p), 0, 0, 0, 2048) < (64 << 20)


def test_short_workspace_is_refused(lib):
    p = problem(n_q=4096, n_k=4096)
    need = lib.idx_workspace_bytes(ctypes.byref(p), 0, 0, 0, 256)
    assert need > 0
    assert score(lib, p, topk=256, ws=FAKE, ws_bytes=need - 1) == -3


def test_static_entry_point_refuses_problems_beyond_its_scratch(lib):
    """idx_score_topk_static checks its fixed 64 MiB scratch on the host: a
    32K-token prefill needs far more and is refused before anything runs."""
    p = problem(n_q=32768, n_k=32768)
    assert lib.idx_workspace_bytes(ctypes.byref(p), 0, 0, 0, 2048) > (64 << 20)
    assert lib.idx_score_topk_static(ctypes.byref(p), 2048, FAKE, None, None) == -5
    assert b"fixed" in lib.idx_status_string(-5)
    assert lib.idx_score_topk_static(ctypes.byref(problem(n_q=0)), 8, FAKE, None, None) == -1
    assert lib.idx_score_topk_static(ctypes.byref(problem()), 0, FAKE, None, None) == -1
