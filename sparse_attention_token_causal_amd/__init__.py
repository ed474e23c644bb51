"""Causal lightning indexer and PIVOT group-shared indexing on MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/idx.h``: it checks
tensor shapes, dtypes, contiguity and devices (caller-supplied ``out`` and
``workspace`` tensors included), allocates outputs and workspace with torch, and
passes raw device pointers and the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no other path, and
the functions raise if the library has not been built.

Entry points (same names as the C ABI):

* ``score_topk``        dense causal scan + per-query top-k
* ``score_topk_static`` the same without allocating (fixed device scratch)
* ``group_proxy_scan``  PIVOT proxy per group + one shared prefix scan -> candidates
* ``refine_topk``       PIVOT-Refine: per-query re-score of the group's candidates
* ``reuse_topk``        PIVOT-Reuse: the group's shared top-k, causally filtered
* ``block_route``       block-mean routing -> Refine candidates
* ``ivf_build``         IVF index of the keys with causal versions
* ``ivf_route``         IVF routing of the group proxies -> Refine candidates
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsatc_idx.so")

IDX_F32, IDX_BF16, IDX_FP8_E4M3 = 0, 1, 2
IDX_OP_SCORE_TOPK, IDX_OP_GROUP_PROXY_SCAN, IDX_OP_REFINE_TOPK, IDX_OP_REUSE_TOPK, IDX_OP_BLOCK_ROUTE = 0, 1, 2, 3, 4
IDX_OP_IVF_BUILD, IDX_OP_IVF_ROUTE = 5, 6
IVF_TILE = 128  # granularity of refit intervals, insert batches and the index's prefix counts

_DTYPES = {torch.float32: IDX_F32, torch.bfloat16: IDX_BF16, torch.float8_e4m3fn: IDX_FP8_E4M3}


class IndexerError(RuntimeError):
    pass


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
        ("q_pos0", ctypes.c_int32), ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("k_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
        ("k", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("w", ctypes.c_void_p),
    ]


_lib = None


def library_path():
    return LIB_PATH


def load_library():
    """Load the built HIP library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise IndexerError(
                f"HIP library {LIB_PATH} is not built; run "
                "`python -m sparse_attention_token_causal_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(_Problem)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.idx_version.restype = i32
        lib.idx_status_string.restype = ctypes.c_char_p
        lib.idx_status_string.argtypes = [i32]
        lib.idx_workspace_bytes.restype = sz
        lib.idx_workspace_bytes.argtypes = [P, i32, i32, i32, i32]
        lib.idx_score_topk.restype = i32
        lib.idx_score_topk.argtypes = [P, i32, vp, vp, vp, sz, vp]
        lib.idx_score_topk_static.restype = i32
        lib.idx_score_topk_static.argtypes = [P, i32, vp, vp, vp]
        lib.idx_group_proxy_scan.restype = i32
        lib.idx_group_proxy_scan.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        lib.idx_refine_topk.restype = i32
        lib.idx_refine_topk.argtypes = [P, i32, vp, i32, i32, vp, vp, vp, sz, vp]
        lib.idx_reuse_topk.restype = i32
        lib.idx_reuse_topk.argtypes = [P, i32, vp, i32, vp, vp]
        lib.idx_block_route.restype = i32
        lib.idx_block_route.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.idx_ivf_build.restype = i32
        lib.idx_ivf_build.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.idx_ivf_route.restype = i32
        lib.idx_ivf_route.argtypes = [P, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.idx_profile_enable.restype = i32
        lib.idx_profile_enable.argtypes = [i32]
        lib.idx_profile_read.restype = i32
        lib.idx_profile_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
        _lib = lib
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc):
    if rc != 0:
        raise IndexerError(f"indexer call failed: {load_library().idx_status_string(rc).decode()} ({rc})")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise IndexerError("inputs must be contiguous tensors on the GPU")


def make_problem(q, k, w, q_scale=None, k_scale=None, q_pos0=None):
    """q [B, n_q, H, d], k [B, n_k, d], w [B, n_q, H] float32; scales float32 per token.

    q_pos0 defaults to n_k - n_q (prefill when n_q == n_k, decode otherwise).
    The returned struct keeps references to the tensors it points at.
    """
    if q.dim() != 4 or k.dim() != 3 or w.dim() != 3:
        raise IndexerError("expected q [B,n_q,H,d], k [B,n_k,d], w [B,n_q,H]")
    B, n_q, H, d = q.shape
    if k.shape[0] != B or k.shape[2] != d or tuple(w.shape) != (B, n_q, H):
        raise IndexerError("q/k/w shapes disagree")
    if w.dtype != torch.float32:
        raise IndexerError("w must be float32")
    for s, n in ((q_scale, n_q), (k_scale, k.shape[1])):
        if s is not None and (s.dtype != torch.float32 or tuple(s.shape) != (B, n)):
            raise IndexerError("scales must be float32 [B, tokens]")
    if q.dtype not in _DTYPES or k.dtype not in _DTYPES:
        raise IndexerError(f"unsupported storage dtype {q.dtype}/{k.dtype}")
    _need_gpu(q, k, w, q_scale, k_scale)
    n_k = k.shape[1]
    p = _Problem(B, n_q, n_k, n_k - n_q if q_pos0 is None else int(q_pos0), H, d,
                 _DTYPES[q.dtype], _DTYPES[k.dtype], _ptr(q), _ptr(q_scale), _ptr(k),
                 _ptr(k_scale), _ptr(w))
    p._keep = (q, k, w, q_scale, k_scale)
    return p


def workspace_bytes(p, op, group=0, n_cand=0, topk=0):
    return int(load_library().idx_workspace_bytes(ctypes.byref(p), op, group, n_cand, topk))


def _check_out(out, shape, like, name="out"):
    """A caller-supplied int32 output: exactly `shape`, contiguous, on `like`'s
    device (the kernels write every element of it).  None -> a new tensor."""
    if out is None:
        return torch.empty(shape, dtype=torch.int32, device=like.device)
    if not isinstance(out, torch.Tensor) or out.dtype != torch.int32 or tuple(out.shape) != tuple(shape) \
            or not out.is_contiguous():
        raise IndexerError(f"{name} must be a contiguous int32 tensor of shape {list(shape)}")
    if out.device != like.device:
        raise IndexerError(f"{name} must be on {like.device}, not {out.device}")
    return out


def _check_workspace_tensor(workspace, like):
    """A caller-supplied workspace: a contiguous 1-D uint8 tensor on `like`'s device."""
    if workspace is None:
        return
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or workspace.dim() != 1 \
            or not workspace.is_contiguous():
        raise IndexerError("workspace must be a contiguous 1-D uint8 tensor (its length is its size in bytes)")
    if workspace.device != like.device:
        raise IndexerError(f"workspace must be on {like.device}, not {workspace.device}")


def _workspace(p, op, device, group=0, n_cand=0, topk=0, workspace=None):
    n = workspace_bytes(p, op, group, n_cand, topk)
    if workspace is not None:
        if workspace.numel() < n:
            raise IndexerError(f"workspace has {workspace.numel()} bytes, needs {n}")
        return workspace
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def score_topk(q, k, w, topk, q_scale=None, k_scale=None, q_pos0=None, return_scores=False,
               workspace=None, out=None):
    """Dense causal indexer top-k: int32 [B, n_q, topk] (-1 padded; row order unspecified).

    With ``return_scores`` also returns the exact float32 [B, n_q, n_k] scores
    the select used (-inf beyond each query's prefix).
    """
    B, n_q = q.shape[0], q.shape[1]
    idx = _check_out(out, (B, n_q, topk), q)
    _check_workspace_tensor(workspace, q)
    lib = load_library()
    p = make_problem(q, k, w, q_scale, k_scale, q_pos0)
    scores = torch.empty((B, n_q, k.shape[1]), dtype=torch.float32, device=q.device) if return_scores else None
    ws = _workspace(p, IDX_OP_SCORE_TOPK, q.device, topk=topk, workspace=workspace)
    _check(lib.idx_score_topk(ctypes.byref(p), topk, _ptr(idx), _ptr(scores), _ptr(ws), ws.numel(),
                              _stream(q.device)))
    return (idx, scores) if return_scores else idx


def score_topk_static(q, k, w, topk, q_scale=None, k_scale=None, q_pos0=None, out=None):
    """``score_topk`` through the entry point that allocates nothing on the
    device (its scratch is the library's fixed 64 MiB device array; see
    idx_score_topk_static).  ``out`` may be given so that nothing is
    allocated here either."""
    B, n_q = q.shape[0], q.shape[1]
    idx = _check_out(out, (B, n_q, topk), q)
    lib = load_library()
    p = make_problem(q, k, w, q_scale, k_scale, q_pos0)
    _check(lib.idx_score_topk_static(ctypes.byref(p), topk, _ptr(idx), None, _stream(q.device)))
    return idx


def group_proxy_scan(q, k, w, group, n_cand, q_scale=None, k_scale=None, q_pos0=None,
                     return_proxy=False, return_scores=False, workspace=None, out=None):
    """PIVOT proxy + shared scan: candidates int32 [B, n_g, n_cand] (-1 padded).

    ``return_proxy`` adds the stored proxy (q as bfloat16, or float32 for
    float32 q; w float32); ``return_scores`` adds the proxy scores [B, n_g, n_k].
    ``out`` may supply the candidate tensor.
    """
    B, n_q, H, d = q.shape
    n_g = -(-n_q // group)
    cand = _check_out(out, (B, n_g, n_cand), q)
    _check_workspace_tensor(workspace, q)
    lib = load_library()
    p = make_problem(q, k, w, q_scale, k_scale, q_pos0)
    pq = pw = ps = None
    if return_proxy:
        pq = torch.empty((B, n_g, H, d), dtype=torch.float32 if q.dtype == torch.float32 else torch.bfloat16,
                         device=q.device)
        pw = torch.empty((B, n_g, H), dtype=torch.float32, device=q.device)
    if return_scores:
        ps = torch.empty((B, n_g, k.shape[1]), dtype=torch.float32, device=q.device)
    ws = _workspace(p, IDX_OP_GROUP_PROXY_SCAN, q.device, group, n_cand, workspace=workspace)
    _check(lib.idx_group_proxy_scan(ctypes.byref(p), group, n_cand, _ptr(cand), _ptr(pq), _ptr(pw),
                                    _ptr(ps), _ptr(ws), ws.numel(), _stream(q.device)))
    res = [cand]
    if return_proxy:
        res += [pq, pw]
    if return_scores:
        res.append(ps)
    return res[0] if len(res) == 1 else tuple(res)


def refine_topk(q, k, w, cand, group, topk, q_scale=None, k_scale=None, q_pos0=None,
                return_scores=False, workspace=None, out=None):
    """PIVOT-Refine: int32 [B, n_q, topk]; optional per-candidate scores [B, n_q, n_cand]."""
    B, n_q = q.shape[0], q.shape[1]
    n_g = -(-n_q // group)
    if not isinstance(cand, torch.Tensor) or cand.dtype != torch.int32 or cand.dim() != 3 \
            or tuple(cand.shape[:2]) != (B, n_g) or not cand.is_contiguous():
        raise IndexerError("cand must be a contiguous int32 tensor [B, n_g, n_cand]")
    idx = _check_out(out, (B, n_q, topk), q)
    _check_workspace_tensor(workspace, q)
    lib = load_library()
    p = make_problem(q, k, w, q_scale, k_scale, q_pos0)
    _need_gpu(cand)
    n_cand = cand.shape[2]
    sc = torch.empty((B, n_q, n_cand), dtype=torch.float32, device=q.device) if return_scores else None
    ws = _workspace(p, IDX_OP_REFINE_TOPK, q.device, group, n_cand, topk, workspace=workspace)
    _check(lib.idx_refine_topk(ctypes.byref(p), group, _ptr(cand), n_cand, topk, _ptr(idx), _ptr(sc),
                               _ptr(ws), ws.numel(), _stream(q.device)))
    return (idx, sc) if return_scores else idx


def reuse_topk(proxy_topk, group, n_q, n_k, q_pos0=None, out=None):
    """PIVOT-Reuse: int32 [B, n_q, topk] from the proxy top-k [B, n_g, topk]."""
    if not isinstance(proxy_topk, torch.Tensor) or proxy_topk.dtype != torch.int32 or proxy_topk.dim() != 3 \
            or not proxy_topk.is_contiguous():
        raise IndexerError("proxy_topk must be a contiguous int32 tensor [B, n_g, topk]")
    B, n_g, topk = proxy_topk.shape
    if n_g != -(-n_q // group):
        raise IndexerError("proxy_topk has the wrong number of groups")
    idx = _check_out(out, (B, n_q, topk), proxy_topk)
    lib = load_library()
    _need_gpu(proxy_topk)
    p = _Problem(B, n_q, n_k, n_k - n_q if q_pos0 is None else int(q_pos0), 0, 0, 0, 0,
                 None, None, None, None, None)
    _check(lib.idx_reuse_topk(ctypes.byref(p), group, _ptr(proxy_topk), topk, _ptr(idx),
                              _stream(proxy_topk.device)))
    return idx


def block_route(q, k, w, group, block, n_sel, q_scale=None, k_scale=None, q_pos0=None,
                return_means=False, return_scores=False, return_proxy=False, workspace=None):
    """Block-mean routing: candidates int32 [B, n_g, (n_sel + 1) * block] (-1 padded).

    ``return_means`` adds the stored block means [B, n_b, d] (bfloat16, or
    float32 for float32 keys); ``return_scores`` adds the block scores
    [B, n_g, n_b] (-inf where a block is not routable); ``return_proxy`` adds
    the stored proxy q and w.
    """
    _check_workspace_tensor(workspace, q)
    lib = load_library()
    p = make_problem(q, k, w, q_scale, k_scale, q_pos0)
    B, n_q, H, d = q.shape
    n_k = k.shape[1]
    n_g, n_b = -(-n_q // group), -(-n_k // block)
    cand = torch.empty((B, n_g, (n_sel + 1) * block), dtype=torch.int32, device=q.device)
    km = bs = pq = pw = None
    if return_means:
        km = torch.empty((B, n_b, d), dtype=torch.float32 if k.dtype == torch.float32 else torch.bfloat16,
                         device=q.device)
    if return_scores:
        bs = torch.empty((B, n_g, n_b), dtype=torch.float32, device=q.device)
    if return_proxy:
        pq = torch.empty((B, n_g, H, d), dtype=torch.float32 if q.dtype == torch.float32 else torch.bfloat16,
                         device=q.device)
        pw = torch.empty((B, n_g, H), dtype=torch.float32, device=q.device)
    ws = _workspace(p, IDX_OP_BLOCK_ROUTE, q.device, group, block, n_sel, workspace=workspace)
    _check(lib.idx_block_route(ctypes.byref(p), group, block, n_sel, _ptr(cand), _ptr(km), _ptr(bs), _ptr(pq),
                               _ptr(pw), _ptr(ws), ws.numel(), _stream(q.device)))
    res = [cand]
    if return_means:
        res.append(km)
    if return_scores:
        res.append(bs)
    if return_proxy:
        res += [pq, pw]
    return res[0] if len(res) == 1 else tuple(res)


def ivf_build(k, n_clusters, refit, iters, k_scale=None, return_assign=False, workspace=None):
    """IVF index with causal versions over keys k [B, n_k, d] (see idx_ivf_build).

    Returns a dict with ``centroids`` [B, n_v, m, d] (bfloat16, float32 for
    float32 keys), ``offsets`` [B, n_v, m + 1], ``members`` [B, n_v, n_k],
    ``counts`` [B, n_v, ceil(n_k / 128) + 1, m] (int32), and with
    ``return_assign`` the per-version cluster of every key of the window
    ``assign`` [B, n_v, n_k] (-1 beyond it); plus the parameters.
    n_v = n_k // refit may be 0 (then the arrays are empty).
    """
    _check_workspace_tensor(workspace, k)
    lib = load_library()
    if k.dim() != 3 or k.dtype not in _DTYPES:
        raise IndexerError("expected k [B, n_k, d] in float32, bfloat16 or float8_e4m3fn")
    if k_scale is not None and (k_scale.dtype != torch.float32 or tuple(k_scale.shape) != tuple(k.shape[:2])):
        raise IndexerError("k_scale must be float32 [B, n_k]")
    _need_gpu(k, k_scale)
    B, n_k, d = k.shape
    m = int(n_clusters)
    n_v = n_k // int(refit) if refit > 0 else 0
    nt = -(-n_k // IVF_TILE)
    dev = k.device
    p = _Problem(B, 0, n_k, 0, 0, d, 0, _DTYPES[k.dtype], None, None, _ptr(k), _ptr(k_scale), None)
    cdt = torch.float32 if k.dtype == torch.float32 else torch.bfloat16
    idx = dict(centroids=torch.empty((B, n_v, m, d), dtype=cdt, device=dev),
               offsets=torch.empty((B, n_v, m + 1), dtype=torch.int32, device=dev),
               members=torch.empty((B, n_v, n_k), dtype=torch.int32, device=dev),
               counts=torch.empty((B, n_v, nt + 1, m), dtype=torch.int32, device=dev),
               n_clusters=m, refit=int(refit), iters=int(iters))
    asg = torch.empty((B, n_v, n_k), dtype=torch.int32, device=dev) if return_assign else None
    n = int(lib.idx_workspace_bytes(ctypes.byref(p), IDX_OP_IVF_BUILD, 0, m, 0))
    if workspace is not None and workspace.numel() < n:
        raise IndexerError(f"workspace has {workspace.numel()} bytes, needs {n}")
    ws = workspace if workspace is not None else torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _check(lib.idx_ivf_build(ctypes.byref(p), m, int(refit), int(iters), _ptr(idx["centroids"]),
                             _ptr(idx["offsets"]), _ptr(idx["members"]), _ptr(idx["counts"]), _ptr(asg),
                             _ptr(ws), ws.numel(), _stream(dev)))
    if return_assign:
        idx["assign"] = asg
    return idx


def ivf_route(q, k, w, index, group, insert_batch, n_cand, q_scale=None, k_scale=None, q_pos0=None,
              return_scores=False, return_proxy=False, workspace=None):
    """IVF routing through ``index`` (from ``ivf_build`` on the same keys):
    candidates int32 [B, n_g, n_cand] (-1 padded) for ``refine_topk``.

    ``return_scores`` adds the cluster scores [B, n_g, m] (-inf without a
    version); ``return_proxy`` adds the stored proxy q and w.
    """
    _check_workspace_tensor(workspace, q)
    lib = load_library()
    p = make_problem(q, k, w, q_scale, k_scale, q_pos0)
    B, n_q, H, d = q.shape
    n_g = -(-n_q // group)
    m, R = index["n_clusters"], index["refit"]
    cand = torch.empty((B, n_g, n_cand), dtype=torch.int32, device=q.device)
    sc = torch.empty((B, n_g, m), dtype=torch.float32, device=q.device) if return_scores else None
    pq = pw = None
    if return_proxy:
        pq = torch.empty((B, n_g, H, d), dtype=torch.float32 if q.dtype == torch.float32 else torch.bfloat16,
                         device=q.device)
        pw = torch.empty((B, n_g, H), dtype=torch.float32, device=q.device)
    ws = _workspace(p, IDX_OP_IVF_ROUTE, q.device, group, m, workspace=workspace)
    _check(lib.idx_ivf_route(ctypes.byref(p), group, m, R, int(insert_batch), int(n_cand),
                             _ptr(index["centroids"]), _ptr(index["offsets"]), _ptr(index["members"]),
                             _ptr(index["counts"]), _ptr(cand), _ptr(sc), _ptr(pq), _ptr(pw), _ptr(ws),
                             ws.numel(), _stream(q.device)))
    res = [cand]
    if return_scores:
        res.append(sc)
    if return_proxy:
        res += [pq, pw]
    return res[0] if len(res) == 1 else tuple(res)


KERNEL_KINDS = ("score", "select", "proxy", "reuse", "fill", "ivf_build", "ivf_route", "rescan", "proxy_scan",
                "gather_scan")


def profile_enable(on=True):
    """Bracket every kernel the library enqueues with HIP events (measurement aid)."""
    _check(load_library().idx_profile_enable(1 if on else 0))


def profile_read():
    """{kind: (total_ms, launches)} since the last read; synchronizes on the events."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_float * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(load_library().idx_profile_read(ms, cnt))
    return {KERNEL_KINDS[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


__all__ = ["profile_enable", "profile_read", "score_topk", "score_topk_static", "group_proxy_scan", "refine_topk", "reuse_topk",
           "block_route", "ivf_build", "ivf_route", "make_problem",
           "workspace_bytes", "load_library", "library_path", "IndexerError"]
