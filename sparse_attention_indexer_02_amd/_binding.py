"""ctypes binding of libsparse_indexer.so (include/sparse_indexer.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream, every step of the computation runs in the library's HIP
kernels.  Nothing here falls back to a CPU or PyTorch implementation; a
missing library raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_indexer.so")

SI_OK = 0
SI_F32, SI_BF16, SI_FP8_E4M3FN = 0, 1, 2
STATUS_NAMES = {0: "SI_OK", 1: "SI_ERR_INVALID_ARGUMENT", 2: "SI_ERR_ROWS_MISMATCH",
                3: "SI_ERR_SEGMENTS_OUT_OF_RANGE", 4: "SI_ERR_LEARNED_KEEP_OUT_OF_RANGE",
                5: "SI_ERR_UNSUPPORTED_DTYPE", 6: "SI_ERR_WORKSPACE_TOO_SMALL", 7: "SI_ERR_DEVICE",
                8: "SI_ERR_SCRATCH_LIMIT"}


class SparseIndexerError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class DosaParams(C.Structure):
    _fields_ = [("n_seeds", C.c_int32), ("n_rep_queries", C.c_int32), ("rep_topk", C.c_int32),
                ("kept_heads", C.c_int32), ("neg_active_frac", C.c_float),
                ("seed_ids", C.c_void_p), ("survivor_capacity", C.c_int32),
                ("shared_streams", C.c_int32)]


class DosaStats(C.Structure):
    _fields_ = [("tau", C.c_void_p), ("n_survivors", C.c_void_p), ("fallback", C.c_void_p),
                ("n_shared", C.c_void_p)]


_lib = None
vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
SIGNATURES = {
    "idx_score_topk": (i32, [vp, i32, vp, i32, vp, vp, i64, vp, vp, i32, i32, i32, i64, i64, i32,
                             vp, vp, vp, sz, vp]),
    "idx_score_topk_workspace": (sz, [i32, i32, i32, i64, i32]),
    "idx_score_topk_noalloc": (i32, [vp, i32, vp, i32, vp, vp, i64, vp, vp, i32, i32, i32, i64,
                                     i64, i32, vp, vp, vp]),
    "idx_score_topk_witness": (i32, [vp, i32, vp, i32, vp, vp, i64, vp, vp, i32, i32, i32, i64,
                                     i64, i32, vp, vp, vp, i32, i32, i32, vp, sz, vp]),
    "idx_score_topk_fused": (i32, [vp, i32, vp, i32, vp, vp, i64, vp, vp, i32, i32, i32, i64,
                                   i64, i32, vp, vp, vp, i32, i32, i32, vp, sz, vp]),
    "idx_score_topk_prior": (i32, [vp, i32, vp, i32, vp, vp, i64, vp, vp, i32, i32, i32, i64, i64,
                                   i32, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
    "idx_score_topk_prior_workspace": (sz, [i32, i64, i32]),
    "idx_score": (i32, [vp, i32, vp, i32, vp, vp, i64, vp, vp, i32, i32, i32, i64, i64, vp, i64,
                        vp]),
    "rows_topk": (i32, [vp, i64, vp, vp, i64, i64, i32, i32, vp, vp, vp, sz, vp]),
    "rows_topk_workspace": (sz, [i32, i64, i32]),
    "dosa_prune_topk": (i32, [vp, vp, i32, vp, i64, vp, i32, i32, i32, i64, i32, vp, vp, vp, vp,
                              vp, sz, vp]),
    "dosa_prune_topk_workspace": (sz, [i32, i32, i32, i64, i32, vp]),
    "kvwitness_merge": (i32, [vp, i32, i32, vp, i32, i32, i32, vp]),
    "block_sparse_select": (i32, [vp, vp, vp, i32, i32, i32, i64, i32, i32, i32, i32, vp, i32, vp,
                                  vp, sz, vp]),
    "block_sparse_select_workspace": (sz, [i32, i32, i64, i32]),
    "positions_of_blocks": (i32, [vp, i32, i32, i32, vp, i64, i32, vp, i32, vp, vp]),
    "gather_slots": (i32, [vp, i32, i32, vp, vp, vp, i32, i32, vp, vp]),
    "si_status_string": (C.c_char_p, [i32]),
}


def lib():
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_indexer_02_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name, None)
            if f is None:
                continue  # reported by exported_symbols(); calling it raises
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().si_status_string(status).decode()


def _check(status: int, what: str):
    if status != SI_OK:
        raise SparseIndexerError(status, what)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _dev_tensor(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dtype_code(t, name):
    if t.dtype == torch.float32:
        return SI_F32
    if t.dtype == torch.bfloat16:
        return SI_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return SI_FP8_E4M3FN
    raise ValueError(f"{name}: unsupported dtype {t.dtype}")


def _workspace(nbytes, dev, given):
    """The caller's workspace, or a fresh one (the caching allocator returns
    blocks aligned far beyond the 256 bytes the library asks for)."""
    if nbytes == 0:
        return given, 0
    if given is not None:
        return given, given.numel() * given.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=dev), nbytes


def _default_max_vis(n_k, k_row_offset, vis_len, n_q):
    """max_vis when the caller gives none: n_k for shared keys; for per-row
    keys the longest visible length, read back to the host (a device
    synchronisation: callers that must not block pass max_vis)."""
    if k_row_offset is None:
        return n_k
    return int(vis_len.max().item()) if n_q else 0


def idx_score_topk(q, k, w, vis_len, topk, *, k_scale=None, k_row_offset=None, max_vis=None,
                   out_idx=None, out_score=None, want_scores=True, workspace=None):
    """Top-K of s = sum_h w_h relu(q_h . k) per row; returns (idx, scores|None).

    q [n_q, H, D] bf16/f32; k [n_k, D] bf16/f32/fp8-e4m3fn (uint8 storage ok)
    with k_scale [n_k] f32 for fp8; w [n_q, H] or [H] f32; vis_len [n_q] i32;
    k_row_offset [n_q] i64 or None.  max_vis defaults to n_k for shared keys.
    With per-row keys and max_vis=None it is vis_len.max() read back to the
    host, which synchronises the device (the library's calls never do): pass
    max_vis to keep the call asynchronous.
    """
    _dev_tensor(q, "q")
    _dev_tensor(k, "k")
    _dev_tensor(w, "w", torch.float32)
    _dev_tensor(vis_len, "vis_len", torch.int32)
    dev = q.device
    n_q, H, D = q.shape
    n_k = k.shape[0]
    if max_vis is None:
        max_vis = _default_max_vis(n_k, k_row_offset, vis_len, n_q)
    w_stride = H if w.dim() == 2 else 0
    if out_idx is None:
        out_idx = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_scores:
        out_score = torch.empty((n_q, topk), dtype=torch.float32, device=dev)
    need = lib().idx_score_topk_workspace(n_q, H, D, max_vis, topk)
    ws, ws_bytes = _workspace(need, dev, workspace)
    st = lib().idx_score_topk(_ptr(q), _dtype_code(q, "q"), _ptr(k), _dtype_code(k, "k"),
                              _ptr(k_scale), _ptr(w), w_stride, _ptr(k_row_offset),
                              _ptr(vis_len), n_q, H, D, n_k, max_vis, topk, _ptr(out_idx),
                              _ptr(out_score), _ptr(ws), ws_bytes, _stream(dev))
    _check(st, "idx_score_topk")
    return out_idx, out_score


def idx_score_topk_noalloc(q, k, w, vis_len, topk, *, k_scale=None, k_row_offset=None,
                           max_vis=None, out_idx=None, out_score=None, want_scores=True):
    """idx_score_topk with the library's fixed scratch instead of a workspace
    (the C call allocates nothing; this wrapper allocates the outputs only if
    they are not given).  Returns (idx, scores|None)."""
    _dev_tensor(q, "q")
    _dev_tensor(k, "k")
    _dev_tensor(w, "w", torch.float32)
    _dev_tensor(vis_len, "vis_len", torch.int32)
    dev = q.device
    n_q, H, D = q.shape
    n_k = k.shape[0]
    if max_vis is None:
        max_vis = _default_max_vis(n_k, k_row_offset, vis_len, n_q)
    w_stride = H if w.dim() == 2 else 0
    if out_idx is None:
        out_idx = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_scores:
        out_score = torch.empty((n_q, topk), dtype=torch.float32, device=dev)
    st = lib().idx_score_topk_noalloc(_ptr(q), _dtype_code(q, "q"), _ptr(k), _dtype_code(k, "k"),
                                      _ptr(k_scale), _ptr(w), w_stride, _ptr(k_row_offset),
                                      _ptr(vis_len), n_q, H, D, n_k, max_vis, topk,
                                      _ptr(out_idx), _ptr(out_score), _stream(dev))
    _check(st, "idx_score_topk_noalloc")
    return out_idx, out_score


def idx_score_topk_witness(q, k, w, vis_len, topk, context_lens, num_segments, *, keep=None,
                           max_replacements=None, k_scale=None, k_row_offset=None, max_vis=None,
                           out_idx=None, out_score=None, want_scores=True, workspace=None,
                           fused=False):
    """idx_score_topk then the segment-witness merge of its rows, in one pass;
    keep/max_replacements default to the serving convention (topk - S, S).
    fused=True calls idx_score_topk_fused (one kernel; prefill layout only).
    Returns (idx, scores|None)."""
    _dev_tensor(q, "q")
    _dev_tensor(k, "k")
    _dev_tensor(w, "w", torch.float32)
    _dev_tensor(vis_len, "vis_len", torch.int32)
    _dev_tensor(context_lens, "context_lens", torch.int32)
    dev = q.device
    n_q, H, D = q.shape
    n_k = k.shape[0]
    if keep is None:
        keep = max(topk - num_segments, 0)
    if max_replacements is None:
        max_replacements = num_segments
    if max_vis is None:
        max_vis = _default_max_vis(n_k, k_row_offset, vis_len, n_q)
    w_stride = H if w.dim() == 2 else 0
    if out_idx is None:
        out_idx = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_scores:
        out_score = torch.empty((n_q, topk), dtype=torch.float32, device=dev)
    need = lib().idx_score_topk_workspace(n_q, H, D, max_vis, topk)
    ws, ws_bytes = _workspace(need, dev, workspace)
    name = "idx_score_topk_fused" if fused else "idx_score_topk_witness"
    st = getattr(lib(), name)(_ptr(q), _dtype_code(q, "q"), _ptr(k), _dtype_code(k, "k"),
                              _ptr(k_scale), _ptr(w), w_stride, _ptr(k_row_offset),
                              _ptr(vis_len), n_q, H, D, n_k, max_vis, topk, _ptr(out_idx),
                              _ptr(out_score), _ptr(context_lens), num_segments, keep,
                              max_replacements, _ptr(ws), ws_bytes, _stream(dev))
    _check(st, name)
    return out_idx, out_score


def idx_score_topk_prior(q, k, w, vis_len, topk, prior_ids, *, k_scale=None, k_row_offset=None,
                         max_vis=None, out_idx=None, out_score=None, want_scores=True,
                         want_stats=False, workspace=None):
    """idx_score_topk's result through the decode path that selects only among
    keys at or above a threshold from the prior ids [n_q, P] (i32, e.g. the
    previous step's ids).  Returns (idx, scores|None, stats|None) with stats =
    (tau [n_q] f32, survivors [n_q] i32)."""
    _dev_tensor(q, "q")
    _dev_tensor(k, "k")
    _dev_tensor(w, "w", torch.float32)
    _dev_tensor(vis_len, "vis_len", torch.int32)
    _dev_tensor(prior_ids, "prior_ids", torch.int32)
    dev = q.device
    n_q, H, D = q.shape
    n_k = k.shape[0]
    if max_vis is None:
        max_vis = _default_max_vis(n_k, k_row_offset, vis_len, n_q)
    w_stride = H if w.dim() == 2 else 0
    if out_idx is None:
        out_idx = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_scores:
        out_score = torch.empty((n_q, topk), dtype=torch.float32, device=dev)
    tau = surv = None
    if want_stats:
        tau = torch.empty(n_q, dtype=torch.float32, device=dev)
        surv = torch.empty(n_q, dtype=torch.int32, device=dev)
    need = lib().idx_score_topk_prior_workspace(n_q, max_vis, topk)
    ws, ws_bytes = _workspace(need, dev, workspace)
    st = lib().idx_score_topk_prior(_ptr(q), _dtype_code(q, "q"), _ptr(k), _dtype_code(k, "k"),
                                    _ptr(k_scale), _ptr(w), w_stride, _ptr(k_row_offset),
                                    _ptr(vis_len), n_q, H, D, n_k, max_vis, topk,
                                    _ptr(prior_ids), prior_ids.shape[1], _ptr(out_idx),
                                    _ptr(out_score), _ptr(tau), _ptr(surv), _ptr(ws), ws_bytes,
                                    _stream(dev))
    _check(st, "idx_score_topk_prior")
    return out_idx, out_score, ((tau, surv) if want_stats else None)


def idx_score(q, k, w, vis_len, *, k_scale=None, k_row_offset=None, max_vis=None,
              out_scores=None):
    """Score rows only: out_scores [n_q, max_vis] f32 (entries past vis_r untouched)."""
    _dev_tensor(q, "q")
    _dev_tensor(k, "k")
    _dev_tensor(w, "w", torch.float32)
    _dev_tensor(vis_len, "vis_len", torch.int32)
    dev = q.device
    n_q, H, D = q.shape
    n_k = k.shape[0]
    if max_vis is None:
        max_vis = _default_max_vis(n_k, k_row_offset, vis_len, n_q)
    if out_scores is None:
        out_scores = torch.empty((n_q, max_vis), dtype=torch.float32, device=dev)
    stride = out_scores.shape[1] if out_scores.dim() == 2 else max_vis
    st = lib().idx_score(_ptr(q), _dtype_code(q, "q"), _ptr(k), _dtype_code(k, "k"),
                         _ptr(k_scale), _ptr(w), H if w.dim() == 2 else 0, _ptr(k_row_offset),
                         _ptr(vis_len), n_q, H, D, n_k, max_vis, _ptr(out_scores), stride,
                         _stream(dev))
    _check(st, "idx_score")
    return out_scores


def rows_topk(scores, vis_len, topk, *, k_row_offset=None, n_k=None, max_vis=None,
              out_idx=None, out_score=None, want_scores=True, workspace=None):
    """Top-K of each score row's first vis_r entries; returns (idx, scores|None).
    Rows longer than 8192 need a workspace (allocated here when not given)."""
    _dev_tensor(scores, "scores", torch.float32)
    _dev_tensor(vis_len, "vis_len", torch.int32)
    dev = scores.device
    n_rows, stride = scores.shape
    if max_vis is None:
        max_vis = stride
    if n_k is None:
        n_k = max_vis
    if out_idx is None:
        out_idx = torch.empty((n_rows, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_scores:
        out_score = torch.empty((n_rows, topk), dtype=torch.float32, device=dev)
    need = lib().rows_topk_workspace(n_rows, max_vis, topk)
    ws, ws_bytes = _workspace(need, dev, workspace)
    st = lib().rows_topk(_ptr(scores), stride, _ptr(vis_len), _ptr(k_row_offset), n_k, max_vis,
                         n_rows, topk, _ptr(out_idx), _ptr(out_score), _ptr(ws), ws_bytes,
                         _stream(dev))
    _check(st, "rows_topk")
    return out_idx, out_score


def dosa_prune_topk(q, k, w, vis_len, topk, *, n_seeds=12288, n_rep_queries=4, rep_topk=2048,
                    kept_heads=16, neg_active_frac=0.5, seed_ids=None, survivor_capacity=None,
                    out_idx=None, out_score=None, want_scores=True, want_stats=False,
                    workspace=None, shared_streams=False):
    """DoSA certified-prune top-K (bit-identical to idx_score_topk); returns
    (idx, scores|None, stats dict|None)."""
    _dev_tensor(q, "q", torch.bfloat16)
    _dev_tensor(k, "k", torch.bfloat16)
    _dev_tensor(w, "w", torch.float32)
    _dev_tensor(vis_len, "vis_len", torch.int32)
    dev = q.device
    n_q, H, D = q.shape
    n_k = k.shape[0]
    if survivor_capacity is None:
        survivor_capacity = max(4 * topk, 8192)
    w_stride = H if w.dim() == 2 else 0
    p = DosaParams(n_seeds, n_rep_queries, rep_topk, kept_heads, neg_active_frac,
                   _ptr(seed_ids), survivor_capacity, 1 if shared_streams else 0)
    if out_idx is None:
        out_idx = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_scores:
        out_score = torch.empty((n_q, topk), dtype=torch.float32, device=dev)
    stats = None
    sp = None
    if want_stats:
        stats = dict(tau=torch.empty(n_q, dtype=torch.float32, device=dev),
                     n_survivors=torch.empty(n_q, dtype=torch.int32, device=dev),
                     fallback=torch.empty(n_q, dtype=torch.int32, device=dev),
                     n_shared=torch.empty(n_q, dtype=torch.int32, device=dev))
        sp = DosaStats(_ptr(stats["tau"]), _ptr(stats["n_survivors"]), _ptr(stats["fallback"]),
                       _ptr(stats["n_shared"]))
    need = lib().dosa_prune_topk_workspace(n_q, H, D, n_k, topk, C.byref(p))
    ws, ws_bytes = _workspace(need, dev, workspace)
    st = lib().dosa_prune_topk(_ptr(q), _ptr(k), SI_BF16, _ptr(w), w_stride, _ptr(vis_len), n_q, H,
                               D, n_k, topk, C.byref(p), _ptr(out_idx), _ptr(out_score),
                               C.byref(sp) if sp is not None else None, _ptr(ws), ws_bytes,
                               _stream(dev))
    _check(st, "dosa_prune_topk")
    return out_idx, out_score, stats


def kvwitness_merge(topk_idx, context_lens, num_segments, keep=None, max_replacements=None):
    """In-place witness merge of topk_idx [rows, topk]; serving defaults
    keep = topk - S (saturating), max_replacements = S."""
    _dev_tensor(topk_idx, "topk_idx", torch.int32)
    _dev_tensor(context_lens, "context_lens", torch.int32)
    rows, topk = topk_idx.shape
    if keep is None:
        keep = max(topk - num_segments, 0)
    if max_replacements is None:
        max_replacements = num_segments
    st = lib().kvwitness_merge(_ptr(topk_idx), rows, topk, _ptr(context_lens), num_segments, keep,
                               max_replacements, _stream(topk_idx.device))
    _check(st, "kvwitness_merge")
    return topk_idx


def block_sparse_select(index_q, index_k, query_pos, *, block_size=128, top_blocks=32,
                        init_blocks=1, local_blocks=2, out_width=None, out_blocks=None,
                        out_count=None, workspace=None):
    """Per (query, KV head) ascending block lists (-1 padded) and counts."""
    _dev_tensor(index_q, "index_q", torch.float32)
    _dev_tensor(index_k, "index_k", torch.float32)
    _dev_tensor(query_pos, "query_pos", torch.int64)
    dev = index_q.device
    n_q, H, D = index_q.shape
    n_pos = index_k.shape[0]
    if out_width is None:
        out_width = max(top_blocks, init_blocks + local_blocks, 1)
    if out_blocks is None:
        out_blocks = torch.empty((n_q, H, out_width), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((n_q, H), dtype=torch.int32, device=dev)
    need = lib().block_sparse_select_workspace(n_q, H, n_pos, block_size)
    ws, ws_bytes = _workspace(need, dev, workspace)
    st = lib().block_sparse_select(_ptr(index_q), _ptr(index_k), _ptr(query_pos), n_q, H, D, n_pos,
                                   block_size, top_blocks, init_blocks, local_blocks,
                                   _ptr(out_blocks), out_width, _ptr(out_count), _ptr(ws),
                                   ws_bytes, _stream(dev))
    _check(st, "block_sparse_select")
    return out_blocks, out_count


def positions_of_blocks(blocks, query_pos, n_pos, block_size, *, out_width=None, out_pos=None,
                        out_count=None):
    """Positions each (query, KV head) block list covers, ascending, deduplicated and
    causally clipped, then -1; returns (out_pos [n_q, H, out_width] i32, out_count)."""
    _dev_tensor(blocks, "blocks", torch.int32)
    _dev_tensor(query_pos, "query_pos", torch.int64)
    dev = blocks.device
    n_q, H, width = blocks.shape
    if out_width is None:
        out_width = max(min(width * block_size, n_pos), 1)
    if out_pos is None:
        out_pos = torch.empty((n_q, H, out_width), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((n_q, H), dtype=torch.int32, device=dev)
    st = lib().positions_of_blocks(_ptr(blocks), n_q, H, width, _ptr(query_pos), n_pos,
                                   block_size, _ptr(out_pos), out_width, _ptr(out_count),
                                   _stream(dev))
    _check(st, "positions_of_blocks")
    return out_pos, out_count


def gather_slots(idx, lens, *, row_start=None, page_table=None, page_size=0, out=None):
    """KV slots [rows, width] i64 of row-relative entries (-1 where an entry names no
    token of its row), through row starts (flat KV) or a page table (paged KV)."""
    _dev_tensor(idx, "idx", torch.int32)
    _dev_tensor(lens, "lens", torch.int32)
    if row_start is not None:
        _dev_tensor(row_start, "row_start", torch.int64)
    if page_table is not None:
        _dev_tensor(page_table, "page_table", torch.int32)
    dev = idx.device
    rows, width = idx.shape
    ppr = page_table.shape[1] if page_table is not None else 0
    if out is None:
        out = torch.empty((rows, width), dtype=torch.int64, device=dev)
    st = lib().gather_slots(_ptr(idx), rows, width, _ptr(lens), _ptr(row_start), _ptr(page_table),
                            ppr, page_size, _ptr(out), _stream(dev))
    _check(st, "gather_slots")
    return out
