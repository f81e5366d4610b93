"""ctypes wrapper of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It never imports the
HIP library and the library never imports it.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

F32, BF16, FP8_E4M3FN = 0, 1, 2
OK, INVALID_ARGUMENT, ROWS_MISMATCH, SEGMENTS_OUT_OF_RANGE, KEEP_OUT_OF_RANGE, NOT_ENOUGH_KEYS = range(6)


class Problem(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_dtype", C.c_int32), ("k", C.c_void_p),
                ("k_dtype", C.c_int32), ("k_scale", C.c_void_p), ("w", C.c_void_p),
                ("w_row_stride", C.c_int64), ("k_row_offset", C.c_void_p),
                ("vis_len", C.c_void_p), ("n_q", C.c_int32), ("H", C.c_int32),
                ("D", C.c_int32), ("n_k", C.c_int64), ("max_vis", C.c_int64),
                ("topk", C.c_int32)]


class DosaParams(C.Structure):
    _fields_ = [("n_seeds", C.c_int32), ("n_rep_queries", C.c_int32), ("rep_topk", C.c_int32),
                ("kept_heads", C.c_int32), ("neg_active_frac", C.c_double),
                ("survivor_capacity", C.c_int64)]


class DosaRowStats(C.Structure):
    _fields_ = [("tau", C.c_double), ("n_kept_heads", C.c_int32), ("n_pos_omitted", C.c_int32),
                ("n_neg_aggregated", C.c_int32), ("n_neg_dropped", C.c_int32),
                ("n_scanned", C.c_int64), ("n_survivors", C.c_int64),
                ("n_kept_survivors", C.c_int64), ("fallback", C.c_int32),
                ("head_dots", C.c_int64), ("R", C.c_double)]


class DosaDiag(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("head_role", "anchor", "beta", "dnorm", "wfold", "act",
                                          "a_agg", "pos_part", "neg_part", "U")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle.build import build
            build()
        L = C.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = C.c_void_p, C.c_int32, C.c_int64, C.c_double
        sig = {
            "orc_e4m3fn_to_double": (dbl, [C.c_uint8]),
            "orc_visible": (i64, [vp, i32]),
            "orc_score_row": (i64, [vp, i32, vp, vp, vp]),
            "orc_topk": (i32, [vp, vp, i64, i32, vp, vp]),
            "orc_idx_score_topk_rows": (None, [vp, vp, i32, vp, vp, vp, vp, vp, i64]),
            "orc_segment_of": (i64, [i64, i64, i64]),
            "orc_segment_edge": (i64, [i64, i64, i64]),
            "orc_occupied_segment": (i64, [i64, i64, i64]),
            "orc_witness_indices": (i32, [vp, i32, i32, vp, i32, vp]),
            "orc_kvwitness_merge": (i32, [vp, i32, i32, vp, i32, i32, i32]),
            "orc_segment_coverage": (dbl, [vp, i32, i64, i64]),
            "orc_block_dot": (C.c_float, [vp, vp, i32]),
            "orc_causal_blocks": (i64, [i64, i64]),
            "orc_block_select_query": (i32, [vp, vp, i64, i32, i32, i64, i32, i32, i32, i32, vp,
                                             i32, vp, vp]),
            "orc_block_select_rows": (None, [vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, i32,
                                             i32, vp, i32, vp]),
            "orc_positions_of_blocks": (i64, [vp, i32, i64, i64, i32, vp]),
            "orc_positions_of_block_rows": (None, [vp, i32, i32, i32, vp, i64, i32, vp, i64, vp]),
            "orc_gather_slots": (None, [vp, i32, i32, vp, vp, vp, i32, i32, vp]),
            "orc_dosa_common_prefix": (i32, [vp]),
            "orc_dosa_rep_row": (i32, [i32, i32, i32]),
            "orc_dosa_seeds": (i32, [vp, vp, vp, vp]),
            "orc_dosa_row": (i32, [vp, vp, vp, i32, vp, vp, vp, vp]),
            "orc_dosa_rows": (None, [vp, vp, vp, vp, i32, vp, vp, vp]),
            "orc_dosa_head_dots": (i64, [i64, i64, i64, i64, i32]),
            "orc_num_threads": (i32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


class _Keep:
    """Holds the arrays a Problem points at, so they outlive the struct."""

    def __init__(self, cfg):
        self.q = np.ascontiguousarray(cfg["q"])
        self.k = np.ascontiguousarray(cfg["k"])
        ks = cfg.get("k_scale")
        self.k_scale = None if ks is None else np.ascontiguousarray(ks, dtype=np.float32)
        self.w = np.ascontiguousarray(cfg["w"], dtype=np.float32)
        off = cfg.get("k_row_offset")
        self.off = None if off is None else np.ascontiguousarray(off, dtype=np.int64)
        self.vis = np.ascontiguousarray(cfg["vis_len"], dtype=np.int32)
        w_stride = cfg.get("w_row_stride", cfg["H"] if self.w.ndim == 2 else 0)
        self.P = Problem(_p(self.q), cfg["q_dtype"], _p(self.k), cfg["k_dtype"], _p(self.k_scale),
                         _p(self.w), w_stride, _p(self.off), _p(self.vis), cfg["n_q"], cfg["H"],
                         cfg["D"], cfg["n_k"], cfg["max_vis"], cfg["topk"])


def problem(cfg):
    return _Keep(cfg)


def visible(kp, r: int) -> int:
    """Visible key count of row r (the clamped vis_len)."""
    return lib().orc_visible(C.byref(kp.P), r)


def e4m3fn_to_double(b: int) -> float:
    return lib().orc_e4m3fn_to_double(b)


def score_row(cfg_or_keep, r: int):
    """(s, m, n) of every visible key of row r, float64."""
    kp = cfg_or_keep if isinstance(cfg_or_keep, _Keep) else _Keep(cfg_or_keep)
    v = lib().orc_visible(C.byref(kp.P), r)
    s, m, n = (np.empty(max(v, 1)) for _ in range(3))
    lib().orc_score_row(C.byref(kp.P), r, _p(s), _p(m), _p(n))
    return s[:v], m[:v], n[:v]


def topk(s, K: int, ids=None):
    s = np.ascontiguousarray(s, dtype=np.float64)
    ids = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    oi = np.empty(max(K, 1), dtype=np.int32)
    os_ = np.empty(max(K, 1))
    cnt = lib().orc_topk(_p(s), _p(ids), len(s), K, _p(oi), _p(os_))
    return oi[:K], os_[:K], cnt


def idx_score_topk_rows(cfg_or_keep, rows, want_rows: bool = False):
    """Top-K (idx, score) for the given rows; with want_rows also the full
    score / m / n rows (NaN beyond each row's visible length)."""
    kp = cfg_or_keep if isinstance(cfg_or_keep, _Keep) else _Keep(cfg_or_keep)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    K = kp.P.topk
    oi = np.empty((len(rows), K), dtype=np.int32)
    os_ = np.empty((len(rows), K))
    stride = max(int(kp.P.max_vis), 1)
    S = M = N = None
    if want_rows:
        S, M, N = (np.full((len(rows), stride), np.nan) for _ in range(3))
    lib().orc_idx_score_topk_rows(C.byref(kp.P), _p(rows), len(rows), _p(oi), _p(os_), _p(S),
                                  _p(M), _p(N), stride)
    return (oi, os_, S, M, N) if want_rows else (oi, os_)


def segment_of(token, context_len, num_segments):
    return lib().orc_segment_of(token, context_len, num_segments)


def segment_edge(s, L, S_eff):
    return lib().orc_segment_edge(s, L, S_eff)


def occupied_segment(x, L, S):
    return lib().orc_occupied_segment(x, L, S)


def witness_indices(learned, context_lens, num_segments):
    learned = np.ascontiguousarray(learned, dtype=np.int32)
    rows, tk = learned.shape
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.empty((rows, max(num_segments, 1)), dtype=np.int32)
    rc = lib().orc_witness_indices(_p(learned), rows, tk, _p(lens), num_segments, _p(out))
    return rc, out[:, :num_segments]


def kvwitness_merge(rows_arr, context_lens, num_segments, keep, max_replacements):
    """Returns (status, merged copy)."""
    a = np.array(rows_arr, dtype=np.int32, copy=True, order="C")
    rows, tk = a.shape
    lens = None if context_lens is None else np.ascontiguousarray(context_lens, dtype=np.int32)
    rc = lib().orc_kvwitness_merge(_p(a), rows, tk, _p(lens), num_segments, keep,
                                   max_replacements)
    return rc, a


def segment_coverage(cand, L, S):
    c = np.ascontiguousarray(cand, dtype=np.int32)
    return lib().orc_segment_coverage(_p(c), len(c), L, S)


def block_dot(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return lib().orc_block_dot(_p(a), _p(b), len(a))


def causal_blocks(pos, bs):
    return lib().orc_causal_blocks(pos, bs)


def block_select_query(q, k, query_pos, block_size, top_blocks, init_blocks, local_blocks,
                       width=None, want_scores=False):
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    H, D = q.shape
    n_pos = k.shape[0]
    if width is None:
        width = max(top_blocks, init_blocks + local_blocks, 1)
    out = np.empty((H, width), dtype=np.int32)
    cnt = np.empty(H, dtype=np.int32)
    nb = causal_blocks(query_pos, block_size)
    nb = min(nb, -(-n_pos // block_size) if block_size > 0 else 0)
    sc = np.full((H, max(nb, 1)), np.nan, dtype=np.float32) if want_scores else None
    rc = lib().orc_block_select_query(_p(q), _p(k), query_pos, H, D, n_pos, block_size,
                                      top_blocks, init_blocks, local_blocks, _p(out), width,
                                      _p(cnt), _p(sc))
    if rc != 0:
        raise ValueError("width too small for the selection")
    lists = [list(out[h, :cnt[h]]) for h in range(H)]
    return (lists, out, cnt, sc) if want_scores else (lists, out, cnt)


def block_select_rows(cfg, rows):
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    q = np.ascontiguousarray(cfg["q"], dtype=np.float32)
    k = np.ascontiguousarray(cfg["k"], dtype=np.float32)
    pos = np.ascontiguousarray(cfg["query_pos"], dtype=np.int64)
    H, D, width = cfg["H"], cfg["D"], cfg["out_width"]
    out = np.empty((len(rows), H, width), dtype=np.int32)
    cnt = np.empty((len(rows), H), dtype=np.int32)
    lib().orc_block_select_rows(_p(q), _p(k), _p(pos), _p(rows), len(rows), H, D, cfg["n_pos"],
                                cfg["block_size"], cfg["top_blocks"], cfg["init_blocks"],
                                cfg["local_blocks"], _p(out), width, _p(cnt))
    return out, cnt


def positions_of_blocks(blocks, query_pos, n_pos, block_size):
    b = np.ascontiguousarray(blocks, dtype=np.int32)
    out = np.empty(max(len(b) * block_size, 1), dtype=np.int64)
    n = lib().orc_positions_of_blocks(_p(b), len(b), query_pos, n_pos, block_size, _p(out))
    return list(out[:n])


def positions_of_block_rows(blocks, query_pos, n_pos, block_size, out_width):
    """blocks [n_q, n_heads, width] i32 -> (positions [n_q, n_heads, out_width] i32 with -1
    after the covered ones, counts [n_q, n_heads] i32)."""
    b = np.ascontiguousarray(blocks, dtype=np.int32)
    n_q, n_heads, width = b.shape
    qp = np.ascontiguousarray(query_pos, dtype=np.int64)
    out = np.empty((n_q, n_heads, out_width), dtype=np.int32)
    cnt = np.empty((n_q, n_heads), dtype=np.int32)
    lib().orc_positions_of_block_rows(_p(b), n_q, n_heads, width, _p(qp), n_pos, block_size,
                                      _p(out), out_width, _p(cnt))
    return out, cnt


def gather_slots(idx, lens, *, row_start=None, page_table=None, page_size=0):
    """idx [rows, width] i32 row-relative entries -> KV slots [rows, width] i64 (-1: none)."""
    x = np.ascontiguousarray(idx, dtype=np.int32)
    rows, width = x.shape
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    rs = None if row_start is None else np.ascontiguousarray(row_start, dtype=np.int64)
    pt = None if page_table is None else np.ascontiguousarray(page_table, dtype=np.int32)
    ppr = 0 if pt is None else pt.shape[1]
    out = np.empty((rows, width), dtype=np.int64)
    lib().orc_gather_slots(_p(x), rows, width, _p(ln), _p(rs), _p(pt), ppr, page_size, _p(out))
    return out


def dosa_params(n_seeds, n_rep_queries=4, rep_topk=2048, kept_heads=16, neg_active_frac=0.5,
                survivor_capacity=-1):
    return DosaParams(n_seeds, n_rep_queries, rep_topk, kept_heads, neg_active_frac,
                      survivor_capacity)


def dosa_common_prefix(kp):
    return lib().orc_dosa_common_prefix(C.byref(kp.P))


def dosa_rep_row(i, R, n_q):
    return lib().orc_dosa_rep_row(i, R, n_q)


def dosa_seeds(kp, dp):
    c = dosa_common_prefix(kp)
    seeds = np.empty(max(dp.n_seeds, 1), dtype=np.int32)
    counts = np.empty(max(c, 1), dtype=np.int32)
    rc = lib().orc_dosa_seeds(C.byref(kp.P), C.byref(dp), _p(seeds), _p(counts))
    return rc, seeds[:dp.n_seeds], counts[:c]


def dosa_row(kp, dp, seeds, r, diag=False):
    K, H, D = kp.P.topk, kp.P.H, kp.P.D
    seeds = None if seeds is None else np.ascontiguousarray(seeds, dtype=np.int32)
    oi = np.empty(K, dtype=np.int32)
    os_ = np.empty(K)
    st = DosaRowStats()
    dg = None
    arrays = {}
    if diag:
        v = lib().orc_visible(C.byref(kp.P), r)
        arrays = dict(head_role=np.empty(H, np.int32), anchor=np.empty(H, np.int32),
                      beta=np.empty(H), dnorm=np.empty(H), wfold=np.empty(H), act=np.empty(H),
                      a_agg=np.empty(D), pos_part=np.empty(max(v, 1)),
                      neg_part=np.empty(max(v, 1)), U=np.empty(max(v, 1)))
        dg = DosaDiag(*[_p(arrays[n]) for n, _ in DosaDiag._fields_])
    lib().orc_dosa_row(C.byref(kp.P), C.byref(dp), _p(seeds), r, _p(oi), _p(os_), C.byref(st),
                       C.byref(dg) if dg is not None else None)
    return oi, os_, st, arrays


def dosa_rows(kp, dp, seeds, rows):
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    seeds = np.ascontiguousarray(seeds, dtype=np.int32)
    K = kp.P.topk
    oi = np.empty((len(rows), K), dtype=np.int32)
    os_ = np.empty((len(rows), K))
    st = (DosaRowStats * max(len(rows), 1))()
    lib().orc_dosa_rows(C.byref(kp.P), C.byref(dp), _p(seeds), _p(rows), len(rows), _p(oi),
                        _p(os_), st)
    return oi, os_, list(st)[:len(rows)]


def dosa_head_dots(n_seeds, n_scanned, filter_dots_per_key, n_survivors, H):
    return lib().orc_dosa_head_dots(n_seeds, n_scanned, filter_dots_per_key, n_survivors, H)


def num_threads():
    return lib().orc_num_threads()
