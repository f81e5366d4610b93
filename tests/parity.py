"""Comparison rules between the HIP path and the oracle.

Scores: |s_gpu - s_ref| <= 1e-3 * m_ref + 2^-16 * n_ref, where
m = sum_h |w_h| max(0, x_h) and n = sum_h |w_h| |q_h| |k|.  This is the
relative 1e-3 rule of fp32 accumulation made well defined for a signed sum
(a plain relative error is meaningless when cancellation drives s to ~0); it
is the plain relative rule when all weights share a sign.  The 2^-16 * n
term covers fp32 accumulation of D = 128 exact bf16 products
(gamma_128 ~ 2^-17).

Top-K sets: equal, except ids whose oracle score lies within that
tolerance of the oracle's K-th score.  GPU rows must be sorted by their own
scores under (score desc, id asc), distinct, in range and -1 / -inf padded.
"""
import numpy as np

RTOL = 1e-3
NTOL = 2.0 ** -16


def tol(m, n):
    return RTOL * m + NTOL * n


def check_topk_row(gi, gs, s_ref, m_ref, n_ref, K, where=""):
    """gi/gs: GPU ids/scores of one row (gs may be None); s/m/n_ref: oracle
    arrays over the row's visible keys."""
    v = len(s_ref)
    cnt = min(K, v)
    gi = np.asarray(gi)
    assert np.all(gi[cnt:] == -1), f"{where}: padding ids"
    sel = gi[:cnt]
    assert np.all((sel >= 0) & (sel < v)), f"{where}: id out of range"
    assert len(np.unique(sel)) == cnt, f"{where}: duplicate ids"
    if gs is not None:
        gs = np.asarray(gs, dtype=np.float64)
        assert np.all(np.isneginf(gs[cnt:])), f"{where}: padding scores"
        err = np.abs(gs[:cnt] - s_ref[sel])
        bound = tol(m_ref[sel], n_ref[sel])
        bad = np.nonzero(err > bound)[0]
        assert len(bad) == 0, (f"{where}: score mismatch at slots {bad[:5]}: gpu {gs[bad[:5]]} "
                               f"ref {s_ref[sel][bad[:5]]}")
        keys = list(zip(-gs[:cnt], sel))
        assert all(a <= b for a, b in zip(keys, keys[1:])), f"{where}: not (score desc, id asc)"
    if v <= K:
        assert set(sel.tolist()) == set(range(v)), f"{where}: must hold every visible key"
        return 0
    order = np.lexsort((np.arange(v), -s_ref))
    ref_sel = order[:K]
    sK = s_ref[ref_sel[-1]]
    iK = ref_sel[-1]
    diff = set(sel.tolist()) ^ set(ref_sel.tolist())
    for i in diff:
        t = max(tol(m_ref[i], n_ref[i]), tol(m_ref[iK], n_ref[iK]))
        assert abs(s_ref[i] - sK) <= t, (f"{where}: id {i} (ref {s_ref[i]}) differs and is not "
                                         f"within tolerance of the K-th score {sK}")
    return len(diff)


def check_topk_rows(gi, gs, oi, S, M, N, vis, K, where=""):
    """Many rows at once: gi/gs the GPU's ids/scores [R, K] (gs may be None),
    oi the oracle's ids [R, K], S/M/N the oracle's score / m / n rows [R, >=
    max vis], vis the rows' visible lengths.  Rows whose id set equals the
    oracle's need only the score and order checks; the others go through
    check_topk_row's near-K-th rule.  Returns the number of rows whose id set
    differs from the oracle's."""
    gi = np.asarray(gi)
    oi = np.asarray(oi)
    vis = np.asarray(vis, dtype=np.int64)
    R = gi.shape[0]
    cnt = np.minimum(vis, K)
    slot = np.arange(K)[None, :]
    valid = slot < cnt[:, None]
    assert np.all(gi[~valid] == -1), f"{where}: padding ids"
    assert np.all(gi[valid] >= 0) and np.all((gi < vis[:, None])[valid]), f"{where}: id range"
    srt = np.sort(np.where(valid, gi, np.iinfo(np.int32).max).astype(np.int64), axis=1)
    dup = (srt[:, 1:] == srt[:, :-1]) & valid[:, 1:]
    assert not dup.any(), f"{where}: duplicate ids in rows {np.nonzero(dup.any(1))[0][:5]}"
    rows = np.arange(R)[:, None]
    safe = np.where(valid, gi, 0)
    if gs is not None:
        gs = np.asarray(gs, dtype=np.float64)
        assert np.all(np.isneginf(gs[~valid])), f"{where}: padding scores"
        err = np.abs(gs - S[rows, safe])
        bound = tol(M[rows, safe], N[rows, safe])
        bad = (err > bound) & valid
        assert not bad.any(), (f"{where}: score mismatch in rows {np.nonzero(bad.any(1))[0][:5]}")
        a, b = gs[:, :-1], gs[:, 1:]
        ok = (a > b) | ((a == b) & (gi[:, :-1] < gi[:, 1:]))
        pair = valid[:, 1:]
        assert np.all(ok[pair]), f"{where}: rows {np.nonzero((~ok & pair).any(1))[0][:5]} " \
                                 "not in (score desc, id asc) order"
    osrt = np.sort(np.where(valid, oi, np.iinfo(np.int32).max).astype(np.int64), axis=1)
    differ = np.nonzero(np.any(srt != osrt, axis=1))[0]
    for r in differ:
        v = int(vis[r])
        check_topk_row(gi[r], None, S[r, :v], M[r, :v], N[r, :v], K, where=f"{where} row {r}")
    return len(differ)


def oracle_check_rows(orc, cfg, gi, gs, rows=None, chunk=1024, where=""):
    """Every listed row (default: all) of a GPU top-K against the oracle, in
    chunks of rows so that the oracle's score rows stay bounded in memory.
    Returns the number of rows whose id set differs from the oracle's (each
    difference within the near-K-th tolerance)."""
    kp = orc.problem(cfg)
    rows = np.arange(cfg["n_q"]) if rows is None else np.asarray(rows)
    ndiff = 0
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        oi, _, S, M, N = orc.idx_score_topk_rows(kp, rr, want_rows=True)
        vis = np.array([orc.visible(kp, int(r)) for r in rr], dtype=np.int64)
        ndiff += check_topk_rows(gi[rr], None if gs is None else gs[rr], oi, S, M, N, vis,
                                 cfg["topk"], where=where)
    return ndiff
