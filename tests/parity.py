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
