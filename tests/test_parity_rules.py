"""The many-row parity checker used by the full-size GPU tests, exercised on
the CPU: the oracle's own rows pass, and planted mistakes in the rows under
test (a dropped id, a duplicate, a wrong score, a swapped order, bad padding)
are caught."""
import numpy as np
import pytest

import synth
from parity import check_topk_rows


@pytest.fixture(scope="module")
def case(orc):
    cfg = synth.prefill(seed=3, n_q=40, L=300, H=8, D=32, topk=64)
    kp = orc.problem(cfg)
    rows = np.arange(cfg["n_q"])
    oi, os_, S, M, N = orc.idx_score_topk_rows(kp, rows, want_rows=True)
    vis = np.array([orc.visible(kp, int(r)) for r in rows])
    return cfg, oi, os_.astype(np.float32), S, M, N, vis


def test_oracle_rows_pass(case):
    cfg, oi, os_, S, M, N, vis = case
    assert check_topk_rows(oi, os_, oi, S, M, N, vis, cfg["topk"]) == 0


@pytest.mark.parametrize("mistake", ["drop", "dup", "score", "swap", "pad_id", "pad_score",
                                     "range"])
def test_planted_mistakes_fail(case, mistake):
    cfg, oi, os_, S, M, N, vis = case
    gi, gs = oi.copy(), os_.copy()
    r = 30  # vis 291 > K: a selecting row
    K = cfg["topk"]
    if mistake == "drop":      # the best id replaced by a poor one outside the set
        out = np.setdiff1d(np.arange(vis[r]), gi[r])
        worst = out[np.argmin(S[r, out])]
        gi[r, 0], gs[r, 0] = worst, np.float32(S[r, worst])
        gi[r], gs[r] = gi[r][np.lexsort((gi[r], -gs[r]))], np.sort(gs[r])[::-1]
    elif mistake == "dup":
        gi[r, 5] = gi[r, 4]
    elif mistake == "score":
        gs[r, 3] += np.float32(0.05) * (abs(gs[r, 3]) + 1)
    elif mistake == "swap":
        gi[r, [2, 3]] = gi[r, [3, 2]]
        gs[r, [2, 3]] = gs[r, [3, 2]]
    elif mistake == "pad_id":   # a padding id inside the selected slots
        gi[r, 0] = -1
    elif mistake == "pad_score":
        gi[r, K - 1] = -1
    elif mistake == "range":
        gi[r, 10] = vis[r] + 3
    with pytest.raises(AssertionError):
        check_topk_rows(gi, gs, oi, S, M, N, vis, K)
