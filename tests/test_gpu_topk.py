"""GPU top-K stage (rows_topk) on given f32 score rows: ids and scores must
equal the oracle's (score desc, id asc) top-K exactly - the scores are
inputs, so there is no tolerance."""
import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


def _rows(kind, rng, n_rows, L):
    if kind == "normal":
        return rng.standard_normal((n_rows, L)).astype(np.float32) * 30
    if kind == "equal":
        return np.full((n_rows, L), 3.5, np.float32)
    if kind == "few_values":
        return rng.integers(-3, 4, (n_rows, L)).astype(np.float32)
    if kind == "narrow":  # thousands of items share the top 11 key bits
        return (100.0 + rng.random((n_rows, L)) * 0.01).astype(np.float32)
    if kind == "signed_zero":
        x = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), (n_rows, L))
        return x.astype(np.float32)
    if kind == "wide":
        return (rng.standard_normal((n_rows, L)) *
                np.exp(rng.uniform(-20, 20, (n_rows, L)))).astype(np.float32)
    if kind == "nan_inf":  # non-finite scores mixed into a normal row
        x = rng.standard_normal((n_rows, L)).astype(np.float32)
        m = rng.random((n_rows, L))
        x[m < 0.01] = np.nan
        x[(m >= 0.01) & (m < 0.015)] = np.inf
        x[(m >= 0.015) & (m < 0.02)] = -np.inf
        return x
    if kind == "bits":  # arbitrary 32-bit patterns: NaNs, infinities, subnormals
        return rng.integers(0, 2**32, (n_rows, L), dtype=np.uint64).astype(np.uint32).view(np.float32)
    raise ValueError(kind)


def _check(orc, scores, vis, K):
    import sparse_attention_indexer_02_amd as si
    st = torch.from_numpy(scores).cuda()
    vt = torch.from_numpy(vis.astype(np.int32)).cuda()
    gi, gs = si.rows_topk(st, vt, K)
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    for r in range(scores.shape[0]):
        v = int(min(max(vis[r], 0), scores.shape[1]))
        # a NaN score ranks as -inf (its order is otherwise unspecified)
        row = np.where(np.isnan(scores[r, :v]), -np.inf, scores[r, :v]).astype(np.float64)
        oi, os_, _ = orc.topk(row, K)
        np.testing.assert_array_equal(gi[r], oi, err_msg=f"row {r} n={v} K={K}")
        np.testing.assert_array_equal(gs[r].astype(np.float64), os_, err_msg=f"row {r}")


@pytest.mark.parametrize("kind", ["normal", "equal", "few_values", "narrow", "signed_zero", "wide",
                                  "nan_inf", "bits"])
@pytest.mark.parametrize("L,K", [(8192, 2048), (5000, 2048), (3000, 100), (8192, 1), (700, 513)])
def test_short_rows(orc, kind, L, K):
    rng = np.random.default_rng(L + K)
    n_rows = 24
    scores = _rows(kind, rng, n_rows, L)
    vis = rng.integers(0, L + 1, n_rows)
    vis[:4] = [0, 1, min(K, L), L]
    say(f"topk {kind} L={L} K={K}")
    _check(orc, scores, vis, K)


@pytest.mark.parametrize("kind", ["normal", "few_values", "nan_inf", "bits"])
def test_long_rows(orc, kind):
    """Rows longer than the register-resident path (up to 40000); K = 4096
    takes the radix-select kernel."""
    rng = np.random.default_rng(3)
    scores = _rows(kind, rng, 6, 40000)
    vis = np.array([40000, 8193, 12288, 20000, 2, 0])
    say(f"topk long {kind}")
    _check(orc, scores, vis, 2048)
    _check(orc, scores, vis, 4096)


@pytest.mark.parametrize("kind", ["equal", "signed_zero", "narrow", "nan_inf", "bits"])
@pytest.mark.parametrize("K", [1, 100, 2048])
def test_deep_rows(orc, kind, K):
    """Rows with three chunk levels (140000 scores: 18 chunks, then 5, then
    2, then the last pass), ties spanning chunks and levels: chunk passes
    keep their sets in position order, so the index tie-break must come out
    exact at the last level."""
    rng = np.random.default_rng(K + 7)
    L = 140000
    scores = _rows(kind, rng, 4, L)
    vis = np.array([L, 8192 * 3 + 5, 16385, 9000])
    say(f"topk deep {kind} K={K}")
    _check(orc, scores, vis, K)


@pytest.mark.parametrize("kind", ["normal", "signed_zero", "nan_inf", "bits"])
@pytest.mark.parametrize("L,K", [(5000, 3000), (700, 4096), (8192, 2049)])
def test_short_rows_large_k(orc, kind, L, K):
    """K above the block kernel's 2048 on rows of at most 8192 scores: the
    radix-select kernel with the row staged in LDS, including rows shorter
    than K and non-finite scores (NaN ranks and is reported as -inf)."""
    rng = np.random.default_rng(L + 3 * K)
    scores = _rows(kind, rng, 12, L)
    vis = rng.integers(0, L + 1, 12)
    vis[:4] = [0, 1, min(K, L), L]
    say(f"topk large K {kind} L={L} K={K}")
    _check(orc, scores, vis, K)
