"""Pins of the oracle's indexer score, element decoding and top-K.

Each check is anchored outside the oracle: a worked example printed on the
DoSA notes page, a library routine for a special case, or a property that
fully characterises the result.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(q, k, w, vis, q_dtype=0, k_dtype=0, k_scale=None, topk=4, k_row_offset=None):
    q = np.asarray(q)
    n_q, H, D = q.shape
    return dict(q=q, q_dtype=q_dtype, k=np.asarray(k), k_dtype=k_dtype, k_scale=k_scale,
                w=np.asarray(w, dtype=np.float32), k_row_offset=k_row_offset,
                vis_len=np.asarray(vis, dtype=np.int32), n_q=n_q, H=H, D=D,
                n_k=np.asarray(k).shape[0], max_vis=np.asarray(k).shape[0], topk=topk)


def test_score_worked_example(orc):
    """DoSA notes section 3: activations 4, 3 with weights 2, -1 -> 5; a negative
    dot is clipped to 0 before its (negative) weight, so it deducts nothing."""
    g = json.load(open(os.path.join(GOLD, "dosa_pins.json")))["score_example"]
    # D=1 queries holding the activations directly, key = [1].
    q = np.array([[[a] for a in g["activations"]]], dtype=np.float32)
    cfg = _cfg(q, np.array([[1.0]], np.float32), [g["weights"]], [1])
    s, m, n = orc.score_row(cfg, 0)
    assert s[0] == g["expected"]
    nd = g["negative_dot"]
    q2 = np.array([[[a] for a in nd["activations"]]], dtype=np.float32)
    s2, _, _ = orc.score_row(_cfg(q2, np.array([[1.0]], np.float32), [nd["weights"]], [1]), 0)
    assert s2[0] == nd["expected"]


def test_score_unit_keys_pick_one_coordinate(orc):
    """Special case: key e_d gives x_h = q[h, d] exactly, so the score is
    sum_h w_h max(0, q[h, d]) -- checks the operand orientation (q rows are
    heads, the contraction runs over d) and the per-row weights."""
    rng = np.random.default_rng(1)
    n_q, H, D = 3, 5, 7
    q = rng.standard_normal((n_q, H, D)).astype(np.float32)
    w = rng.uniform(-1, 1, (n_q, H)).astype(np.float32)
    k = np.eye(D, dtype=np.float32)
    cfg = _cfg(q, k, w, [D] * n_q)
    for r in range(n_q):
        s, m, n = orc.score_row(cfg, r)
        want = (w[r][:, None].astype(np.float64) * np.maximum(q[r].astype(np.float64), 0)).sum(0)
        np.testing.assert_allclose(s, want, rtol=0, atol=1e-12)
        assert np.all(m >= np.abs(s) - 1e-12)
        assert np.all(n >= m - 1e-12)  # Cauchy-Schwarz on every head


def test_tolerance_scales_by_value(orc):
    """The tolerance scales m = sum_h |w_h| max(0, x_h) and n = sum_h |w_h|
    |q_h| |k| of the parity rule, pinned by value on hand-worked integer
    cases (the score itself is the one of the DoSA notes, section 3).
    Heads q_0 = (3, 4) with |q_0| = 5 and q_1 = (-6, 8) with |q_1| = 10,
    weights 2 and -1/2, so sum_h |w_h| |q_h| = 2*5 + 5 = 15:
      k = (1, 0):  x = (3, -6)    s = 6     m = 6             n = 15
      k = (0, 2):  x = (8, 16)    s = 16-8  m = 16+8 = 24     n = 15*2 = 30
      k = (3, -4): x = (-7, -50)  s = 0     m = 0             n = 15*5 = 75
      k = (-3, 4): x = (7, 50)    s = 14-25 m = 14+25 = 39    n = 75
    A signed weight in m (m = -11 on the last key), a dropped |w_h| in n
    (n = 10 - 5 = 5 on the first), 1-norms of q (n = 2*7 + 14/2 = 21) or of
    k (n = 15*7 = 105 on the third) all miss these values."""
    q = np.array([[[3.0, 4.0], [-6.0, 8.0]]], np.float32)
    k = np.array([[1.0, 0.0], [0.0, 2.0], [3.0, -4.0], [-3.0, 4.0]], np.float32)
    cfg = _cfg(q, k, [[2.0, -0.5]], [4])
    s, m, n = orc.score_row(cfg, 0)
    assert list(s) == [6.0, 8.0, 0.0, -11.0]
    assert list(m) == [6.0, 24.0, 0.0, 39.0]
    assert list(n) == [15.0, 30.0, 75.0, 75.0]


def test_tolerance_scales_fp8_key_carries_its_scale(orc):
    """n takes the norm of the dequantised key: e4m3fn bytes 0x44 = 3 and
    0x48 = 4 with per-token scale 2 give k = (6, 8), |k| = 10.  With the heads
    and weights above: x = (18 + 32, -36 + 64) = (50, 28), s = 100 - 14 = 86,
    m = 100 + 14 = 114, n = 15 * 10 = 150 (75 if the scale were left out of
    the norm)."""
    assert orc.e4m3fn_to_double(0x44) == 3.0 and orc.e4m3fn_to_double(0x48) == 4.0
    q = synth.f32_to_bf16_bits(np.array([[[3.0, 4.0], [-6.0, 8.0]]], np.float32))
    kb = np.array([[0x44, 0x48]], np.uint8)
    cfg = _cfg(q, kb, [[2.0, -0.5]], [1], q_dtype=1, k_dtype=2,
               k_scale=np.array([2.0], np.float32))
    s, m, n = orc.score_row(cfg, 0)
    assert (s[0], m[0], n[0]) == (86.0, 114.0, 150.0)


def test_score_positive_scale_commutes_with_relu(orc):
    """fp8 keys: the per-token scale c > 0 satisfies ReLU(c x) = c ReLU(x), so
    doubling every scale doubles every score exactly."""
    rng = np.random.default_rng(2)
    q = synth.f32_to_bf16_bits(rng.standard_normal((2, 4, 16)).astype(np.float32))
    kf = rng.standard_normal((40, 16)).astype(np.float32)
    kb = synth.f32_to_e4m3fn_bytes(kf)
    sc = rng.uniform(0.5, 2.0, 40).astype(np.float32)
    w = rng.uniform(-1, 1, (2, 4)).astype(np.float32)
    a = _cfg(q, kb, w, [40, 33], q_dtype=1, k_dtype=2, k_scale=sc)
    b = _cfg(q, kb, w, [40, 33], q_dtype=1, k_dtype=2, k_scale=(2 * sc).astype(np.float32))
    for r in range(2):
        sa, _, _ = orc.score_row(a, r)
        sb, _, _ = orc.score_row(b, r)
        assert len(sa) == [40, 33][r]
        np.testing.assert_array_equal(2 * sa, sb)


def test_row_offsets_select_each_rows_keys(orc):
    """A ragged layout equals the same rows laid out as separate shared-key problems."""
    rng = np.random.default_rng(3)
    lens = [5, 1, 9]
    off = np.array([0, 5, 6], np.int64)
    k = rng.standard_normal((15, 8)).astype(np.float32)
    q = rng.standard_normal((3, 2, 8)).astype(np.float32)
    w = rng.uniform(-1, 1, (3, 2)).astype(np.float32)
    cfg = _cfg(q, k, w, lens, k_row_offset=off)
    for r in range(3):
        s, _, _ = orc.score_row(cfg, r)
        solo = _cfg(q[r:r + 1], k[off[r]:off[r] + lens[r]], w[r:r + 1], [lens[r]])
        s2, _, _ = orc.score_row(solo, 0)
        np.testing.assert_array_equal(s, s2)


def test_e4m3fn_decoding_matches_torch_and_the_spec(orc):
    """OCP e4m3fn: all 256 codes against torch's float8_e4m3fn cast (a library
    routine), plus the spec's landmarks."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    mine = np.array([orc.e4m3fn_to_double(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert orc.e4m3fn_to_double(0x7E) == 448.0
    assert orc.e4m3fn_to_double(0x01) == 2.0 ** -9
    assert orc.e4m3fn_to_double(0x38) == 1.0


def test_bf16_storage_roundtrip(orc):
    """bf16 inputs decode exactly: 1.0 = 0x3F80, -2.5 = 0xC020."""
    q = np.array([[[0x3F80, 0xC020]]], dtype=np.uint16)
    k = np.array([[1.0, 0.0], [0.0, 1.0]], dtype=np.float32)
    cfg = _cfg(q, k, [[1.0]], [2], q_dtype=1)
    s, _, _ = orc.score_row(cfg, 0)
    assert list(s) == [1.0, 0.0]  # the -2.5 activation is clipped


def _check_topk(orc, s, K, ids=None):
    idx, sc, cnt = orc.topk(s, K, ids)
    n = len(s)
    ids_arr = np.arange(n) if ids is None else np.asarray(ids)
    assert cnt == min(K, n)
    sel = idx[:cnt]
    assert len(set(sel.tolist())) == cnt
    assert np.all(idx[cnt:] == -1) and np.all(np.isneginf(sc[cnt:]))
    pos = {int(i): p for p, i in enumerate(ids_arr)}
    key = [(-s[pos[int(i)]], int(i)) for i in sel]
    assert key == sorted(key), "not in (score desc, id asc) order"
    np.testing.assert_array_equal(sc[:cnt], [s[pos[int(i)]] for i in sel])
    if cnt:
        last = key[-1]
        chosen = set(sel.tolist())
        for p, i in enumerate(ids_arr):
            if int(i) not in chosen:
                assert (-s[p], int(i)) > last, "a better item was left out"


def test_topk_characterisation_with_ties(orc):
    """Top-K is fully characterised by: sorted by (score desc, id asc), distinct,
    min(K, n) entries, and no left-out item ranks before the last chosen one."""
    rng = np.random.default_rng(4)
    for trial in range(200):
        n = int(rng.integers(0, 60))
        K = int(rng.integers(1, 40))
        s = rng.integers(-3, 4, n).astype(np.float64)  # many exact ties
        ids = None
        if trial % 3 == 0:
            ids = rng.permutation(1000)[:n]
        _check_topk(orc, s, K, ids)


def test_topk_signed_zero_ties_break_by_id(orc):
    s = np.array([0.0, -0.0, 1.0, -0.0, 0.0])
    idx, _, _ = orc.topk(s, 5)
    assert list(idx) == [2, 0, 1, 3, 4]


def test_topk_threshold_example(orc):
    """DoSA notes section 2: seed scores 9, 6, 2 with K = 2 -> tau = 6."""
    g = json.load(open(os.path.join(GOLD, "dosa_pins.json")))["threshold"]
    idx, sc, _ = orc.topk(np.array(g["seed_scores"]), g["K"])
    assert sc[g["K"] - 1] == g["tau"]


def test_idx_rows_match_score_then_topk(orc):
    c = synth.prefill(n_q=20, L=70, H=8, D=32, topk=16)
    rows = [0, 5, 19]
    oi, os_, S, M, N = orc.idx_score_topk_rows(c, rows, want_rows=True)
    for i, r in enumerate(rows):
        s, m, n = orc.score_row(c, r)
        v = len(s)
        assert v == 70 - 20 + r + 1
        np.testing.assert_array_equal(S[i, :v], s)
        _check_topk(orc, s, 16)
        idx, sc, _ = orc.topk(s, 16)
        np.testing.assert_array_equal(oi[i], idx)
