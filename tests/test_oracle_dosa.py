"""Pins of the oracle's DoSA certified prune.

The plain definition of what DoSA returns is the unpruned top-K, so the
step-by-step oracle is pinned to (a) the worked numbers of the DoSA notes
(threshold, single-anchor residual bound, negative aggregation, dot count),
(b) bound soundness U >= s on every scanned key, and (c) equality with the
unpruned top-K on random, structured and integer-valued (tie-heavy) inputs,
including forced survivor-capacity fallbacks."""
import json
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD, "dosa_pins.json")))


def _cfg(q, k, w, vis, topk):
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    return dict(q=q, q_dtype=0, k=k, k_dtype=0, k_scale=None, w=np.asarray(w, np.float32),
                k_row_offset=None, vis_len=np.asarray(vis, np.int32), n_q=q.shape[0],
                H=q.shape[1], D=q.shape[2], n_k=k.shape[0], max_vis=k.shape[0], topk=topk)


def test_threshold_and_negative_aggregate_example(orc):
    """Sections 2 and 3.2 in one row.  Head 0 is kept (q=(0,1), w=3); heads 1, 2
    are the page's omitted negative heads q1=(1,0), q2=(0,1), w=-1.  Seeds are
    built to score 9, 6, 2, so K=2 gives tau=6.  Key (3,4): positive bound 12,
    aggregate deduction 7 (exact), U=5 < 6 -> pruned.  Key (3,-2): aggregate 1
    against a true deduction of 3.  Key (0,3): U = 6 = tau -> kept and tied
    with the seed scoring 6; the lower id wins."""
    th, ng = G["threshold"], G["negative_aggregate"]
    seeds_k = [[1.0, 5.0], [1.0, 3.5], [1.0, 1.5]]
    keys = seeds_k + [ng["k1"], ng["k2"], [0.0, 3.0], [-1.0, 2.8]]
    q = [[[0.0, 1.0], ng["q"][0], ng["q"][1]]]
    w = [[3.0] + ng["w"]]
    cfg = _cfg(q, keys, w, [len(keys)], th["K"])
    kp = orc.problem(cfg)
    dp = orc.dosa_params(n_seeds=3, n_rep_queries=1, rep_topk=3, kept_heads=1)
    seeds = np.array([0, 1, 2], np.int32)
    idx, sc, st, dg = orc.dosa_row(kp, dp, seeds, 0, diag=True)
    s_full, _, _ = orc.score_row(cfg, 0)
    assert list(s_full[:3]) == th["seed_scores"]
    assert st.tau == th["tau"]
    assert dg["head_role"].tolist() == [1, 3, 3]
    np.testing.assert_array_equal(dg["a_agg"], ng["a_A"])
    # key 3 = (3,4)
    assert dg["pos_part"][3] == ng["pos_bound"]
    assert dg["neg_part"][3] == ng["agg1"] == ng["true1"]
    assert dg["pos_part"][3] - dg["neg_part"][3] == ng["U1"]
    assert dg["U"][3] < ng["tau"]
    # key 4 = (3,-2)
    assert dg["neg_part"][4] == ng["agg2"]
    true2 = sum(max(0.0, np.dot(qh, ng["k2"])) for qh in ng["q"])
    assert true2 == ng["true2"]
    # key 5 = (0,3): U = 6 -> kept; ties the seed (1, 3.5) scoring 6
    assert dg["pos_part"][5] - dg["neg_part"][5] == th["kept_U"]
    assert dg["U"][5] >= st.tau
    assert s_full[5] == 6.0
    assert idx.tolist() == [0, 1]  # 9 (id 0), then the 6-tie goes to id 1 < 5
    # key 6 = (-1, 2.8): the aggregate is loose (U = 8.4 - 1.8 = 6.6 >= tau) but
    # its exact score 5.6 < tau, so rescoring drops it
    assert dg["U"][6] >= st.tau and s_full[6] < st.tau
    assert st.n_survivors == 2 and st.n_kept_survivors == 1


def test_bound_equal_to_tau_is_kept(orc):
    """Section 2: a key whose bound equals tau must be kept.  A zero key has
    U = 0 exactly (no margin: its norm is 0); seeds make tau = 0; the zero
    key (id 0) then ties at 0 and, being the lowest id, enters the top-K."""
    keys = [[0.0, 0.0], [3.0, 0.0], [-1.0, 0.0], [-2.0, 0.0]]
    cfg = _cfg([[[1.0, 0.0]]], keys, [[1.0]], [4], 2)
    kp = orc.problem(cfg)
    dp = orc.dosa_params(n_seeds=3, n_rep_queries=1, rep_topk=2, kept_heads=1)
    idx, sc, st, dg = orc.dosa_row(kp, dp, np.array([1, 2, 3], np.int32), 0, diag=True)
    assert st.tau == 0.0 and dg["U"][0] == 0.0
    assert idx.tolist() == [1, 0]


def test_anchor_projection_is_clamped(orc):
    """Section 3.1 requires beta >= 0.  Reading taken for the planner: beta is
    the projection coefficient clamped at 0, so a head pointing away from
    every kept head gets beta = 0 and its whole norm as the residual."""
    keys = [[1.0, 1.0], [2.0, 1.0], [1.0, 2.0], [3.0, 4.0]]
    cfg = _cfg([[[1.0, 0.0], [-2.0, 1.0]]], keys, [[100.0, 2.0]], [4], 2)
    kp = orc.problem(cfg)
    dp = orc.dosa_params(n_seeds=3, n_rep_queries=1, rep_topk=2, kept_heads=1)
    idx, sc, st, dg = orc.dosa_row(kp, dp, np.array([0, 1, 2], np.int32), 0, diag=True)
    assert dg["anchor"][1] == 0 and dg["beta"][1] == 0.0
    assert dg["dnorm"][1] == np.sqrt(5.0)


def test_residual_bound_example(orc):
    """Section 3.1: kept q_j=(1,0), omitted positive q_h=(2,1) with w=2:
    beta=2, d=(0,1); for k=(3,4) the bound is 11 against a true 10, and the
    weighted bound 22 against 20."""
    g = G["residual_bound"]
    w_j = 100.0  # large enough that head j is the kept one
    seeds_k = [[1.0, 1.0], [2.0, 1.0], [1.0, 2.0]]
    keys = seeds_k + [g["k"]]
    cfg = _cfg([[g["q_j"], g["q_h"]]], keys, [[w_j, g["w_h"]]], [4], 2)
    kp = orc.problem(cfg)
    dp = orc.dosa_params(n_seeds=3, n_rep_queries=1, rep_topk=3, kept_heads=1)
    idx, sc, st, dg = orc.dosa_row(kp, dp, np.array([0, 1, 2], np.int32), 0, diag=True)
    assert dg["head_role"].tolist() == [1, 2]
    assert dg["anchor"][1] == 0
    assert dg["beta"][1] == g["beta"] and dg["dnorm"][1] == g["dnorm"]
    x_j = float(np.dot(g["q_j"], g["k"]))
    head_bound = (dg["pos_part"][3] - w_j * max(x_j, 0.0)) / g["w_h"]
    assert head_bound == g["bound"]
    assert g["w_h"] * head_bound == g["weighted_bound"]
    assert max(0.0, float(np.dot(g["q_h"], g["k"]))) == g["true"]


def test_cost_model_counter(orc):
    g = G["cost_model"]
    assert g["keys"] * g["H"] == g["dense"]
    assert orc.dosa_head_dots(0, g["keys"], g["filter"], g["survivors"], g["H"]) == g["pruned"]


def _assert_equals_unpruned(orc, cfg, rows, dp, seeds=None, expect_prune=False):
    kp = orc.problem(cfg)
    if seeds is None:
        rc, seeds, counts = orc.dosa_seeds(kp, dp)
        assert rc == orc.OK
    c = orc.dosa_common_prefix(kp)
    assert len(set(seeds.tolist())) == dp.n_seeds
    assert np.all(np.diff(seeds) > 0) and seeds[0] >= 0 and seeds[-1] < c
    ref_i, ref_s = orc.idx_score_topk_rows(kp, rows)
    pruned = 0
    for n, r in enumerate(rows):
        idx, sc, st, dg = orc.dosa_row(kp, dp, seeds, r, diag=True)
        np.testing.assert_array_equal(idx, ref_i[n])
        np.testing.assert_array_equal(sc, ref_s[n])
        s, _, _ = orc.score_row(kp, r)
        scanned = ~np.isnan(dg["U"][:len(s)])
        assert np.all(dg["U"][:len(s)][scanned] >= s[scanned]), "unsound bound"
        assert st.n_scanned == scanned.sum() == len(s) - dp.n_seeds
        pruned += st.n_scanned - st.n_survivors
    if expect_prune:
        assert pruned > 0
    return pruned


def test_equals_unpruned_random(orc):
    cfg = synth.dosa(seed=1, n_q=24, L=300, H=8, D=16, topk=20, n_seeds=60, n_rep=4,
                     rep_topk=20, kept_heads=4)
    dp = orc.dosa_params(**{k: cfg["dosa"][k] for k in ("n_seeds", "n_rep_queries", "rep_topk",
                                                         "kept_heads", "neg_active_frac")})
    _assert_equals_unpruned(orc, cfg, list(range(24)), dp)


def test_equals_unpruned_structured_prunes(orc):
    cfg = synth.dosa_structured(seed=2, n_q=16, L=400, H=8, D=16, topk=16, n_seeds=64,
                                n_rep=4, rep_topk=16, kept_heads=4)
    dp = orc.dosa_params(64, 4, 16, 4, 0.5)
    _assert_equals_unpruned(orc, cfg, list(range(16)), dp, expect_prune=True)


def test_equals_unpruned_integer_ties(orc):
    """Integer-valued queries/keys and dyadic weights: scores are exact and tie
    often, including exactly at tau; the result must still equal the unpruned
    top-K id for id."""
    rng = np.random.default_rng(11)
    for trial in range(30):
        n_q, L, H, D, K = 6, 80, 6, 4, 8
        q = rng.integers(-2, 3, (n_q, H, D)).astype(np.float32)
        k = rng.integers(-2, 3, (L, D)).astype(np.float32)
        w = rng.choice([-1.0, -0.5, 0.5, 1.0, 2.0], (n_q, H)).astype(np.float32)
        vis = L - n_q + 1 + np.arange(n_q)
        cfg = _cfg(q, k, w, vis, K)
        dp = orc.dosa_params(n_seeds=int(rng.integers(K, 40)), n_rep_queries=3, rep_topk=K,
                             kept_heads=int(rng.integers(0, H + 1)), neg_active_frac=0.5)
        _assert_equals_unpruned(orc, cfg, list(range(n_q)), dp)


def test_capacity_overflow_falls_back_exactly(orc):
    cfg = synth.dosa(seed=3, n_q=8, L=200, H=8, D=16, topk=16, n_seeds=40, n_rep=4,
                     rep_topk=16, kept_heads=2)
    kp = orc.problem(cfg)
    dp = orc.dosa_params(40, 4, 16, 2, 0.5, survivor_capacity=0)
    rc, seeds, _ = orc.dosa_seeds(kp, dp)
    ref_i, ref_s = orc.idx_score_topk_rows(kp, list(range(8)))
    fell = 0
    for r in range(8):
        idx, sc, st, _ = orc.dosa_row(kp, dp, seeds, r)
        np.testing.assert_array_equal(idx, ref_i[r])
        fell += st.fallback
    assert fell > 0


def test_seed_rule(orc):
    """Cold prior: representative rows are evenly spaced with both ends; seeds
    lie in the common visible prefix, and every key counted by a
    representative list is a seed when the union fits."""
    assert [orc.dosa_rep_row(i, 4, 4096) for i in range(4)] == [0, 1365, 2730, 4095]
    cfg = synth.dosa(seed=4, n_q=12, L=150, H=4, D=8, topk=8, n_seeds=40, n_rep=4, rep_topk=8)
    kp = orc.problem(cfg)
    dp = orc.dosa_params(40, 4, 8, 2, 0.5)
    rc, seeds, counts = orc.dosa_seeds(kp, dp)
    assert rc == orc.OK
    c = orc.dosa_common_prefix(kp)
    assert c == 150 - 12 + 1
    assert set(np.nonzero(counts)[0].tolist()) <= set(seeds.tolist())
    assert counts.sum() == 4 * 8
    # too few common keys -> refused, rows fall back to the exact path
    bad = orc.dosa_params(c + 1, 4, 8, 2, 0.5)
    assert orc.dosa_seeds(kp, bad)[0] == orc.NOT_ENOUGH_KEYS
