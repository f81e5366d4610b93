"""Pins of the oracle's block-sparse selection: the ten scenarios of the
ferrox-core block_sparse.rs tests, the page's f32 dot definition, and the
selection rule's characterising properties on random geometries."""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD, "block_pins.json")))


def _keys(spec):
    if "zeros" in spec:
        k = np.zeros((spec["zeros"], 2), np.float32)
        for p, v in spec.get("set", {}).items():
            k[int(p)] = v
        return k
    if "const" in spec:
        return np.tile(np.array(spec["const"], np.float32), (spec["n"], 1))
    k = np.tile(np.array([0.0, 0.01], np.float32), (spec["n"], 1))
    for p in spec["hot"]:
        k[p] = [1.0, 0.0]
    return k


@pytest.mark.parametrize("case", G["cases"], ids=[c["cite"][:48] for c in G["cases"]])
def test_page_scenarios(orc, case):
    bs, top, init, local = case["cfg"]
    k = _keys(case["keys"])
    q = np.array(case["q"], np.float32)
    for pos in case["positions"]:
        lists, _, cnt = orc.block_select_query(q, k, pos, bs, top, init, local)
        for h, sel in enumerate(lists):
            cov = orc.positions_of_blocks(sel, pos, len(k), bs)
            if case.get("check") == "nonempty_causal":
                assert sel and cov and all(p <= pos for p in cov)
            if "contains" in case:
                assert set(case["contains"][h]) <= set(sel), (h, sel)
            if "expected" in case:
                assert sel == case["expected"][h]
            if "max_block" in case:
                assert all(b <= case["max_block"] for b in sel)
            if "covered" in case:
                assert cov == case["covered"]
            if "count" in case:
                assert len(sel) == case["count"]
        if case.get("heads_differ"):
            assert lists[0] != lists[1]
        if "scale_invariant" in case:
            lists2, _, _ = orc.block_select_query(q, k * case["scale_invariant"], pos, bs, top,
                                                  init, local)
            assert lists2 == lists
        for _ in range(case.get("repeat", 0)):
            assert orc.block_select_query(q, k, pos, bs, top, init, local)[0] == lists


def test_geometry(orc):
    g = G["geometry"]
    assert g["block_size"] == 128
    for pos, want in g["causal_blocks"]:
        assert orc.causal_blocks(pos, g["block_size"]) == want
    assert orc.causal_blocks(5, 0) == 0


def test_dot_is_sequential_and_unfused(orc):
    """The page's dot is an f32 sum of f32 products in index order.  A fused
    multiply-add would keep the 2^-24 that the rounded product drops, and any
    other summation order would not cancel 1e8 + 1 - 1e8 to 0."""
    a = np.array([-1.0, 1 + 2.0 ** -12], np.float32)
    b = np.array([1 + 2.0 ** -11, 1 + 2.0 ** -12], np.float32)
    assert orc.block_dot(a, b) == 0.0
    a = np.array([1e8, 1.0, -1e8], np.float32)
    assert orc.block_dot(a, np.ones(3, np.float32)) == 0.0
    # numpy's accumulate is a strictly sequential f32 running sum: same value
    rng = np.random.default_rng(9)
    for _ in range(200):
        D = int(rng.integers(1, 160))
        x = rng.standard_normal(D).astype(np.float32)
        y = (rng.standard_normal(D) * 10 ** rng.uniform(-3, 3, D)).astype(np.float32)
        prod = (x * y).astype(np.float32)
        seq = np.add.accumulate(np.concatenate([[np.float32(0.0)], prod]), dtype=np.float32)[-1]
        assert orc.block_dot(x, y) == seq
    # the +0 start: all-(-0) products still give +0, never -0
    z = orc.block_dot(np.array([-0.0], np.float32), np.array([1.0], np.float32))
    assert z == 0.0 and np.copysign(1.0, z) == 1.0


def test_selection_properties_random(orc):
    """On random geometries: ascending and distinct, count = min(n_blocks,
    budget), forced blocks present, and every scored block chosen ranks ahead
    (score desc, block asc) of every scored block left out; block scores equal
    the max over visible positions of the page's dot."""
    rng = np.random.default_rng(10)
    for _ in range(120):
        bs = int(rng.integers(1, 6))
        n_pos = int(rng.integers(1, 50))
        D = int(rng.integers(1, 6))
        H = int(rng.integers(1, 4))
        top, init, local = (int(rng.integers(0, 7)), int(rng.integers(0, 3)),
                            int(rng.integers(0, 3)))
        pos = int(rng.integers(0, 70))
        q = rng.integers(-2, 3, (H, D)).astype(np.float32)  # integer data: many ties
        k = rng.integers(-2, 3, (n_pos, D)).astype(np.float32)
        width = max(top, init + local, 1)
        lists, out, cnt, sc = orc.block_select_query(q, k, pos, bs, top, init, local, width,
                                                     want_scores=True)
        nb = min(pos // bs + 1, -(-n_pos // bs))
        forced = set(range(min(init, nb))) | set(range(max(nb - local, 0), nb))
        budget = max(top, len(forced))
        for h in range(H):
            sel = lists[h]
            assert sel == sorted(set(sel))
            assert len(sel) == min(nb, budget)
            assert forced <= set(sel)
            scored = [b for b in range(nb) if b not in forced]
            if len(forced) >= budget or len(forced) == nb:
                assert set(sel) == forced
                continue
            for b in scored:
                vis = range(b * bs, min((b + 1) * bs, n_pos, pos + 1))
                assert sc[h, b] == max(orc.block_dot(q[h], k[p]) for p in vis)
            chosen = [b for b in scored if b in sel]
            left = [b for b in scored if b not in sel]
            for c in chosen:
                for l in left:
                    assert (-sc[h, c], c) < (-sc[h, l], l)
