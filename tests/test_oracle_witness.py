"""Pins of the oracle's segment-witness merge against the "Segment Witnesses"
page: its hand examples, its contract table, its invariants (1)-(3) and the
uncovered-run bound, and its caveats."""
import json
import math
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD, "witness_pins.json")))


def test_hand_examples(orc):
    for c in G["witness_indices"]:
        rc, out = orc.witness_indices([c["learned"]], [c["L"]], c["S"])
        assert rc == orc.OK
        assert out[0].tolist() == c["expected"], c["cite"]
    for c in G["merge"]:
        rc, out = orc.kvwitness_merge([c["learned"]], [c["L"]], c["S"], c["keep"], c["max_rep"])
        assert rc == orc.OK
        if "expected" in c:
            assert out[0].tolist() == c["expected"], c["cite"]
        if "expected_set" in c:
            assert sorted(x for x in out[0].tolist() if x >= 0) == c["expected_set"], c["cite"]
        if "coverage" in c:
            assert orc.segment_coverage(out[0], c["L"], c["S"]) == c["coverage"]
    for c in G["segment_of"]:
        assert orc.segment_of(c["token"], c["L"], c["S"]) == c["expected"], c["cite"]
    for c in G["occupied_segment"]:
        assert orc.occupied_segment(c["x"], c["L"], c["S"]) == c["expected"], c["cite"]
    for c in G["coverage"]:
        assert orc.segment_coverage(c["cand"], c["L"], c["S"]) == c["expected"], c["cite"]


def test_out_of_range_entry_passes_through(orc):
    """Contract table, out-of-range row: L=4, S=8, entry 20 marks segment 7
    (outside the 4-segment partition) and stays in the row."""
    rc, out = orc.kvwitness_merge([[20, -1, -1, -1, -1, -1]], [4], 8, 1, 8)
    assert rc == orc.OK
    # S_eff = 4 one-token segments, none occupied -> witnesses 0,1,2,3 into slots 1..4
    assert out[0].tolist() == [20, 0, 1, 2, 3, -1]


def test_disabled_policy_is_identity(orc):
    """Contract table, Disabled row: S = 0, B = 0 or zero rows change nothing."""
    rows, lens = synth.witness_rows(seed=5, rows=8, topk=16, max_len=40)
    for S, keep, B in [(0, 8, 8), (4, 16, 8), (4, 8, 0)]:
        rc, out = orc.kvwitness_merge(rows, lens, S, keep, B)
        assert rc == orc.OK
        np.testing.assert_array_equal(out, rows)
    rc, out = orc.kvwitness_merge(np.zeros((0, 16), np.int32), np.zeros(0, np.int32), 4, 8, 8)
    assert rc == orc.OK


def test_short_and_empty_rows(orc):
    """Contract table, Fallback row: L <= 0 gets no witnesses (an all-padding row
    stays all padding); L < S gives S_eff = L and every unheld token is a witness."""
    pad = np.full((2, 6), -1, np.int32)
    rc, out = orc.kvwitness_merge(pad, [0, -3], 4, 0, 6)
    assert rc == orc.OK and np.all(out == -1)
    rc, out = orc.kvwitness_merge([[1, -1, -1, -1, -1, -1]], [3], 8, 1, 5)
    assert out[0].tolist() == [1, 0, 2, -1, -1, -1]


def test_refusals_leave_buffer_untouched(orc):
    """Refusals: each error kind, and a refused call writes nothing."""
    rows, lens = synth.witness_rows(seed=6, rows=4, topk=8, max_len=30)
    cases = [((rows, lens, 65, 4, 4), orc.SEGMENTS_OUT_OF_RANGE),
             ((rows, lens, -1, 4, 4), orc.SEGMENTS_OUT_OF_RANGE),
             ((rows, lens, 4, 9, 4), orc.KEEP_OUT_OF_RANGE),
             ((rows, None, 4, 4, 4), orc.ROWS_MISMATCH),
             ((rows, lens, 4, -1, 4), orc.INVALID_ARGUMENT),
             ((rows, lens, 4, 4, -2), orc.INVALID_ARGUMENT)]
    for args, want in cases:
        rc, out = orc.kvwitness_merge(*args)
        assert rc == want
        np.testing.assert_array_equal(out, rows)
    rc, _ = orc.witness_indices(rows, lens, 0)
    assert rc == orc.SEGMENTS_OUT_OF_RANGE  # "zero segments" is refused here


def test_every_witness_lands_in_its_own_segment(orc):
    """Invariant: sigma(e_s) = s for every s < S_eff and every S the merge accepts."""
    for L in list(range(1, 140)) + [1000, 4097, 131071, 131072]:
        for S in range(1, 65):
            Se = min(S, L)
            for s in range(Se):
                e = orc.segment_edge(s, L, Se)
                assert 0 <= e < L
                assert orc.segment_of(e, L, S) == s
                assert e == math.ceil(s * L / Se)


def _segments(orc, xs, L, S):
    return {orc.segment_of(x, L, S) for x in xs if 0 <= x < L}


def test_properties_1_to_3_and_run_bound(orc):
    """Invariant and consequences: W(K) and K are disjoint, witnesses are
    distinct, K u W covers every segment, and any run of unselected tokens is
    at most 2 ceil(L / S_eff) - 2 long."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        L = int(rng.integers(1, 400))
        S = int(rng.integers(1, 65))
        n = int(rng.integers(0, min(L, 40) + 1))
        K = rng.choice(L, size=n, replace=False).astype(np.int32)
        row = np.concatenate([K, np.full(3, -1, np.int32)])
        rc, W = orc.witness_indices([row], [L], S)
        W = [int(x) for x in W[0] if x >= 0]
        Se = min(S, L)
        assert not (set(W) & set(K.tolist()))
        assert len(set(W)) == len(W)
        assert _segments(orc, set(K.tolist()) | set(W), L, S) == set(range(Se))
        sel = sorted(set(K.tolist()) | set(W))
        gaps = [b - a - 1 for a, b in zip([-1] + sel, sel + [L])]
        assert max(gaps) <= 2 * math.ceil(L / Se) - 2


def test_serving_rows(orc):
    """200 randomised serving rows (keep = topk - S, B = S): the prefix is
    bit-identical, the witnesses form one ascending run starting at keep,
    the row stays distinct; with a padded tail every segment is covered."""
    rng = np.random.default_rng(8)
    for _ in range(200):
        S = int(rng.integers(1, 17))
        topk = int(rng.integers(S, 48))
        L = int(rng.integers(1, 300))
        keep = topk - S
        n = min(keep, L)
        row = np.full(topk, -1, np.int32)
        row[:n] = rng.choice(L, size=n, replace=False)
        rc, out = orc.kvwitness_merge([row], [L], S, keep, S)
        out = out[0]
        assert np.array_equal(out[:keep], row[:keep])
        tail = out[keep:]
        changed = [i for i in range(S) if tail[i] != row[keep + i]]
        assert changed == list(range(len(changed)))
        assert all(a < b for a, b in zip(tail[:len(changed)], tail[1:len(changed)]))
        valid = [x for x in out.tolist() if x >= 0]
        assert len(set(valid)) == len(valid)
        assert orc.segment_coverage(out, L, S) == 1.0
