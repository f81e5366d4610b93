"""Pins of the oracle's consumer-side steps: the positions a block selection
covers (ferrox-core block_sparse.rs, positions_of_blocks and the module
tests that call it) and the KV gather slots of a selection row (Segment
Witnesses, Implementation rule and contracts: Coordinates)."""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD, "block_pins.json")))


def _covered_by_definition(blocks, qp, n_pos, bs):
    """The covered set written as a set: positions p visible to the query
    (p < n_pos, p <= qp) whose block p // bs is listed, ascending."""
    listed = {int(b) for b in blocks if b >= 0}
    return [p for p in range(max(0, min(n_pos, qp + 1))) if p // bs in listed]


@pytest.mark.parametrize("case", [c for c in G["cases"] if "covered" in c],
                         ids=lambda c: c["cite"][:48])
def test_positions_page_examples(orc, case):
    """The page's causal-clip example (blocks [0, 1] at query 6 of 16 keys,
    block 4 -> 0..6) and its past-the-end example (query 100 over 6 keys ->
    0..5), through the rows function with -1 padding after the list."""
    bs = case["cfg"][0]
    k_n = case["keys"].get("n", case["keys"].get("zeros"))
    for pos in case["positions"]:
        lists, _, cnt = orc.block_select_query(np.array(case["q"], np.float32),
                                               np.zeros((k_n, 2), np.float32), pos, bs,
                                               *case["cfg"][1:])
        sel = lists[0]
        blocks = np.full((1, 1, len(sel) + 2), -1, np.int32)
        blocks[0, 0, :len(sel)] = sel
        out, c = orc.positions_of_block_rows(blocks, [pos], k_n, bs, blocks.shape[2] * bs)
        assert list(out[0, 0, :c[0, 0]]) == case["covered"]
        assert (out[0, 0, c[0, 0]:] == -1).all()


def test_positions_literal_cases(orc):
    # the page: blocks [0, 1], query 6, 16 keys, block 4
    out, c = orc.positions_of_block_rows(np.array([[[0, 1]]], np.int32), [6], 16, 4, 8)
    assert list(out[0, 0]) == [0, 1, 2, 3, 4, 5, 6, -1] and c[0, 0] == 7
    # the page: blocks [0, 1], query 100 past 6 keys
    out, c = orc.positions_of_block_rows(np.array([[[0, 1]]], np.int32), [100], 6, 4, 8)
    assert list(out[0, 0, :c[0, 0]]) == [0, 1, 2, 3, 4, 5]
    # unordered, repeated and padded entries: sorted and deduplicated
    out, c = orc.positions_of_block_rows(np.array([[[3, 1, 1, -1]]], np.int32), [100], 16, 4, 16)
    assert list(out[0, 0, :c[0, 0]]) == [4, 5, 6, 7, 12, 13, 14, 15]
    # a negative query position sees nothing; a block past the query nothing
    out, c = orc.positions_of_block_rows(np.array([[[0, 2]]], np.int32), [-1], 16, 4, 8)
    assert c[0, 0] == 0 and (out == -1).all()
    out, c = orc.positions_of_block_rows(np.array([[[2]]], np.int32), [5], 16, 4, 4)
    assert c[0, 0] == 0


def test_positions_match_the_set_definition(orc):
    """Random lists (unordered, repeated, padded, past the keys, past the
    query) against the covered set written as a set."""
    rng = np.random.default_rng(5)
    for trial in range(200):
        bs = int(rng.choice([1, 2, 3, 4, 7]))
        n_pos = int(rng.integers(0, 40))
        n_q, heads, width = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 7))
        nb = -(-n_pos // bs) + 2
        blocks = rng.integers(-1, nb + 1, (n_q, heads, width)).astype(np.int32)
        qp = rng.integers(-2, n_pos + 6, n_q).astype(np.int64)
        ow = width * bs
        out, cnt = orc.positions_of_block_rows(blocks, qp, n_pos, bs, ow)
        for q in range(n_q):
            for h in range(heads):
                want = _covered_by_definition(blocks[q, h], int(qp[q]), n_pos, bs)
                got = list(out[q, h, :cnt[q, h]])
                assert got == want, (trial, q, h)
                assert (out[q, h, cnt[q, h]:] == -1).all()


def test_gather_flat_and_paged_examples(orc):
    """A witness-merged row [0, 5, 12, -1] of a 16-token context: flat rows
    add the row's start; paged rows (4-token pages, page table [7, 2, 9, 0])
    put token x at table[x / 4] * 4 + x % 4; an entry >= L_r (the contract's
    pass-through learned entry, e.g. 20) and -1 gather nothing."""
    idx = np.array([[0, 5, 12, -1, 20, 15]], np.int32)
    flat = orc.gather_slots(idx, [16], row_start=[100])
    assert list(flat[0]) == [100, 105, 112, -1, -1, 115]
    paged = orc.gather_slots(idx, [16], page_table=[[7, 2, 9, 0]], page_size=4)
    assert list(paged[0]) == [28, 9, 0, -1, -1, 3]
    # a page past the table, or an unallocated (negative) page, gathers nothing
    short = orc.gather_slots(idx, [16], page_table=[[7, -1]], page_size=4)
    assert list(short[0]) == [28, -1, -1, -1, -1, -1]


def test_gather_identity_pages_equal_flat_rows(orc):
    """With each row's pages laid out consecutively from its start (a page
    table start/page + i), paged and flat gathers agree; every gathered slot
    minus the row start gives back the entry."""
    rng = np.random.default_rng(9)
    rows, width, page = 7, 50, 16
    lens = rng.integers(0, 300, rows).astype(np.int32)
    starts = (np.concatenate([[0], np.cumsum(-(-lens // page) * page)[:-1]])).astype(np.int64)
    ppr = int(-(-lens.max() // page)) + 1
    table = (starts[:, None] // page + np.arange(ppr)[None, :]).astype(np.int32)
    idx = rng.integers(-3, 320, (rows, width)).astype(np.int32)
    flat = orc.gather_slots(idx, lens, row_start=starts)
    paged = orc.gather_slots(idx, lens, page_table=table, page_size=page)
    np.testing.assert_array_equal(flat, paged)
    ok = (idx >= 0) & (idx < lens[:, None])
    np.testing.assert_array_equal(flat[ok], (idx + starts[:, None])[ok])
    assert (flat[~ok] == -1).all()
