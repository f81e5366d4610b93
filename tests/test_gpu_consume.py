"""GPU parity of the consumer-side steps, bit-exact against the oracle:
positions_of_blocks (the positions a block list covers) and gather_slots
(the KV slots of selection rows, flat and paged)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def _positions(blocks, qpos, n_pos, bs, out_width):
    import sparse_attention_indexer_02_amd as si
    b = torch.from_numpy(np.ascontiguousarray(blocks, np.int32)).cuda()
    q = torch.from_numpy(np.ascontiguousarray(qpos, np.int64)).cuda()
    pos, cnt = si.positions_of_blocks(b, q, n_pos, bs, out_width=out_width)
    torch.cuda.synchronize()
    return pos.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("width,bs,n_pos", [(1, 4, 37), (5, 3, 40), (32, 128, 20000),
                                            (64, 1, 300), (65, 7, 2000), (300, 16, 9000),
                                            (4096, 1, 5000)])
def test_positions_random_lists(orc, width, bs, n_pos):
    """Unordered lists with repeats, padding anywhere, blocks past the keys
    and past the query, queries before 0 and past the end."""
    say(f"positions width {width} bs {bs} n_pos {n_pos}")
    rng = np.random.default_rng(width * 7 + bs)
    n_q, H = 9, 3
    nb = -(-n_pos // bs)
    blocks = rng.integers(-2, nb + 3, (n_q, H, width)).astype(np.int32)
    blocks[0, 0] = np.sort(blocks[0, 0])[::-1]  # descending input
    blocks[1] = np.sort(np.abs(blocks[1]), axis=1)  # ascending, already in order
    qpos = rng.integers(-2, n_pos + 5, n_q).astype(np.int64)
    ow = min(width * bs, n_pos) + 3
    gp, gc = _positions(blocks, qpos, n_pos, bs, ow)
    op, oc = orc.positions_of_block_rows(blocks, qpos, n_pos, bs, ow)
    np.testing.assert_array_equal(gc, oc)
    np.testing.assert_array_equal(gp, op)


def test_positions_selection_shaped_lists(orc):
    """Selection-shaped lists (forced first/last blocks, ascending, -1
    padded) and messy ones at 256 queries x 8 heads over 32768 positions."""
    for messy in (False, True):
        blocks, qpos = synth.block_lists(seed=3, n_q=256, H=8, n_pos=32768, messy=messy)
        ow = blocks.shape[2] * 128
        gp, gc = _positions(blocks, qpos, 32768, 128, ow)
        op, oc = orc.positions_of_block_rows(blocks, qpos, 32768, 128, ow)
        np.testing.assert_array_equal(gc, oc)
        np.testing.assert_array_equal(gp, op)


def test_positions_full_size(orc):
    """4096 queries x 8 KV heads x 32 blocks of 128 over 131072 positions
    (the block-select workload's output shape): every list, bit-exact."""
    blocks, qpos = synth.block_lists(seed=1)
    ow = 32 * 128
    gp, gc = _positions(blocks, qpos, 131072, 128, ow)
    op, oc = orc.positions_of_block_rows(blocks, qpos, 131072, 128, ow)
    say(f"covered positions {int(gc.sum())}")
    np.testing.assert_array_equal(gc, oc)
    np.testing.assert_array_equal(gp, op)


def _gather(idx, lens, **kw):
    import sparse_attention_indexer_02_amd as si
    dev = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dt)).cuda()
    out = si.gather_slots(dev(idx, np.int32), dev(lens, np.int32),
                          row_start=dev(kw.get("row_start"), np.int64),
                          page_table=dev(kw.get("page_table"), np.int32),
                          page_size=kw.get("page_size", 0))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("rows,width,page", [(1, 1, 1), (7, 5, 4), (64, 64, 128), (33, 1500, 16),
                                             (5, 2049, 128)])
def test_gather_random_rows(orc, rows, width, page):
    """Witness-merge-shaped rows (padding, out-of-range learned entries,
    non-positive lengths) through flat starts and a shuffled page table with
    unallocated entries."""
    say(f"gather rows {rows} width {width} page {page}")
    idx, lens = synth.witness_rows(seed=rows + width, rows=rows, topk=width,
                                   max_len=max(2 * width, 4))
    starts, table = synth.kv_layout(seed=page, lens=np.maximum(lens, 0), page_size=page)
    for kw in (dict(row_start=starts), dict(page_table=table, page_size=page),
               dict(page_table=table[:, :1], page_size=page)):
        np.testing.assert_array_equal(_gather(idx, lens, **kw), orc.gather_slots(idx, lens, **kw))


@pytest.mark.parametrize("what", ["prefill", "decode"])
def test_gather_full_size(orc, what):
    """8192 rows x 2048 (prefill rows, one shared paged sequence) and 128 rows
    x 2048 of ragged lengths up to 131072 (decode, flat), every entry."""
    if what == "prefill":
        rows, L, page = 8192, 8192, 128
        lens = (L - rows + 1 + np.arange(rows)).astype(np.int32)
        idx, _ = synth.witness_rows(seed=11, rows=rows, topk=2048, max_len=8192)
        _, table1 = synth.kv_layout(seed=12, lens=[L], page_size=page)
        kw = dict(page_table=np.repeat(table1, rows, axis=0), page_size=page)
    else:
        idx, lens = synth.witness_rows(seed=13, rows=128, topk=2048, max_len=131072)
        starts, _ = synth.kv_layout(seed=14, lens=np.maximum(lens, 0))
        kw = dict(row_start=starts)
    np.testing.assert_array_equal(_gather(idx, lens, **kw), orc.gather_slots(idx, lens, **kw))
