"""GPU parity of block_sparse_select against the oracle: bit-exact block lists
and counts (the page fixes the f32 dot, so the selection is exact)."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from gpu_util import full_config, say

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_select(q, k, pos, bs, top, init, local, width=None):
    import sparse_attention_indexer_02_amd as si
    qt = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float32)).cuda()
    pt = torch.from_numpy(np.ascontiguousarray(pos, np.int64)).cuda()
    out, cnt = si.block_sparse_select(qt, kt, pt, block_size=bs, top_blocks=top,
                                      init_blocks=init, local_blocks=local, out_width=width)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cnt.cpu().numpy()


def _oracle(orc, q, k, pos, bs, top, init, local, width):
    outs, cnts = [], []
    for i in range(len(pos)):
        _, o, c = orc.block_select_query(q[i], k, int(pos[i]), bs, top, init, local, width)
        outs.append(o)
        cnts.append(c)
    return np.stack(outs), np.stack(cnts)


def test_page_scenarios(orc):
    from test_oracle_block import _keys
    g = json.load(open(os.path.join(GOLD, "block_pins.json")))
    for case in g["cases"]:
        bs, top, init, local = case["cfg"]
        k = _keys(case["keys"])
        q = np.array(case["q"], np.float32)
        pos = np.array(case["positions"], np.int64)
        qq = np.repeat(q[None], len(pos), axis=0)
        width = max(top, init + local, 1)
        got, gc = _gpu_select(qq, k, pos, bs, top, init, local, width)
        want, wc = _oracle(orc, qq, k, pos, bs, top, init, local, width)
        np.testing.assert_array_equal(got, want, err_msg=case["cite"])
        np.testing.assert_array_equal(gc, wc)
        if "expected" in case:
            for h, e in enumerate(case["expected"]):
                assert got[0, h, :gc[0, h]].tolist() == e


@pytest.mark.parametrize("seed", range(4))
def test_random_geometries(orc, seed):
    rng = np.random.default_rng(200 + seed)
    for trial in range(15):
        bs = int(rng.integers(1, 9))
        n_pos = int(rng.integers(0, 200))
        D = int(rng.integers(1, 40))
        H = int(rng.integers(1, 12))
        top, init, local = (int(rng.integers(0, 12)), int(rng.integers(0, 4)),
                            int(rng.integers(0, 4)))
        n_q = int(rng.integers(1, 20))
        width = max(top, init + local, 1) + int(rng.integers(0, 3))
        pos = rng.integers(-3, 260, n_q).astype(np.int64)
        if trial % 2:
            q = rng.integers(-2, 3, (n_q, H, D)).astype(np.float32)  # ties
            k = rng.integers(-2, 3, (n_pos, D)).astype(np.float32)
        else:
            q = rng.standard_normal((n_q, H, D)).astype(np.float32)
            k = rng.standard_normal((n_pos, D)).astype(np.float32)
        say(f"block seed={seed} trial={trial} bs={bs} n_pos={n_pos} D={D} H={H} "
            f"cfg=({top},{init},{local}) width={width}")
        got, gc = _gpu_select(q, k, pos, bs, top, init, local, width)
        want, wc = _oracle(orc, q, k, pos, bs, top, init, local, width)
        np.testing.assert_array_equal(got, want)
        np.testing.assert_array_equal(gc, wc)


def test_minimax_geometry_medium(orc):
    """128-token blocks, D = 128, 32 blocks with 1 init + 2 local, 8 heads."""
    cfg = synth.block(seed=3, n_q=64, n_pos=6000)
    say("block medium")
    got, gc = _gpu_select(cfg["q"], cfg["k"], cfg["query_pos"], 128, 32, 1, 2)
    want, wc = _oracle(orc, cfg["q"], cfg["k"], cfg["query_pos"], 128, 32, 1, 2, 32)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(gc, wc)


def test_full_size_queries(orc):
    """4096 queries over 131072 positions, 8 KV heads, D = 128.  Query j sits at
    32 j + 31, so queries 4m + 3 end a 128-position block and queries 4m + 4
    open the next one with 32 visible positions.  384 queries against the
    oracle: both sides of 128 block boundaries spread over the range (the
    partial newest block, the local pair shifting), the first 32 queries
    (fewer blocks than the budget, forced blocks overlapping) and the last
    one (every position visible)."""
    cfg = full_config("block")
    say("block full size")
    got, gc = _gpu_select(cfg["q"], cfg["k"], cfg["query_pos"], 128, 32, 1, 2)
    m = np.linspace(0, 1022, 128).astype(np.int64)
    rows = sorted(set(range(32)) | set((4 * m + 3).tolist()) | set((4 * m + 4).tolist()) |
                  {4095})
    rows = np.array(rows, np.int32)
    say(f"block full size: {len(rows)} queries against the oracle")
    out, cnt = orc.block_select_rows(cfg, rows)
    np.testing.assert_array_equal(got[rows], out)
    np.testing.assert_array_equal(gc[rows], cnt)
    # every query: ascending, forced blocks present, full budget once possible
    nb = np.minimum(cfg["query_pos"] // 128 + 1, 1024)
    assert np.all(gc == np.minimum(nb, 32)[:, None])
    assert np.all(got[:, :, 0] == 0)
    sel = np.where(got >= 0, got, np.iinfo(np.int32).max)
    assert np.all(np.diff(sel, axis=2)[got[:, :, 1:] >= 0] > 0)
    last = np.take_along_axis(got, (gc - 1)[:, :, None], axis=2)[:, :, 0]
    assert np.all(last == (nb - 1)[:, None])
