"""Calls made at once from several host threads, each on a stream of its own,
give the same bits as the same calls made one after another: the header's
promise that no call keeps state between calls and that calls are safe from
several threads on different streams."""
import threading

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_inputs, say

pytestmark = pytest.mark.gpu


def _workloads():
    """One closure per entry point family; each returns host copies of its
    outputs (after synchronising its own stream)."""
    import sparse_attention_indexer_02_amd as si
    pre = synth.prefill(seed=3, n_q=384, L=2000, H=64, D=128, topk=256, S=16)
    dec = synth.decode(seed=4, rows=16, max_len=20000, H=64, D=128, topk=512, S=32)
    dsa = synth.dosa(seed=5, n_q=64, L=4096, H=32, D=128, topk=256, n_seeds=1024, n_rep=4,
                     rep_topk=256, kept_heads=16)
    blk = synth.block(seed=6, n_q=64, n_pos=8192, H=4, D=64, block_size=128, top_blocks=8)
    dp, dd, ds = dev_inputs(pre), dev_inputs(dec), dev_inputs(dsa)
    bq = torch.from_numpy(blk["q"]).cuda()
    bk = torch.from_numpy(blk["k"]).cuda()
    bp = torch.from_numpy(blk["query_pos"]).cuda()

    def host(*ts):
        torch.cuda.current_stream().synchronize()
        return [t.cpu().numpy().copy() for t in ts if t is not None]

    def prefill():
        w = pre["witness"]
        i, s = si.idx_score_topk_witness(dp["q"], dp["k"], dp["w"], dp["vis_len"], pre["topk"],
                                         dp["vis_len"], w["S"], keep=w["keep"],
                                         max_replacements=w["max_rep"], max_vis=pre["max_vis"])
        return host(i, s)

    def decode():
        i, s = si.idx_score_topk(dd["q"], dd["k"], dd["w"], dd["vis_len"], dec["topk"],
                                 k_scale=dd["k_scale"], k_row_offset=dd["k_row_offset"],
                                 max_vis=dec["max_vis"])
        return host(i, s)

    def dosa():
        p = dsa["dosa"]
        i, s, _ = si.dosa_prune_topk(ds["q"], ds["k"], ds["w"], ds["vis_len"], dsa["topk"],
                                     n_seeds=p["n_seeds"], n_rep_queries=p["n_rep_queries"],
                                     rep_topk=p["rep_topk"], kept_heads=p["kept_heads"],
                                     neg_active_frac=p["neg_active_frac"])
        return host(i, s)

    def block():
        o, c = si.block_sparse_select(bq, bk, bp, block_size=blk["block_size"],
                                      top_blocks=blk["top_blocks"],
                                      init_blocks=blk["init_blocks"],
                                      local_blocks=blk["local_blocks"],
                                      out_width=blk["out_width"])
        return host(o, c)

    return dict(prefill=prefill, decode=decode, dosa=dosa, block=block)


def _same(a, b):
    return len(a) == len(b) and all(x.dtype == y.dtype and np.array_equal(x.view(np.uint8),
                                                                          y.view(np.uint8))
                                    for x, y in zip(a, b))


def test_threads_on_own_streams():
    calls = _workloads()
    say("streams: reference, one call after another")
    ref = {n: f() for n, f in calls.items()}
    torch.cuda.synchronize()
    n_threads, rounds = 3, 3
    results = [[] for _ in range(n_threads)]
    errors = []

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for r in range(rounds):
                    # each thread walks the entry points in its own order
                    names = list(calls)[t:] + list(calls)[:t]
                    for n in names:
                        results[t].append((n, calls[n]()))
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    say(f"streams: {n_threads} threads x {rounds} rounds x {len(calls)} entry points")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=300)
    torch.cuda.synchronize()
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    for t in range(n_threads):
        assert len(results[t]) == rounds * len(calls)
        for n, out in results[t]:
            assert _same(out, ref[n]), f"thread {t}: {n} differs from the one-at-a-time result"
