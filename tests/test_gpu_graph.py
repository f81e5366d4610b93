"""The allocation-free entry point under stream capture: a graph holding one
idx_score_topk_noalloc call, replayed several times with new query values
written in place and eager work between the replays, matches an eager
idx_score_topk on the same inputs after every replay (ids and score bits)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16_dev, dev_inputs, say

pytestmark = pytest.mark.gpu


def test_noalloc_graph_replays():
    import sparse_attention_indexer_02_amd as si
    cfg = synth.prefill(seed=11, n_q=256, L=1500, H=64, D=128, topk=128)
    d = dev_inputs(cfg)
    n_q, K, mv = cfg["n_q"], cfg["topk"], cfg["max_vis"]
    out_i = torch.empty((n_q, K), dtype=torch.int32, device="cuda")
    out_s = torch.empty((n_q, K), dtype=torch.float32, device="cuda")

    def call():
        si.idx_score_topk_noalloc(d["q"], d["k"], d["w"], d["vis_len"], K, max_vis=mv,
                                  out_idx=out_i, out_score=out_s)

    say("graph: warm-up call on a side stream, then capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(3):
        say(f"graph: replay {rep}")
        q_new = synth.prefill(seed=100 + rep, n_q=n_q, L=1500, H=64, D=128, topk=K)["q"]
        d["q"].copy_(bf16_dev(q_new))
        out_i.fill_(-9)  # eager work between replays: the replay must rewrite everything
        out_s.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ei, es = si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], K, max_vis=mv)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_i.cpu().numpy(), ei.cpu().numpy())
        np.testing.assert_array_equal(out_s.cpu().numpy().view(np.uint32),
                                      es.cpu().numpy().view(np.uint32))
