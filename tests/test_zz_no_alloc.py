"""The allocation-free entry point (idx_score_topk_noalloc) through the C
ABI: two calls in a row on one GPU - the second on a smaller problem, so
the shared scratch still holds the first call's contents - each equal to
idx_score_topk (with its own workspace) bit for bit, ids and scores."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_inputs, say

pytestmark = pytest.mark.gpu

SCRATCH_LIMIT = 8


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _code(t):
    return {torch.float32: 0, torch.bfloat16: 1, torch.uint8: 2}[t.dtype]


def _call(L, fn, d, cfg, K, out_i, out_s, extra):
    n_q, H, D = d["q"].shape
    w_stride = H if d["w"].dim() == 2 else 0
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(_p(d["q"]), _code(d["q"]), _p(d["k"]), _code(d["k"]), _p(d["k_scale"]), _p(d["w"]),
              w_stride, _p(d["k_row_offset"]), _p(d["vis_len"]), n_q, H, D, d["k"].shape[0],
              cfg["max_vis"], K, _p(out_i), _p(out_s), *extra, stream)


def _compare(cfg, label):
    import sparse_attention_indexer_02_amd as si
    L = si.lib()
    d = dev_inputs(cfg)
    n_q, K = cfg["n_q"], cfg["topk"]
    dev = d["q"].device
    ws_n = L.idx_score_topk_workspace(n_q, cfg["H"], cfg["D"], cfg["max_vis"], K)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    ri = torch.empty((n_q, K), dtype=torch.int32, device=dev)
    rs = torch.empty((n_q, K), dtype=torch.float32, device=dev)
    ni = torch.full((n_q, K), -7, dtype=torch.int32, device=dev)
    ns = torch.full((n_q, K), 7.0, dtype=torch.float32, device=dev)
    say(f"no-alloc {label}: n_q={n_q} max_vis={cfg['max_vis']} K={K} scratch need {ws_n}")
    st = _call(L, L.idx_score_topk, d, cfg, K, ri, rs, (_p(ws), ws_n))
    assert st == 0, st
    st = _call(L, L.idx_score_topk_noalloc, d, cfg, K, ni, ns, ())
    assert st == 0, st
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ni.cpu().numpy(), ri.cpu().numpy())
    np.testing.assert_array_equal(ns.cpu().numpy().view(np.uint32), rs.cpu().numpy().view(np.uint32))


def test_two_calls_second_smaller():
    # first: decode rows past 8192 keys (the chunked top-K keeps candidate
    # lists in the scratch too), fp8 keys with row offsets
    _compare(synth.decode(seed=71, rows=40, max_len=60000, topk=1024), "decode, larger")
    # second: a smaller causal prefill on the same scratch
    _compare(synth.prefill(seed=72, n_q=96, L=700, H=64, D=128, topk=128), "prefill, smaller")


def test_beyond_the_limit_is_refused():
    import sparse_attention_indexer_02_amd as si
    L = si.lib()
    cfg = synth.prefill(seed=73, n_q=16, L=300, H=64, D=128, topk=64)
    d = dev_inputs(cfg)
    out = torch.full((cfg["n_q"], 64), -7, dtype=torch.int32, device="cuda")
    big = dict(cfg, max_vis=(128 << 20) // 4 // 16 + 1)  # 16 rows x max_vis floats > 128 MiB
    say("no-alloc refusal beyond the scratch")
    assert _call(L, L.idx_score_topk_noalloc, d, big, 64, out, None, ()) == SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(out == -7).item()
