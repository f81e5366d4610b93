"""Helpers shared by the GPU parity tests: move synthetic inputs to the device
and print the case name before each GPU step."""
import functools
import sys

import numpy as np
import torch

import synth


@functools.lru_cache(maxsize=None)
def full_config(name):
    """Full-size workloads, generated once per test session."""
    return {"prefill": synth.prefill, "decode": synth.decode, "block": synth.block,
            "dosa": synth.dosa, "dosa_structured": synth.dosa_structured}[name]()


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_inputs(cfg):
    q = bf16_dev(cfg["q"]) if cfg["q_dtype"] == synth.BF16 else torch.from_numpy(cfg["q"]).cuda()
    if cfg["k_dtype"] == synth.BF16:
        k = bf16_dev(cfg["k"])
    else:
        k = torch.from_numpy(np.ascontiguousarray(cfg["k"])).cuda()
    ks = None if cfg.get("k_scale") is None else torch.from_numpy(cfg["k_scale"]).cuda()
    w = torch.from_numpy(np.ascontiguousarray(cfg["w"], dtype=np.float32)).cuda()
    vis = torch.from_numpy(np.ascontiguousarray(cfg["vis_len"], dtype=np.int32)).cuda()
    off = cfg.get("k_row_offset")
    off = None if off is None else torch.from_numpy(np.ascontiguousarray(off, np.int64)).cuda()
    return dict(q=q, k=k, k_scale=ks, w=w, vis_len=vis, k_row_offset=off)


def run_idx(cfg, want_scores=True):
    import sparse_attention_indexer_02_amd as si
    d = dev_inputs(cfg)
    idx, sc = si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], cfg["topk"],
                                k_scale=d["k_scale"], k_row_offset=d["k_row_offset"],
                                max_vis=cfg["max_vis"], want_scores=want_scores)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)
