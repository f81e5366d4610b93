#!/usr/bin/env python3
"""Benchmark of the sparse-attention indexer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload prefill|decode|dosa|dosa_structured|block]

Default workload: the DSA-style causal prefill chunk, 8192 queries x 8192
keys, H=64, D=128, bf16, K=2048, then the segment-witness merge (S=16,
serving keep/budget).  One step = idx_score_topk (score rows with the MFMA
kernel, then the block top-K) -> witness merge, all on the current HIP stream
with inputs resident in HBM.  value = visible query-key pairs per second of
the whole step.  Per-kernel times come from HIP events recorded on that
stream around each stage.

Prints ONE JSON line.  With --gpus N > 1 it exits: it measures one GPU (row
sharding across GPUs is described in the design notes).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer query·key pairs scored+top-K'd /sec at H64 D128 K2048; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# fp32 vector issue rate: the published 157.3 TFLOP/s counts an FMA as two
# flops, i.e. 78.6 T fp32 lane-operations/s (256 CUs x 128 lanes x 2.4 GHz).
# The block kernel issues its multiplies and adds as separate instructions,
# each one lane-operation.
PEAK_VALU_TOPS = 256 * 128 * 2.4e9 / 1e12


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def counters_for(workload):
    """HBM bytes per launch of the workload's dominant kernel, measured with
    rocprofv3 FETCH_SIZE / WRITE_SIZE and scaled against a plain copy, if that
    measurement was taken on the kernel sources as they are now (else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        ent = json.load(open(path))[workload]
        h = hashlib.sha256()
        for f in ent["sources"]:
            h.update(open(os.path.join(ROOT, "sparse_attention_indexer_02_amd", "csrc", f),
                          "rb").read())
        if ent["source_sha256"] != h.hexdigest():
            return None
        return ent["hbm_bytes_per_launch"]
    except (KeyError, ValueError, OSError):
        return None


def to_device(cfg):
    """Synthetic host arrays -> torch device tensors (bf16 travels as int16 bits)."""
    import numpy as np
    import torch

    def bits(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).cuda()

    q = bits(cfg["q"], torch.bfloat16) if cfg["q_dtype"] == 1 else torch.from_numpy(cfg["q"]).cuda()
    k = bits(cfg["k"], torch.bfloat16) if cfg["k_dtype"] == 1 else \
        torch.from_numpy(np.ascontiguousarray(cfg["k"])).cuda()
    opt = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dt)).cuda()
    return dict(q=q, k=k, k_scale=opt(cfg.get("k_scale"), np.float32),
                w=opt(cfg["w"], np.float32), vis_len=opt(cfg["vis_len"], np.int32),
                k_row_offset=opt(cfg.get("k_row_offset"), np.int64))


def timed_steps(stages, steps, warmup):
    """Run warmup + steps; return wall ms/step and mean ms per stage (events)."""
    import torch
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        evs[s][0].record()
        for i, (_, fn) in enumerate(stages):
            fn()
            evs[s][i + 1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = {}
    for i, (name, _) in enumerate(stages):
        per[name] = sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)) / steps
    return wall_ms, per


def cpu_baseline_rows(cfg, seconds, witness=None):
    """The oracle, as it stands, on evenly spaced rows of the workload: grows
    the sample until it has run about `seconds` (bounded)."""
    import numpy as np

    import oracle
    kp = oracle.problem(cfg)
    n = 16
    elapsed, pairs, rows = 0.0, 0, []
    while True:
        rows = np.unique(np.linspace(0, cfg["n_q"] - 1, min(n, cfg["n_q"])).astype(np.int32))
        t0 = time.perf_counter()
        idx, _ = oracle.idx_score_topk_rows(kp, rows)
        if witness is not None:
            oracle.kvwitness_merge(idx, cfg["vis_len"][rows], witness["S"], witness["keep"],
                                   witness["max_rep"])
        elapsed = time.perf_counter() - t0
        pairs = int(sum(oracle.visible(kp, int(r)) for r in rows))
        if elapsed >= seconds * 0.5 or len(rows) >= cfg["n_q"]:
            break
        n = int(n * min(8.0, max(2.0, seconds / max(elapsed, 1e-3))))
    return dict(value=pairs / elapsed, unit="pairs/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{len(rows)} evenly spaced rows of the {cfg['n_q']}-row workload "
                       f"({pairs} pairs, {elapsed:.1f} s: score + top-K"
                       f"{' + witness' if witness else ''})")


def bench_indexer(args, cfg, workload):
    """One step = idx_score_topk_witness: the score kernel, then the block
    top-K kernel that also does each row's witness merge.  The same result as
    two calls (idx_score_topk, then kvwitness_merge) and the score and top-K
    stages on their own (idx_score, rows_topk) are timed too, for the
    per-kernel view."""
    import numpy as np
    import torch

    import sparse_attention_indexer_02_amd as si
    d = to_device(cfg)
    n_q, H, D, K, mv = cfg["n_q"], cfg["H"], cfg["D"], cfg["topk"], cfg["max_vis"]
    dev = d["q"].device
    scores = torch.empty((n_q, mv), dtype=torch.float32, device=dev)
    out_idx = torch.empty((n_q, K), dtype=torch.int32, device=dev)
    st_idx = torch.empty((n_q, K), dtype=torch.int32, device=dev)
    wit = cfg["witness"]
    pairs = int(np.minimum(np.maximum(cfg["vis_len"].astype(np.int64), 0), mv).sum())
    ws = torch.empty(max(si.lib().idx_score_topk_workspace(n_q, H, D, mv, K), 1),
                     dtype=torch.uint8, device=dev)
    topk_ws = torch.empty(max(si.lib().rows_topk_workspace(n_q, mv, K), 1), dtype=torch.uint8,
                          device=dev)

    def score_topk():
        si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], K, k_scale=d["k_scale"],
                          k_row_offset=d["k_row_offset"], max_vis=mv, out_idx=out_idx,
                          want_scores=False, workspace=ws)

    def witness():
        si.kvwitness_merge(out_idx, d["vis_len"], wit["S"], wit["keep"], wit["max_rep"])

    def fused():
        si.idx_score_topk_witness(d["q"], d["k"], d["w"], d["vis_len"], K, d["vis_len"], wit["S"],
                                  keep=wit["keep"], max_replacements=wit["max_rep"],
                                  k_scale=d["k_scale"], k_row_offset=d["k_row_offset"],
                                  max_vis=mv, out_idx=out_idx, want_scores=False, workspace=ws)

    def score():
        si.idx_score(d["q"], d["k"], d["w"], d["vis_len"], k_scale=d["k_scale"],
                     k_row_offset=d["k_row_offset"], max_vis=mv, out_scores=scores)

    def topk():
        si.rows_topk(scores, d["vis_len"], K, k_row_offset=d["k_row_offset"], n_k=cfg["n_k"],
                     max_vis=mv, out_idx=st_idx, want_scores=False, workspace=topk_ws)

    log(f"{workload}: {pairs} visible pairs, warmup {args.warmup}, steps {args.steps}")
    # the step as two calls (idx_score_topk, then the merge kernel), for the
    # per-stage view
    _, per = timed_steps([("score_topk", score_topk), ("witness", witness)], args.steps,
                         args.warmup)
    # the step: one call, the merge done by the top-K kernel on each row
    wall_ms, fz = timed_steps([("step", fused)], args.steps, args.warmup)
    _, st = timed_steps([("score", score), ("topk", topk)], args.steps, args.warmup)
    # the witness kernel alone, eight launches back to back per timed step:
    # its average launch time without the gap a single short launch carries
    # (every launch reads the whole rows; with a budget of S every segment
    # the first one finds empty gets its witness, so the repeats write
    # nothing)
    WIT_REP = 8
    _, wt = timed_steps([("witness", lambda: [witness() for _ in range(WIT_REP)])], args.steps,
                        args.warmup)
    # a plain device copy of the id rows the merge works on, one launch per
    # event like the merge: the pages measure the merge against such a copy
    row_copy = torch.empty_like(out_idx)
    _, cp = timed_steps([("copy", lambda: row_copy.copy_(out_idx))], args.steps, args.warmup)

    flops = pairs * 2.0 * H * D
    kbytes = cfg["k"].nbytes + (cfg["k_scale"].nbytes if cfg["k_scale"] is not None else 0)
    score_bytes = cfg["q"].nbytes + kbytes + cfg["w"].nbytes + pairs * 4
    topk_bytes = pairs * 4 + n_q * K * 4
    B = min(wit["max_rep"], K - wit["keep"])
    wit_bytes = n_q * K * 4 + n_q * 4 + n_q * B * 4
    kern = {
        "score_topk_witness": dict(ms=fz["step"], tflops=flops / fz["step"] / 1e9,
                                   algo_flops=flops, note="the step: one fused call"),
        "score_topk": dict(ms=per["score_topk"], tflops=flops / per["score_topk"] / 1e9,
                           algo_flops=flops),
        "witness": dict(ms=per["witness"], gbs=wit_bytes / per["witness"] / 1e6,
                        algo_bytes=wit_bytes, row_copy_ms=cp["copy"],
                        vs_row_copy=per["witness"] / cp["copy"]),
        "witness_stage": dict(ms=wt["witness"] / WIT_REP,
                              gbs=wit_bytes / (wt["witness"] / WIT_REP) / 1e6,
                              algo_bytes=wit_bytes, launches_per_event=WIT_REP),
        "score_stage": dict(ms=st["score"], tflops=flops / st["score"] / 1e9,
                            gbs=score_bytes / st["score"] / 1e6, algo_flops=flops,
                            algo_bytes=score_bytes),
        "topk_stage": dict(ms=st["topk"], gbs=topk_bytes / st["topk"] / 1e6,
                           algo_bytes=topk_bytes),
    }
    for kk in kern.values():
        if "gbs" in kk:
            kk["hbm_frac"] = kk["gbs"] / PEAK_HBM_GBS
        if "tflops" in kk:
            kk["mfma_frac"] = kk["tflops"] / PEAK_BF16_TFLOPS

    if workload == "decode":
        # per-row keys: every key byte is read once; HBM-bound
        ach = score_bytes / st["score"] / 1e6
        roof = dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=ach / PEAK_HBM_GBS, traffic=counters_for(workload),
                    kernel="score_mfma_rows_fp8")
    else:
        # the score kernel: MFMA work over its own (stage) time
        ach = kern["score_stage"]["tflops"]
        roof = dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=ach / PEAK_BF16_TFLOPS, traffic=counters_for(workload),
                    kernel="score_mfma_shared")
    # the step's other passes against their own (HBM) bound, beside the
    # dominant kernel's figure
    roof["other_passes"] = {
        "topk_block": dict(bound="hbm", achieved=kern["topk_stage"]["gbs"], peak=PEAK_HBM_GBS,
                           unit="GB/s", frac=kern["topk_stage"]["hbm_frac"]),
        "witness_merge": dict(bound="hbm", achieved=kern["witness"]["gbs"], peak=PEAK_HBM_GBS,
                              unit="GB/s", frac=kern["witness"]["hbm_frac"],
                              note="one launch between events"),
    }
    step_ms = fz["step"]
    kern["two_calls"] = dict(ms=per["score_topk"] + per["witness"],
                             note="idx_score_topk then kvwitness_merge")
    out = dict(metric=METRIC, value=pairs / (wall_ms / 1e3), unit="pairs/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=wall_ms, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
               config=dict(workload=workload_name(cfg, workload), n_q=n_q, H=H, D=D,
                           n_keys=cfg["n_k"], topk=K, witness_segments=wit["S"],
                           key_dtype={0: "f32", 1: "bf16", 2: "fp8_e4m3fn"}[cfg["k_dtype"]],
                           pairs_per_step=pairs),
               roofline=roof, kernels=kern, event_ms_per_step=step_ms)
    out["consumer"] = bench_gather(args, cfg, d, out_idx, workload)
    if workload == "decode":
        out["prior_path"] = [bench_prior(args, cfg, d, out_idx, wit, eps) for eps in PRIOR_EPS]
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_rows(cfg, args.cpu_seconds, wit)
    return out


def bench_gather(args, cfg, d, idx, workload):
    """The consumer's gather list of the step's witness-merged rows (not part
    of the step): decode rows live back to back in a flat KV buffer (row
    starts = the rows' key offsets); prefill rows share one sequence held in
    shuffled 128-token pages."""
    import numpy as np
    import torch

    import sparse_attention_indexer_02_amd as si
    import synth
    n_q, K = idx.shape
    dev = idx.device
    kw = {}
    if workload == "decode":
        kw["row_start"] = d["k_row_offset"]
        extra = n_q * 8
    else:
        _, table = synth.kv_layout(seed=5, lens=[cfg["n_k"]], page_size=128)
        kw["page_table"] = torch.from_numpy(np.repeat(table, n_q, axis=0)).to(dev)
        kw["page_size"] = 128
        extra = n_q * table.size * 4  # every row's copy of the sequence's table
    out = torch.empty((n_q, K), dtype=torch.int64, device=dev)

    def gather():
        si.gather_slots(idx, d["vis_len"], out=out, **kw)

    _, per = timed_steps([("gather", gather)], args.steps, args.warmup)
    nbytes = n_q * K * (4 + 8) + n_q * 4 + extra
    return dict(gather_slots=dict(ms=per["gather"], algo_bytes=nbytes,
                                  gbs=nbytes / per["gather"] / 1e6,
                                  hbm_frac=nbytes / per["gather"] / 1e6 / PEAK_HBM_GBS,
                                  layout="flat row starts" if workload == "decode"
                                  else "paged, 128-token pages"))


# query perturbations standing in for the previous decode step (the prior
# then holds about 90% and 73% of the step's selected ids)
PRIOR_EPS = (0.1, 0.3)


def bench_prior(args, cfg, d, ref_idx, wit, eps):
    """The same decode step through idx_score_topk_prior.  The prior is the
    top-K of the previous step, stood in for by the plain top-K of the queries
    plus eps * N(0, 1) noise (seeded), computed before the timed region.
    Checks that the ids equal the plain path's."""
    import numpy as np
    import torch

    import sparse_attention_indexer_02_amd as si
    n_q, H, D, K, mv = cfg["n_q"], cfg["H"], cfg["D"], cfg["topk"], cfg["max_vis"]
    dev = d["q"].device
    g = torch.Generator(device="cpu").manual_seed(11)
    qp = (d["q"].float() + eps * torch.randn(d["q"].shape, generator=g).to(dev))
    qp = qp.to(torch.bfloat16).contiguous()
    prior, _ = si.idx_score_topk(qp, d["k"], d["w"], d["vis_len"], K, k_scale=d["k_scale"],
                                 k_row_offset=d["k_row_offset"], max_vis=mv, want_scores=False)
    out_idx = torch.empty((n_q, K), dtype=torch.int32, device=dev)
    ws = torch.empty(max(si.lib().idx_score_topk_prior_workspace(n_q, mv, K), 1),
                     dtype=torch.uint8, device=dev)

    def step():
        si.idx_score_topk_prior(d["q"], d["k"], d["w"], d["vis_len"], K, prior,
                                k_scale=d["k_scale"], k_row_offset=d["k_row_offset"],
                                max_vis=mv, out_idx=out_idx, want_scores=False, workspace=ws)

    def witness():
        si.kvwitness_merge(out_idx, d["vis_len"], wit["S"], wit["keep"], wit["max_rep"])

    def fused():
        si.idx_score_topk_witness(d["q"], d["k"], d["w"], d["vis_len"], K, d["vis_len"], wit["S"],
                                  keep=wit["keep"], max_replacements=wit["max_rep"],
                                  k_scale=d["k_scale"], k_row_offset=d["k_row_offset"],
                                  max_vis=mv, out_idx=out_idx, want_scores=False, workspace=ws)

    wall_ms, per = timed_steps([("score_topk_prior", step), ("witness", witness)], args.steps,
                               args.warmup)
    # (the timed output went through the witness merge; compare fresh ids)
    pid, _, (tau, surv) = si.idx_score_topk_prior(
        d["q"], d["k"], d["w"], d["vis_len"], K, prior, k_scale=d["k_scale"],
        k_row_offset=d["k_row_offset"], max_vis=mv, want_scores=False, want_stats=True)
    plain, _ = si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], K, k_scale=d["k_scale"],
                                 k_row_offset=d["k_row_offset"], max_vis=mv, want_scores=False)
    torch.cuda.synchronize()
    same = bool(torch.equal(plain, pid))
    # share of this step's selected ids that the prior also holds, per row
    pr, pl = prior.cpu().numpy(), plain.cpu().numpy()
    overlap = float(np.mean([np.intersect1d(a[a >= 0], b[b >= 0]).size / max(1, int((b >= 0).sum()))
                             for a, b in zip(pr, pl)]))
    vis = np.minimum(cfg["vis_len"].astype(np.int64), mv)
    return dict(ms_per_step=wall_ms, stage_ms={k: v for k, v in per.items()},
                ids_equal_plain=same, survivors=int(surv.sum().item()), visible=int(vis.sum()),
                survival=float(surv.sum().item()) / float(vis.sum()),
                prior=f"plain top-K of q + {eps} N(0,1) (seed 11); "
                      f"it holds {overlap:.3f} of this step's selected ids")


def workload_name(cfg, workload):
    if workload == "prefill":
        return (f"causal prefill {cfg['n_q']}x{cfg['n_k']} H{cfg['H']} D{cfg['D']} bf16 "
                f"K{cfg['topk']} + witness S{cfg['witness']['S']}")
    if workload == "decode":
        return (f"decode {cfg['n_q']} ragged rows (sum L {cfg['n_k']}) fp8 keys H{cfg['H']} "
                f"D{cfg['D']} K{cfg['topk']} + witness S{cfg['witness']['S']}")
    return workload


def bench_block(args):
    import numpy as np
    import torch

    import oracle
    import sparse_attention_indexer_02_amd as si
    import synth
    cfg = synth.block()
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(cfg["q"]).to(dev)
    k = torch.from_numpy(cfg["k"]).to(dev)
    pos = torch.from_numpy(cfg["query_pos"]).to(dev)
    H, D, bs = cfg["H"], cfg["D"], cfg["block_size"]
    width = cfg["out_width"]
    out = torch.empty((cfg["n_q"], H, width), dtype=torch.int32, device=dev)
    cnt = torch.empty((cfg["n_q"], H), dtype=torch.int32, device=dev)
    ws = torch.empty(si.lib().block_sparse_select_workspace(cfg["n_q"], H, cfg["n_pos"], bs),
                     dtype=torch.uint8, device=dev)

    def step():
        si.block_sparse_select(q, k, pos, block_size=bs, top_blocks=cfg["top_blocks"],
                               init_blocks=cfg["init_blocks"], local_blocks=cfg["local_blocks"],
                               out_width=width, out_blocks=out, out_count=cnt, workspace=ws)

    wall_ms, per = timed_steps([("select", step)], args.steps, args.warmup)
    # the consumer's positions of the selection (not part of the step)
    ow = width * bs
    cov = torch.empty((cfg["n_q"], H, ow), dtype=torch.int32, device=dev)
    cov_n = torch.empty((cfg["n_q"], H), dtype=torch.int32, device=dev)

    def positions():
        si.positions_of_blocks(out, pos, cfg["n_pos"], bs, out_width=ow, out_pos=cov,
                               out_count=cov_n)

    _, pp = timed_steps([("positions", positions)], args.steps, args.warmup)
    pbytes = cfg["n_q"] * H * (width * 4 + ow * 4 + 4) + cfg["n_q"] * 8
    pos_np = np.minimum(cfg["query_pos"], cfg["n_pos"] - 1)
    dots = int((pos_np + 1).sum()) * H  # (query, head, visible position) dots
    ops = dots * 2.0 * D
    ach = ops / per["select"] / 1e9
    out_d = dict(metric="block-sparse (query, head, position) dots scored+selected /sec",
                 value=dots / (wall_ms / 1e3), unit="dots/s", n_gpus=1, steps=args.steps,
                 warmup=args.warmup, ms_per_step=wall_ms, higher_is_better=True,
                 scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
                 config=dict(workload=f"block-sparse select {cfg['n_q']} queries x "
                                      f"{cfg['n_pos']} positions, {H} KV heads, D{D}, "
                                      f"block {bs}, top {cfg['top_blocks']}"),
                 roofline=dict(bound="alu", achieved=ach, peak=PEAK_VALU_TOPS, unit="TFLOP/s",
                               frac=ach / PEAK_VALU_TOPS,
                               traffic=counters_for("block"),
                               kernel="block_max128"),
                 consumer=dict(positions_of_blocks=dict(
                     ms=pp["positions"], algo_bytes=pbytes, gbs=pbytes / pp["positions"] / 1e6,
                     hbm_frac=pbytes / pp["positions"] / 1e6 / PEAK_HBM_GBS,
                     out_width=ow)))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        n = 4
        while True:
            rows = np.linspace(0, cfg["n_q"] - 1, n).astype(np.int32)
            t0 = time.perf_counter()
            oracle.block_select_rows(cfg, rows)
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds * 0.5 or n >= cfg["n_q"]:
                break
            n = min(cfg["n_q"], int(n * min(8.0, max(2.0, args.cpu_seconds / max(el, 1e-3)))))
        d = int((pos_np[rows] + 1).sum()) * H
        out_d["cpu_baseline"] = dict(value=d / el, unit="dots/s", cores=oracle.num_threads(),
                                     kind="oracle",
                                     sample=f"{len(rows)} evenly spaced queries ({d} dots, "
                                            f"{el:.1f} s)")
    return out_d


def bench_dosa(args):
    """DoSA certified prune on the 4096 x 32768 causal chunk (H32 D128 K2048,
    12,288 cold-prior seeds, 16 kept heads) next to the unpruned top-K of the
    same inputs; value = visible pairs whose top-K membership is decided per
    second (the unpruned-equivalent throughput)."""
    import numpy as np
    import torch

    import sparse_attention_indexer_02_amd as si
    import synth
    log(f"generating {args.workload} inputs")
    cfg = synth.dosa() if args.workload == "dosa" else synth.dosa_structured()
    d = to_device(cfg)
    n_q, H, D, K, n_k = cfg["n_q"], cfg["H"], cfg["D"], cfg["topk"], cfg["n_k"]
    dp = cfg["dosa"]
    dev = d["q"].device
    cap = 8192
    out_i = torch.empty((n_q, K), dtype=torch.int32, device=dev)
    out_s = torch.empty((n_q, K), dtype=torch.float32, device=dev)
    ref_i = torch.empty_like(out_i)
    ref_s = torch.empty_like(out_s)
    p = si._binding.DosaParams(dp["n_seeds"], dp["n_rep_queries"], dp["rep_topk"],
                               dp["kept_heads"], dp["neg_active_frac"], None, cap)
    import ctypes
    ws = torch.empty(si.lib().dosa_prune_topk_workspace(n_q, H, D, n_k, K, ctypes.byref(p)),
                     dtype=torch.uint8, device=dev)
    ws_u = torch.empty(si.lib().idx_score_topk_workspace(n_q, H, D, n_k, K), dtype=torch.uint8,
                       device=dev)
    stats = {}

    def dosa(shared=False):
        _, _, st = si.dosa_prune_topk(d["q"], d["k"], d["w"], d["vis_len"], K,
                                      n_seeds=dp["n_seeds"], n_rep_queries=dp["n_rep_queries"],
                                      rep_topk=dp["rep_topk"], kept_heads=dp["kept_heads"],
                                      neg_active_frac=dp["neg_active_frac"],
                                      survivor_capacity=cap, out_idx=out_i, out_score=out_s,
                                      want_stats=True, workspace=ws, shared_streams=shared)
        stats.update(st)

    def unpruned():
        si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], K, out_idx=ref_i,
                          out_score=ref_s, workspace=ws_u)

    pairs = int(cfg["vis_len"].astype(np.int64).sum())
    # 4-query shared streams: the same result, timed first so that the
    # per-row run's outputs and stats are the ones checked below
    unpruned()
    _, per_g = timed_steps([("groups", lambda: dosa(True))], args.steps, args.warmup)
    torch.cuda.synchronize()
    eq_g = bool(torch.equal(out_i, ref_i) and torch.equal(out_s.view(torch.int32),
                                                          ref_s.view(torch.int32)))
    shared_n = int(stats["n_shared"].sum().item())
    wall_ms, per = timed_steps([("dosa", dosa)], args.steps, args.warmup)
    _, per_u = timed_steps([("unpruned", unpruned)], args.steps, args.warmup)
    torch.cuda.synchronize()
    equal = bool(torch.equal(out_i, ref_i) and torch.equal(out_s.view(torch.int32),
                                                            ref_s.view(torch.int32)))
    surv = stats["n_survivors"].cpu().numpy().astype(np.int64)
    fb = stats["fallback"].cpu().numpy()
    kept = dp["kept_heads"]
    scanned_rows = cfg["vis_len"].astype(np.int64) - dp["n_seeds"]
    # The method's own work (2 D flop per head-key dot): the representative
    # rows over the common prefix, every row's seeds at H heads, and then per
    # row either the bound over its other visible keys at kept + 1 rows plus
    # its survivors at H heads, or (rows over the capacity) the exact path
    # over every visible key at H heads.  The bound's rows beyond kept + 1
    # (its 32-row MFMA tile) and a fallback row's partial bound are not
    # counted.
    vis64 = np.minimum(cfg["vis_len"].astype(np.int64), n_k)
    c_common = int(vis64.min())
    fbm = fb.astype(bool)
    alg_dots = (dp["n_rep_queries"] * c_common * H + n_q * dp["n_seeds"] * H +
                int(((vis64 - dp["n_seeds"])[~fbm]).sum()) * (kept + 1) +
                int(surv.clip(0)[~fbm].sum()) * H + int(vis64[fbm].sum()) * H)
    alg_flops = 2.0 * D * alg_dots
    ach = alg_flops / per["dosa"] / 1e9
    # survival over the rows that kept their pruned path (a row over the
    # capacity stops counting once past it)
    kept_scan = int(scanned_rows[~fbm].sum())
    survival = float(surv[~fbm].sum()) / kept_scan if kept_scan > 0 else None
    out = dict(metric=METRIC, value=pairs / (wall_ms / 1e3), unit="pairs/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=wall_ms, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
               config=dict(workload=f"DoSA prefill {n_q}x{n_k} causal H{H} D{D} K{K}, "
                                    f"{dp['n_seeds']} cold-prior seeds, {kept} kept heads"
                                    f"{' (structured heads)' if 'structured' in args.workload else ''}",
                           pairs_per_step=pairs),
               roofline=dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                             frac=ach / PEAK_BF16_TFLOPS, traffic=None,
                             kernel="dosa_prune_topk (all kernels; the method's own head-key "
                                    "dots, 2 D flop each)", algo_flops=alg_flops),
               dosa=dict(ms=per["dosa"], unpruned_ms=per_u["unpruned"],
                         speedup_vs_unpruned=per_u["unpruned"] / per["dosa"],
                         bit_identical_to_unpruned=equal,
                         survival_of_pruned_rows=survival,
                         fallback_rows=int(fb.sum()), head_dots=alg_dots,
                         dense_head_dots=pairs * H,
                         shared_streams=dict(ms=per_g["groups"], survivors_shared=shared_n,
                                             bit_identical_to_unpruned=eq_g)))
    return out


def bench_topk_lengths(args):
    """The top-K stage (rows_topk, K = 2048) on 8192 rows of N(0, 9) scores
    with every row of one length, for several lengths, and with the causal
    prefill's lengths 1..8192: how its time splits into a per-row part that
    does not depend on the length and one that does."""
    import numpy as np
    import torch

    import sparse_attention_indexer_02_amd as si
    R, N, K = 8192, 8192, 2048
    dev = torch.device("cuda", 0)
    g = torch.Generator(device="cpu").manual_seed(0)
    scores = (torch.randn((R, N), generator=g) * 3.0).to(dev)
    out = torch.empty((R, K), dtype=torch.int32, device=dev)
    cases = [("causal 1..8192", torch.arange(1, R + 1, dtype=torch.int32))]
    cases += [(f"all rows {n}", torch.full((R,), n, dtype=torch.int32))
              for n in (256, 1024, 2048, 4096, 6144, 8192)]
    res = {}
    for name, vis in cases:
        vis = vis.to(dev)
        _, per = timed_steps([("topk", lambda: si.rows_topk(scores, vis, K, out_idx=out,
                                                            want_scores=False))],
                             args.steps, args.warmup)
        res[name] = per["topk"]
    # reference: torch.topk (sorted) on the same full-length rows
    vals = torch.empty((R, K), dtype=torch.float32, device=dev)
    idx = torch.empty((R, K), dtype=torch.int64, device=dev)
    _, per = timed_steps([("ref", lambda: torch.topk(scores, K, dim=1, sorted=True,
                                                     out=(vals, idx)))], args.steps, args.warmup)
    return dict(metric="top-K stage time by row length (8192 rows, K 2048)", unit="ms",
                ms=res, torch_topk_all_rows_8192_ms=per["ref"], n_gpus=1, steps=args.steps,
                warmup=args.warmup, data="synthetic", higher_is_better=False)


def bench_mfma_ref(args):
    """The MFMA rate a vendor library reaches on this machine: bf16 GEMMs
    through torch.matmul (hipBLASLt), large and square, so the score
    kernel's fraction of the published peak can be read against what a
    plain GEMM attains under the same power and clock limits."""
    import torch
    dev = torch.device("cuda", 0)
    res = {}
    for n in (4096, 8192, 16384):
        g = torch.Generator(device="cpu").manual_seed(n)
        a = torch.randn((n, n), generator=g).to(dev, torch.bfloat16)
        b = torch.randn((n, n), generator=g).to(dev, torch.bfloat16)
        c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
        steps = max(3, args.steps // (n // 4096) ** 2)
        _, per = timed_steps([("mm", lambda: torch.matmul(a, b, out=c))], steps,
                             max(2, args.warmup // 4))
        tf = 2.0 * n ** 3 / per["mm"] / 1e9
        res[f"{n}x{n}x{n}"] = dict(ms=per["mm"], tflops=tf, frac=tf / PEAK_BF16_TFLOPS)
        del a, b, c
    return dict(metric="bf16 GEMM rate of torch.matmul (hipBLASLt)", unit="TFLOP/s",
                gemms=res, peak=PEAK_BF16_TFLOPS, n_gpus=1, data="synthetic",
                higher_is_better=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "decode", "dosa", "dosa_structured", "block",
                             "topk_lengths", "mfma_ref"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB (outside "
                         "the timed region) so HBM byte counters can be scaled against it")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps(dict(metric=METRIC, error="only one GPU is measured: the path runs "
                              "on a single device and no multi-GPU sharding is implemented",
                              n_gpus=args.gpus)))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst
    import synth
    if args.workload == "block":
        out = bench_block(args)
    elif args.workload == "topk_lengths":
        out = bench_topk_lengths(args)
    elif args.workload == "mfma_ref":
        out = bench_mfma_ref(args)
    elif args.workload in ("dosa", "dosa_structured"):
        out = bench_dosa(args)
    else:
        log(f"generating {args.workload} inputs")
        cfg = synth.prefill() if args.workload == "prefill" else synth.decode()
        out = bench_indexer(args, cfg, args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
