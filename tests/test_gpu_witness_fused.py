"""GPU parity of idx_score_topk_witness (the witness merge done by the top-K
kernel as it writes each row): bit-identical to idx_score_topk followed by
kvwitness_merge, which the witness tests pin to the oracle."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_inputs, full_config, say
from parity import oracle_check_rows

pytestmark = pytest.mark.gpu


def _both(d, cfg, lens, S, keep, B, K=None, max_vis=None):
    import sparse_attention_indexer_02_amd as si
    K = K or cfg["topk"]
    mv = max_vis or cfg["max_vis"]
    kw = dict(k_scale=d["k_scale"], k_row_offset=d["k_row_offset"], max_vis=mv)
    ui, us = si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], K, **kw)
    si.kvwitness_merge(ui, lens, S, keep, B)
    fi, fs = si.idx_score_topk_witness(d["q"], d["k"], d["w"], d["vis_len"], K, lens, S,
                                       keep=keep, max_replacements=B, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fi.cpu().numpy(), ui.cpu().numpy())
    np.testing.assert_array_equal(fs.cpu().numpy().view(np.uint32), us.cpu().numpy().view(np.uint32))
    return fi.cpu().numpy()


def _lens(d, shift=0):
    v = d["vis_len"].clone()
    return (v + shift).contiguous()


@pytest.mark.parametrize("S", [1, 4, 16, 64])
def test_fused_prefill_small(S):
    cfg = synth.prefill(seed=S, n_q=96, L=700, H=64, D=128, topk=128, S=S)
    d = dev_inputs(cfg)
    say(f"fused witness prefill S={S}")
    K = cfg["topk"]
    _both(d, cfg, _lens(d), S, max(K - S, 0), S)
    _both(d, cfg, _lens(d), S, 0, 7)        # witnesses at the front of the row
    _both(d, cfg, _lens(d), S, K - 2, 100)  # budget clipped to K - keep


def test_fused_decode_levels():
    """fp8 per-row keys with rows past 8192 (chunk levels; the merge runs in
    the last one)."""
    cfg = synth.decode(seed=3, rows=10, max_len=30000, topk=512)
    d = dev_inputs(cfg)
    say("fused witness decode levels")
    _both(d, cfg, _lens(d), 64, 512 - 64, 64)


def test_fused_context_lengths_differ():
    """Context lengths unlike the visible lengths: ids past L (the clamped
    segment rule), rows with no context, and rows that see no key but have a
    context (every segment takes its witness)."""
    cfg = synth.decode(seed=4, rows=12, max_len=3000, topk=256)
    d = dev_inputs(cfg)
    lens = d["vis_len"].clone()
    lens[0] = 0
    lens[1] = -3
    lens[2] = 5
    lens[3] = lens[3] // 3
    lens[4] = lens[4] + 1000
    d["vis_len"][5] = 0  # sees nothing, context kept
    say("fused witness context lengths")
    _both(d, cfg, lens.contiguous(), 16, 240, 16)


def test_fused_large_k():
    """K above the block kernel's 2048: radix-select rows, then the merge
    kernel."""
    cfg = synth.decode(seed=5, rows=6, max_len=9000, topk=3000)
    d = dev_inputs(cfg)
    say("fused witness K 3000")
    _both(d, cfg, _lens(d), 32, 3000 - 32, 32)


def _full_step_against_oracle(orc, name, chunk):
    """The timed step, idx_score_topk_witness without scores, at full size:
    its unmerged rows (idx_score_topk) are checked row by row against the
    oracle, and the step's ids must equal the oracle's witness merge applied
    to those same rows, bit for bit (both sides merge the same learned
    rows)."""
    import sparse_attention_indexer_02_amd as si
    cfg = full_config(name)
    d = dev_inputs(cfg)
    w = cfg["witness"]
    K, mv = cfg["topk"], cfg["max_vis"]
    kw = dict(k_scale=d["k_scale"], k_row_offset=d["k_row_offset"], max_vis=mv)
    say(f"fused witness full {name}: the timed call, then every row against the oracle")
    ui, us = si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], K, **kw)
    fi, _ = si.idx_score_topk_witness(d["q"], d["k"], d["w"], d["vis_len"], K, d["vis_len"],
                                      w["S"], keep=w["keep"], max_replacements=w["max_rep"],
                                      want_scores=False, **kw)
    torch.cuda.synchronize()
    ui, us, fi = ui.cpu().numpy(), us.cpu().numpy(), fi.cpu().numpy()
    ndiff = oracle_check_rows(orc, cfg, ui, us, chunk=chunk, where=f"{name} full step")
    rc, merged = orc.kvwitness_merge(ui, cfg["vis_len"], w["S"], w["keep"], w["max_rep"])
    assert rc == 0
    np.testing.assert_array_equal(fi, merged)
    changed = int((fi != ui).sum())
    say(f"{name}: {ndiff} rows differ from the oracle's top-K within the near-K-th rule; "
        f"{changed} slots hold witnesses")


def test_fused_full_prefill(orc):
    cfg = full_config("prefill")
    d = dev_inputs(cfg)
    w = cfg["witness"]
    say("fused witness full prefill")
    _both(d, cfg, _lens(d), w["S"], w["keep"], w["max_rep"])
    _full_step_against_oracle(orc, "prefill", 1024)


def test_fused_full_decode(orc):
    """The decode workload as timed: fp8 per-row keys, rows up to 131072
    (chunk levels), K2048, S64."""
    cfg = full_config("decode")
    d = dev_inputs(cfg)
    w = cfg["witness"]
    say("fused witness full decode")
    _both(d, cfg, _lens(d), w["S"], w["keep"], w["max_rep"])
    _full_step_against_oracle(orc, "decode", 32)


@pytest.mark.parametrize("S,keep,B", [(64, 100, 3), (64, 0, 64), (7, 120, 8), (1, 127, 1)])
def test_fused_budgets(S, keep, B):
    """Budgets below the empty-segment count (only the first B witnesses in
    segment order), keep far below topk - S, keep 0, and a budget past the
    row's tail (clipped to topk - keep)."""
    cfg = synth.prefill(seed=S + keep, n_q=64, L=900, H=64, D=128, topk=128, S=S)
    d = dev_inputs(cfg)
    say(f"fused witness budgets S={S} keep={keep} B={B}")
    _both(d, cfg, _lens(d), S, keep, B)


def _one_kernel_equal(cfg, S, keep, B, label):
    """idx_score_topk_fused (one kernel) against idx_score_topk_witness (score
    kernel, then top-K kernel): ids and scores bit for bit."""
    import sparse_attention_indexer_02_amd as si
    d = dev_inputs(cfg)
    K = cfg["topk"]
    lens = _lens(d)
    say(f"one-kernel prefill {label}: n_q={cfg['n_q']} L={cfg['n_k']} H={cfg['H']} "
        f"D={cfg['D']} K={K} S={S}")
    ri, rs = si.idx_score_topk_witness(d["q"], d["k"], d["w"], d["vis_len"], K, lens, S,
                                       keep=keep, max_replacements=B)
    fi, fs = si.idx_score_topk_witness(d["q"], d["k"], d["w"], d["vis_len"], K, lens, S,
                                       keep=keep, max_replacements=B, fused=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fi.cpu().numpy(), ri.cpu().numpy())
    np.testing.assert_array_equal(fs.cpu().numpy().view(np.uint32), rs.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("n_q,L,H,D,K,S", [(96, 700, 64, 128, 128, 16), (61, 500, 32, 128, 64, 4),
                                           (40, 2100, 64, 64, 300, 0), (9, 33, 20, 128, 48, 64)])
def test_one_kernel_small(n_q, L, H, D, K, S):
    cfg = synth.prefill(seed=n_q + L, n_q=n_q, L=L, H=H, D=D, topk=K, S=max(S, 1))
    _one_kernel_equal(cfg, S, max(K - S, 0), S, "small")


def test_one_kernel_full_prefill():
    cfg = full_config("prefill")
    w = cfg["witness"]
    _one_kernel_equal(cfg, w["S"], w["keep"], w["max_rep"], "full size")


def test_one_kernel_refuses_other_layouts():
    import sparse_attention_indexer_02_amd as si
    cfg = synth.decode(seed=8, rows=4, max_len=900, topk=64)
    d = dev_inputs(cfg)
    with pytest.raises(si.SparseIndexerError) as e:
        si.idx_score_topk_witness(d["q"], d["k"], d["w"], d["vis_len"], 64, _lens(d), 8,
                                  k_scale=d["k_scale"], k_row_offset=d["k_row_offset"],
                                  max_vis=cfg["max_vis"], fused=True)
    assert e.value.status == 5  # SI_ERR_UNSUPPORTED_DTYPE
