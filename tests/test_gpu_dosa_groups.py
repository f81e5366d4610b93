"""GPU parity of dosa_prune_topk with 4-query shared streams (the DoSA
reading notes' section 4 compaction and rescoring variant): bit-identical
(ids and scores) to the unpruned top-K, with the same survivors as per-row
streams, and within the score tolerance of the oracle."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_inputs, full_config, say
from test_gpu_dosa import _assert_bit_exact, _oracle_rows, _run_both, _small

pytestmark = pytest.mark.gpu


def _both_modes(cfg, **kw):
    ui, us, di, ds, st = _run_both(cfg, shared_streams=True, **kw)
    _, _, pi, ps, pst = _run_both(cfg, shared_streams=False, **kw)
    _assert_bit_exact(ui, us, di, ds)
    _assert_bit_exact(ui, us, pi, ps)
    return ui, us, di, ds, st, pst


@pytest.mark.parametrize("structured", [False, True])
@pytest.mark.parametrize("H,D,n_q", [(32, 128, 48), (64, 128, 47), (32, 64, 45), (20, 128, 46)])
def test_groups_small(orc, structured, H, D, n_q):
    """Group counts not a multiple of 4 leave a short last group."""
    cfg = _small(structured, seed=H + D + n_q, n_q=n_q, H=H, D=D, kept=min(16, H - 1))
    say(f"dosa groups structured={structured} H={H} D={D} n_q={n_q}")
    ui, us, di, ds, st, pst = _both_modes(cfg)
    np.testing.assert_array_equal(st["n_survivors"], pst["n_survivors"])
    np.testing.assert_array_equal(st["fallback"], pst["fallback"])
    assert np.all(st["n_shared"] <= st["n_survivors"])
    assert np.all(pst["n_shared"] == 0)
    if structured:
        assert st["n_shared"].sum() > 0, "no key reached a shared stream"
    _oracle_rows(orc, cfg, di, ds, list(range(0, n_q, 5)))


def test_groups_integer_ties(orc):
    rng = np.random.default_rng(23)
    n_q, L, H, D, K = 42, 400, 32, 128, 48
    q = rng.integers(-2, 3, (n_q, H, D)).astype(np.float32)
    q[:, 8:] = q[:, :8].repeat(3, axis=1)[:, :H - 8]
    k = rng.integers(-2, 3, (L, D)).astype(np.float32)
    k[rng.random((L, D)) < 0.8] = 0
    w = rng.choice([-1.0, -0.5, 0.5, 1.0], (n_q, H)).astype(np.float32)
    cfg = dict(name="dosa-int", q=synth.f32_to_bf16_bits(q), q_dtype=synth.BF16,
               k=synth.f32_to_bf16_bits(k), k_dtype=synth.BF16, k_scale=None, w=w,
               k_row_offset=None, vis_len=(L - n_q + 1 + np.arange(n_q)).astype(np.int32),
               n_q=n_q, H=H, D=D, n_k=L, max_vis=L, topk=K,
               dosa=dict(n_seeds=120, n_rep_queries=3, rep_topk=K, kept_heads=8,
                         neg_active_frac=0.5))
    say("dosa groups integer ties")
    ui, us, di, ds, st, _ = _both_modes(cfg)
    kp = orc.problem(cfg)
    oi, os_ = orc.idx_score_topk_rows(kp, list(range(n_q)))
    np.testing.assert_array_equal(di, oi)
    np.testing.assert_array_equal(ds.astype(np.float64), os_)


@pytest.mark.parametrize("cap", [1, 40, 120])
def test_groups_capacity(cap):
    """Rows whose shared + solo streams pass the capacity take the exact
    path (at 1 every row with a survivor does)."""
    cfg = _small(True, seed=11)
    say(f"dosa groups capacity {cap}")
    ui, us, di, ds, st, _ = _both_modes(cfg, survivor_capacity=cap)
    if cap == 1:
        assert st["fallback"].sum() > 0


def test_groups_fallback_and_prior():
    cfg = _small(True, seed=12)
    c = int(cfg["vis_len"].min())
    seeds = np.sort(np.random.default_rng(3).choice(c, 256, replace=False)).astype(np.int32)
    say("dosa groups caller prior, global fallback")
    _, _, _, _, st, _ = _both_modes(cfg, seed_ids=torch.from_numpy(seeds).cuda())
    assert np.all(st["fallback"] == 0)
    cfg["vis_len"] = cfg["vis_len"].copy()
    cfg["vis_len"][3] = 100
    _, _, _, _, st, _ = _both_modes(cfg)
    assert np.all(st["fallback"] == 1) and np.all(st["n_shared"] == 0)


def test_groups_full_size(orc):
    """The structured-head 4096 x 32768 workload with shared streams."""
    cfg = full_config("dosa_structured")
    say("dosa groups full size")
    ui, us, di, ds, st = _run_both(cfg, shared_streams=True)
    _assert_bit_exact(ui, us, di, ds)
    _oracle_rows(orc, cfg, di, ds, [0, 3, 2048, 4095])
    say(f"survivors {st['n_survivors'].clip(0).sum()}, through shared streams "
        f"{st['n_shared'].sum()}, fallback rows {st['fallback'].sum()}")
