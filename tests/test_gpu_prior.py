"""GPU parity of idx_score_topk_prior (the decode path with a threshold from
recently selected keys): its ids and scores equal idx_score_topk's bit for
bit for any prior, and they match the oracle on sampled rows."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_inputs, full_config, say
from parity import oracle_check_rows

pytestmark = pytest.mark.gpu


def _plain(d, cfg):
    import sparse_attention_indexer_02_amd as si
    return si.idx_score_topk(d["q"], d["k"], d["w"], d["vis_len"], cfg["topk"],
                             k_scale=d["k_scale"], k_row_offset=d["k_row_offset"],
                             max_vis=cfg["max_vis"])


def _prior(d, cfg, prior):
    import sparse_attention_indexer_02_amd as si
    return si.idx_score_topk_prior(d["q"], d["k"], d["w"], d["vis_len"], cfg["topk"], prior,
                                   k_scale=d["k_scale"], k_row_offset=d["k_row_offset"],
                                   max_vis=cfg["max_vis"], want_stats=True)


def _perturbed_prior(d, cfg, eps, seed):
    """The ids a slightly different query would select: a stand-in for the
    previous decode step's selection."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    qf = d["q"].float()
    noise = torch.randn(qf.shape, generator=g).to(qf.device)
    d2 = dict(d, q=(qf + eps * noise).to(torch.bfloat16).contiguous())
    ids, _ = _plain(d2, cfg)
    return ids


def _check_equal(d, cfg, prior, what):
    say(f"prior path: {what}")
    ui, us = _plain(d, cfg)
    pi, ps, (tau, surv) = _prior(d, cfg, prior)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pi.cpu().numpy(), ui.cpu().numpy(), err_msg=what)
    np.testing.assert_array_equal(ps.cpu().numpy().view(np.uint32), us.cpu().numpy().view(np.uint32),
                                  err_msg=what)
    # tau is a lower bound of each full row's K-th score; every selected key survived
    us_np, tau_np, surv_np = us.cpu().numpy(), tau.cpu().numpy(), surv.cpu().numpy()
    vis = np.minimum(cfg["vis_len"], cfg["max_vis"])
    K = cfg["topk"]
    for r in range(cfg["n_q"]):
        if vis[r] >= K:
            assert tau_np[r] <= us_np[r, K - 1], (what, r)
        assert surv_np[r] >= min(K, vis[r]), (what, r)
    return ui.cpu().numpy(), us_np, surv_np


def _decode(seed, rows=12, max_len=3000, H=64, D=128, K=256, bf16_keys=False, orc=None):
    cfg = synth.decode(seed=seed, rows=rows, max_len=max_len, H=H, D=D, topk=K)
    if bf16_keys:
        kf = np.array([orc.e4m3fn_to_double(b) for b in range(256)])[cfg["k"]] * cfg["k_scale"][:, None]
        cfg["k"] = synth.f32_to_bf16_bits(kf.astype(np.float32))
        cfg["k_dtype"] = synth.BF16
        cfg["k_scale"] = None
    return cfg


@pytest.mark.parametrize("H,D", [(64, 128), (32, 128), (64, 64)])
def test_priors_small_fp8(orc, H, D):
    cfg = _decode(seed=H + D, H=H, D=D)
    d = dev_inputs(cfg)
    n_q, K = cfg["n_q"], cfg["topk"]
    exact, _ = _plain(d, cfg)
    _check_equal(d, cfg, exact, "the exact ids")
    _check_equal(d, cfg, _perturbed_prior(d, cfg, 0.3, 1), "a perturbed query's ids")
    rng = np.random.default_rng(H * D)
    rnd = torch.from_numpy(rng.integers(-50, 4000, (n_q, K), dtype=np.int32)).cuda()
    _check_equal(d, cfg, rnd, "random ids, some out of range")
    dup = torch.full((n_q, K), 3, dtype=torch.int32, device="cuda")
    _check_equal(d, cfg, dup, "one id repeated (fewer than K distinct)")
    none = torch.full((n_q, 5), -1, dtype=torch.int32, device="cuda")
    _check_equal(d, cfg, none, "an empty prior narrower than K")
    wide = torch.cat([exact, exact.flip(1), rnd], dim=1)[:, :2048].contiguous()
    _check_equal(d, cfg, wide, "a prior wider than K with repeats")


def test_prior_bf16_keys(orc):
    cfg = _decode(seed=6, rows=10, max_len=2500, K=300, bf16_keys=True, orc=orc)
    d = dev_inputs(cfg)
    _check_equal(d, cfg, _perturbed_prior(d, cfg, 0.3, 2), "bf16 keys, perturbed prior")


def test_prior_integer_ties(orc):
    """Integer-valued keys and queries: many exact score ties at the K-th
    place; survivors at the threshold must still be taken by lower key."""
    rng = np.random.default_rng(21)
    rows, H, D, K = 8, 64, 128, 64
    lens = rng.integers(100, 3000, rows)
    off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    n_k = int(lens.sum())
    q = rng.integers(-2, 3, (rows, H, D)).astype(np.float32)
    k = rng.integers(-2, 3, (n_k, D)).astype(np.float32)
    k[rng.random((n_k, D)) < 0.8] = 0
    w = rng.choice([-1.0, 0.5, 1.0, 2.0], (rows, H)).astype(np.float32)
    cfg = dict(name="ties", q=synth.f32_to_bf16_bits(q), q_dtype=synth.BF16,
               k=synth.f32_to_bf16_bits(k), k_dtype=synth.BF16, k_scale=None, w=w,
               k_row_offset=off, vis_len=lens.astype(np.int32), n_q=rows, H=H, D=D, n_k=n_k,
               max_vis=int(lens.max()), topk=K)
    d = dev_inputs(cfg)
    exact, _ = _plain(d, cfg)
    _check_equal(d, cfg, exact, "integer ties, exact prior")
    _check_equal(d, cfg, exact[:, K // 2:].contiguous(), "integer ties, half the ids")


def test_prior_overflow_rows(orc):
    """Long rows with a prior that keeps far more than 8192 keys take the
    chunked selection over all survivors; others the single-workgroup one."""
    cfg = _decode(seed=31, rows=6, max_len=40000, K=512)
    d = dev_inputs(cfg)
    weak = torch.arange(512, dtype=torch.int32, device="cuda").repeat(cfg["n_q"], 1)
    _, _, surv = _check_equal(d, cfg, weak.contiguous(), "first 512 keys as the prior")
    say(f"survivors {surv.tolist()} of {cfg['vis_len'].tolist()}")


def test_prior_full_size(orc):
    """128 ragged rows up to 131072 fp8 keys with a perturbed-query prior:
    equal to idx_score_topk; every row against the oracle."""
    cfg = full_config("decode")
    d = dev_inputs(cfg)
    prior = _perturbed_prior(d, cfg, 0.3, 3)
    ui, us, surv = _check_equal(d, cfg, prior, "full-size decode, perturbed prior")
    say(f"survivors {int(surv.sum())} of {int(np.minimum(cfg['vis_len'], cfg['max_vis']).sum())}")
    ndiff = oracle_check_rows(orc, cfg, ui, us, chunk=32, where="prior full-size")
    say(f"prior full size: every row against the oracle, {ndiff} differ within the near-K-th rule")


@pytest.mark.parametrize("lens", [[0, 3000, 1, 9000], [0, 600000, 5000, 1]])
def test_prior_empty_and_long_rows(orc, lens):
    """An empty row, a one-key row, and (second case) a row longer than the
    per-row LDS bitmap of prior ids covers, which takes the one-workgroup
    threshold kernel."""
    cfg = synth.decode(seed=41, lens=lens, topk=256)
    d = dev_inputs(cfg)
    _check_equal(d, cfg, _perturbed_prior(d, cfg, 0.3, 4), "empty and long rows, perturbed prior")
    exact, _ = _plain(d, cfg)
    _check_equal(d, cfg, exact, "empty and long rows, exact prior")


def test_prior_large_k(orc):
    """K above the block top-K's 2048: every prior is narrower than K, so
    tau is -inf and the radix select takes every row through the candidate
    id map."""
    cfg = _decode(seed=51, rows=6, max_len=9000, K=3000)
    d = dev_inputs(cfg)
    exact, _ = _plain(d, cfg)
    _check_equal(d, cfg, exact[:, :2048].contiguous(), "K 3000, the first 2048 exact ids")
