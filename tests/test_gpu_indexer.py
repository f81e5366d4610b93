"""GPU parity of idx_score_topk (lightning-indexer score + top-K) against the
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_inputs, full_config, run_idx, say
from parity import check_topk_row, oracle_check_rows

pytestmark = pytest.mark.gpu


def _compare(orc, cfg, gi, gs, rows):
    kp = orc.problem(cfg)
    oi, os_, S, M, N = orc.idx_score_topk_rows(kp, rows, want_rows=True)
    ndiff = 0
    for n, r in enumerate(rows):
        v = orc.visible(kp, int(r))
        ndiff += check_topk_row(gi[r], None if gs is None else gs[r], S[n, :v], M[n, :v],
                                N[n, :v], cfg["topk"], where=f"{cfg['name']} row {r}")
    return ndiff


def _all_rows(orc, cfg):
    say(f"{cfg['name']} n_q={cfg['n_q']} H={cfg['H']} D={cfg['D']} K={cfg['topk']}")
    gi, gs = run_idx(cfg)
    return _compare(orc, cfg, gi, gs, list(range(cfg["n_q"])))


def test_tiny_fp32(orc):
    """The tiny fp32 configuration (H4 D16): the fp32 MFMA score kernel."""
    _all_rows(orc, synth.tiny())


@pytest.mark.parametrize("n_q,L,H,D,K", [(9, 301, 5, 24, 40), (37, 700, 40, 64, 100),
                                         (20, 180, 64, 2, 33)])
def test_fp32_mfma_shapes(orc, n_q, L, H, D, K):
    """fp32 MFMA tiles with padded head rows (H 5, 40 -> two head tiles, 64),
    D from 2 up, ragged causal rows with a partial last tile."""
    _all_rows(orc, synth.tiny(seed=n_q, n_q=n_q, L=L, H=H, D=D, topk=K))


def test_fp32_mfma_row_offsets(orc):
    """fp32 per-row keys (row offsets, ragged lengths) through the fp32 MFMA
    kernel's rotated (rows x tiles) grid."""
    cfg = synth.tiny(seed=21, n_q=12, L=900, H=8, D=32, topk=64)
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 400, cfg["n_q"]).astype(np.int32)
    cfg["k_row_offset"] = (np.cumsum(lens) - lens).astype(np.int64)
    cfg["k"] = rng.standard_normal((int(lens.sum()), cfg["D"]), dtype=np.float32)
    cfg["n_k"] = int(lens.sum())
    cfg["vis_len"] = lens
    cfg["max_vis"] = int(lens.max())
    cfg["name"] = "fp32 row offsets"
    _all_rows(orc, cfg)


def test_generic_fp32_odd_shape(orc):
    """Odd D stays on the generic VALU kernel."""
    _all_rows(orc, synth.tiny(seed=3, n_q=9, L=301, H=5, D=23, topk=40))


@pytest.mark.parametrize("n_q,L,H,D,K", [(300, 700, 64, 128, 128), (600, 600, 64, 128, 512),
                                         (200, 333, 32, 128, 64), (97, 257, 40, 64, 300),
                                         (64, 1000, 64, 64, 2048)])
def test_prefill_small(orc, n_q, L, H, D, K):
    _all_rows(orc, synth.prefill(seed=n_q, n_q=n_q, L=L, H=H, D=D, topk=K))


@pytest.mark.parametrize("n_q,L,H,D,K", [(96, 12500, 32, 128, 512), (48, 20000, 64, 64, 1024)])
def test_prefill_key_segments(orc, n_q, L, H, D, K):
    """Shared keys beyond 2 MiB are scored in 1 MiB key segments (4 and 3
    segments here, the last one ragged); every row against the oracle."""
    _all_rows(orc, synth.prefill(seed=L, n_q=n_q, L=L, H=H, D=D, topk=K))


def test_shared_weights(orc):
    cfg = synth.prefill(seed=5, n_q=128, L=400, H=64, D=128, topk=100)
    cfg["w"] = np.ascontiguousarray(cfg["w"][0])
    cfg["w_row_stride"] = 0
    _all_rows(orc, cfg)


def test_bf16_keys_with_row_offsets(orc):
    cfg = synth.decode(seed=6, rows=10, max_len=2500, H=64, D=128, topk=300)
    # same rows with bf16 keys: decode the fp8 keys with their scales
    kf = np.array([orc.e4m3fn_to_double(b) for b in range(256)])[cfg["k"]] * cfg["k_scale"][:, None]
    cfg["k"] = synth.f32_to_bf16_bits(kf.astype(np.float32))
    cfg["k_dtype"] = synth.BF16
    cfg["k_scale"] = None
    _all_rows(orc, cfg)


@pytest.mark.parametrize("H,D", [(64, 128), (32, 128), (64, 64)])
def test_decode_fp8_small(orc, H, D):
    _all_rows(orc, synth.decode(seed=H + D, rows=12, max_len=3000, H=H, D=D, topk=256))


def test_integer_inputs_exact(orc):
    """Integer-valued bf16 q/k and dyadic weights: every partial sum is an
    exact fp32 integer, so GPU scores equal the oracle's bit for bit and the
    id lists match exactly, ties included."""
    rng = np.random.default_rng(12)
    n_q, L, H, D, K = 96, 300, 64, 128, 64
    q = rng.integers(-3, 4, (n_q, H, D)).astype(np.float32)
    k = rng.integers(-3, 4, (L, D)).astype(np.float32)
    k[rng.random((L, D)) < 0.7] = 0  # sparse keys: many exact score ties
    w = rng.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], (n_q, H)).astype(np.float32)
    cfg = dict(name="integer", q=synth.f32_to_bf16_bits(q), q_dtype=synth.BF16,
               k=synth.f32_to_bf16_bits(k), k_dtype=synth.BF16, k_scale=None, w=w,
               k_row_offset=None, vis_len=(L - n_q + 1 + np.arange(n_q)).astype(np.int32),
               n_q=n_q, H=H, D=D, n_k=L, max_vis=L, topk=K)
    say("integer-valued inputs")
    gi, gs = run_idx(cfg)
    kp = orc.problem(cfg)
    oi, os_ = orc.idx_score_topk_rows(kp, list(range(n_q)))
    np.testing.assert_array_equal(gi, oi)
    np.testing.assert_array_equal(gs.astype(np.float64), os_)


def test_edges(orc):
    """Empty rows, rows shorter than K, vis_len beyond max_vis (clamped), K > n_k."""
    cfg = synth.prefill(seed=7, n_q=8, L=50, H=64, D=128, topk=64)
    cfg["vis_len"] = np.array([0, 1, 2, 49, 50, 50, 7, 0], np.int32)
    _all_rows(orc, cfg)
    cfg2 = synth.tiny(seed=8, n_q=4, L=30, H=3, D=8, topk=40)
    cfg2["vis_len"] = np.array([0, 30, 31, 1000], np.int32)  # last two clamp to 30
    _all_rows(orc, cfg2)


def test_deterministic(orc):
    cfg = synth.prefill(seed=9, n_q=256, L=900, H=64, D=128, topk=256)
    say("determinism")
    a = run_idx(cfg)
    b = run_idx(cfg)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_prefill_full_size_all_rows(orc):
    """The 8192 x 8192, H64 D128 K2048 prefill in the benchmark's launch
    configuration: every row against the oracle."""
    cfg = full_config("prefill")
    say("prefill full size, all 8192 rows against the oracle")
    gi, gs = run_idx(cfg)
    ndiff = oracle_check_rows(orc, cfg, gi, gs, where="prefill full")
    say(f"prefill full size: {ndiff} rows differ from the oracle within the near-K-th rule")


def test_decode_full_size_all_rows(orc):
    """128 ragged rows up to 131072 fp8 keys (chunked top-K levels): every row
    against the oracle."""
    cfg = full_config("decode")
    say(f"decode full size, sum L = {cfg['n_k']}, all rows against the oracle")
    gi, gs = run_idx(cfg)
    ndiff = oracle_check_rows(orc, cfg, gi, gs, chunk=32, where="decode full")
    say(f"decode full size: {ndiff} rows differ from the oracle within the near-K-th rule")
