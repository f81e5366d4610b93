"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only draws random numbers and packs them into the storage types
the library consumes (bf16 as uint16 bit patterns, OCP fp8 e4m3fn as bytes).
It holds none of the indexer's arithmetic: no scores, no selection, no
segment maps.  Both sides read the exact same bytes from here.

Workloads follow the shapes of the pages' settings:

* "tiny"      - 8 queries over 256 causal keys, H=4, D=16, fp32, K=16.
* "prefill"   - DSA-style causal prefill, H=64, D=128, bf16, K=2048, with 1%
                salient keys scaled by 4 (lightning-indexer setting of the
                DoSA notes, section 4: H32/H64, D128, K2048).
* "decode"    - ragged rows with their own keys, fp8 e4m3fn keys with a
                per-token fp32 scale, bf16 queries, K=2048.
* "dosa"      - causal prefill chunk at the end of a long context, H=32.
* "dosa_structured" - same shapes, heads built from 4 shared directions so
                that anchors and negative aggregation actually bite.
* "block"     - MiniMax-M3 block-sparse selection inputs (128-token blocks,
                32 blocks per query, 1 init + 2 local), fp32.

Every generator accepts size overrides so that the same recipe produces the
small cases the oracle finishes in seconds.
"""
from __future__ import annotations

import numpy as np

F32, BF16, FP8_E4M3FN = 0, 1, 2  # storage tags, same numbering as the C ABI


def _streams(seed: int, n: int):
    """Independent PCG64 streams, one per tensor."""
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 storage (uint16).  Inputs finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_e4m3fn_bytes(x: np.ndarray) -> np.ndarray:
    """Storage conversion to OCP fp8 e4m3fn bytes (torch's CPU cast, RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _signed_weights(g, shape, neg_frac=0.3):
    """|w| ~ U[0,1], negative with probability neg_frac, iid per entry."""
    mag = g.random(shape, dtype=np.float32)
    neg = g.random(shape) < neg_frac
    return np.where(neg, -mag, mag).astype(np.float32)


def tiny(seed: int = 0, n_q: int = 8, L: int = 256, H: int = 4, D: int = 16, topk: int = 16):
    gq, gk, gw = _streams(seed, 3)
    q = gq.standard_normal((n_q, H, D), dtype=np.float32)
    k = gk.standard_normal((L, D), dtype=np.float32)
    w = gw.uniform(-1.0, 1.0, (n_q, H)).astype(np.float32)
    vis = (L - n_q + 1 + np.arange(n_q)).astype(np.int32)
    return dict(name="tiny", q=q, q_dtype=F32, k=k, k_dtype=F32, k_scale=None, w=w,
                k_row_offset=None, vis_len=vis, n_q=n_q, H=H, D=D, n_k=L, max_vis=L,
                topk=topk, witness=dict(S=4, keep=topk - 4, max_rep=4))


def prefill(seed: int = 0, n_q: int = 8192, L: int = 8192, H: int = 64, D: int = 128,
            topk: int = 2048, salient_frac: float = 0.01, salient_scale: float = 4.0,
            S: int = 16, neg_frac: float = 0.3):
    """Causal prefill chunk: query i sits at position L - n_q + i."""
    gq, gk, gw, gs = _streams(seed, 4)
    q = f32_to_bf16_bits(gq.standard_normal((n_q, H, D), dtype=np.float32))
    kf = gk.standard_normal((L, D), dtype=np.float32)
    n_sal = int(round(salient_frac * L))
    if n_sal:
        rows = gs.choice(L, size=n_sal, replace=False)
        kf[rows] *= np.float32(salient_scale)
    k = f32_to_bf16_bits(kf)
    w = _signed_weights(gw, (n_q, H), neg_frac)
    vis = (L - n_q + 1 + np.arange(n_q)).astype(np.int32)
    return dict(name="prefill", q=q, q_dtype=BF16, k=k, k_dtype=BF16, k_scale=None, w=w,
                k_row_offset=None, vis_len=vis, n_q=n_q, H=H, D=D, n_k=L, max_vis=L,
                topk=topk, witness=dict(S=S, keep=max(topk - S, 0), max_rep=S))


def decode(seed: int = 0, rows: int = 128, max_len: int = 131072, H: int = 64, D: int = 128,
           topk: int = 2048, S: int = 64, lens=None, neg_frac: float = 0.3):
    """Ragged decode batch: row r owns keys [off_r, off_r + L_r), L_r ~ U{1..max_len}."""
    gl, gq, gw, gk = _streams(seed, 4)
    if lens is None:
        lens = gl.integers(1, max_len, size=rows, endpoint=True)
    lens = np.asarray(lens, dtype=np.int64)
    rows = len(lens)
    off = np.zeros(rows, dtype=np.int64)
    off[1:] = np.cumsum(lens)[:-1]
    n_k = int(lens.sum())
    kbytes = np.empty((n_k, D), dtype=np.uint8)
    kscale = np.empty(n_k, dtype=np.float32)
    key_streams = [np.random.Generator(np.random.PCG64(s))
                   for s in np.random.SeedSequence([seed, 3]).spawn(rows)]

    def fill(r):
        x = key_streams[r].standard_normal((int(lens[r]), D), dtype=np.float32)
        amax = np.max(np.abs(x), axis=1)
        sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        a, b = int(off[r]), int(off[r] + lens[r])
        kbytes[a:b] = f32_to_e4m3fn_bytes(x / sc[:, None])
        kscale[a:b] = sc

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range(rows)))
    q = f32_to_bf16_bits(gq.standard_normal((rows, H, D), dtype=np.float32))
    w = _signed_weights(gw, (rows, H), neg_frac)
    return dict(name="decode", q=q, q_dtype=BF16, k=kbytes, k_dtype=FP8_E4M3FN, k_scale=kscale,
                w=w, k_row_offset=off, vis_len=lens.astype(np.int32), n_q=rows, H=H, D=D,
                n_k=n_k, max_vis=int(lens.max()), topk=topk,
                witness=dict(S=S, keep=max(topk - S, 0), max_rep=S))


def dosa(seed: int = 0, n_q: int = 4096, L: int = 32768, H: int = 32, D: int = 128,
         topk: int = 2048, n_seeds: int = 12288, n_rep: int = 4, rep_topk: int = 2048,
         kept_heads: int = 16, neg_active_frac: float = 0.5):
    """Prefill chunk of n_q queries at the end of an L-key context (prefill recipe)."""
    c = prefill(seed=seed, n_q=n_q, L=L, H=H, D=D, topk=topk)
    c["name"] = "dosa"
    c["dosa"] = dict(n_seeds=n_seeds, n_rep_queries=n_rep, rep_topk=rep_topk,
                     kept_heads=kept_heads, neg_active_frac=neg_active_frac)
    return c


def dosa_structured(seed: int = 0, n_q: int = 4096, L: int = 32768, H: int = 32, D: int = 128,
                    topk: int = 2048, n_seeds: int = 12288, n_rep: int = 4, rep_topk: int = 2048,
                    kept_heads: int = 16, neg_active_frac: float = 0.5, groups: int = 4,
                    noise: float = 0.1):
    """Heads of a query share `groups` base directions; the last group is negative.

    q[r,h] = b[r, h mod groups] + noise * eps[r,h]; |w| ~ U[0,1], sign - for
    group groups-1, + otherwise.  Keys follow the prefill recipe.
    """
    c = dosa(seed=seed, n_q=n_q, L=L, H=H, D=D, topk=topk, n_seeds=n_seeds, n_rep=n_rep,
             rep_topk=rep_topk, kept_heads=kept_heads, neg_active_frac=neg_active_frac)
    gb, ge, gw = _streams(seed + 1000, 3)
    base = gb.standard_normal((n_q, groups, D), dtype=np.float32)
    eps = ge.standard_normal((n_q, H, D), dtype=np.float32)
    grp = np.arange(H) % groups
    qf = base[:, grp, :] + np.float32(noise) * eps
    c["q"] = f32_to_bf16_bits(qf)
    mag = gw.random((n_q, H), dtype=np.float32)
    sign = np.where(grp == groups - 1, -1.0, 1.0).astype(np.float32)
    c["w"] = (mag * sign[None, :]).astype(np.float32)
    c["name"] = "dosa_structured"
    return c


def block(seed: int = 0, n_q: int = 4096, n_pos: int = 131072, H: int = 8, D: int = 128,
          block_size: int = 128, top_blocks: int = 32, init_blocks: int = 1,
          local_blocks: int = 2, query_pos=None):
    """Block-sparse selection inputs; default query j sits at position (j+1)*n_pos/n_q - 1."""
    gq, gk = _streams(seed, 2)
    q = gq.standard_normal((n_q, H, D), dtype=np.float32)
    k = gk.standard_normal((n_pos, D), dtype=np.float32)
    if query_pos is None:
        stride = n_pos // n_q
        query_pos = stride * np.arange(n_q, dtype=np.int64) + (stride - 1)
    query_pos = np.asarray(query_pos, dtype=np.int64)
    return dict(name="block", q=q, k=k, query_pos=query_pos, n_q=len(query_pos), H=H, D=D,
                n_pos=n_pos, block_size=block_size, top_blocks=top_blocks,
                init_blocks=init_blocks, local_blocks=local_blocks,
                out_width=max(top_blocks, init_blocks + local_blocks))


def witness_rows(seed: int = 0, rows: int = 64, topk: int = 64, max_len: int = 300,
                 pad_frac: float = 0.2, oob_frac: float = 0.02, neg_len_frac: float = 0.05):
    """Random learned rows for the witness merge: distinct in-range ids, some -1
    padding, a few out-of-range entries and a few non-positive context lengths."""
    g = _streams(seed, 1)[0]
    lens = g.integers(1, max_len, size=rows, endpoint=True).astype(np.int32)
    bad = g.random(rows) < neg_len_frac
    lens[bad] = -g.integers(0, 3, size=int(bad.sum()))
    out = np.full((rows, topk), -1, dtype=np.int32)
    for r in range(rows):
        L = int(lens[r])
        if L <= 0:
            continue
        n = min(topk, L)
        ids = g.choice(L, size=n, replace=False).astype(np.int32)
        row = np.full(topk, -1, dtype=np.int32)
        row[:n] = ids
        pad = g.random(topk) < pad_frac
        row[pad] = -1
        oob = g.random(topk) < oob_frac
        row[oob] = L + g.integers(0, 4 * L + 1, size=int(oob.sum()))
        out[r] = row
    return out, lens


def block_lists(seed: int = 0, n_q: int = 4096, H: int = 8, n_pos: int = 131072,
                block_size: int = 128, top_blocks: int = 32, init_blocks: int = 1,
                local_blocks: int = 2, query_pos=None, messy: bool = False):
    """Block lists shaped like a selection: per (query, KV head), the forced first and last
    blocks plus random others up to the budget, ascending, -1 padded to the selection width.
    messy: shuffled, with repeats, out-of-range blocks and padding in the middle."""
    g = _streams(seed, 1)[0]
    if query_pos is None:
        stride = n_pos // n_q
        query_pos = stride * np.arange(n_q, dtype=np.int64) + (stride - 1)
    query_pos = np.asarray(query_pos, dtype=np.int64)
    width = max(top_blocks, init_blocks + local_blocks, 1)
    out = np.full((len(query_pos), H, width), -1, dtype=np.int32)
    nb_all = -(-n_pos // block_size)
    for q, p in enumerate(query_pos):
        n = 0 if p < 0 else min(int(p) // block_size + 1, nb_all)
        for h in range(H):
            forced = set(range(min(init_blocks, n))) | set(range(max(0, n - local_blocks), n))
            budget = max(top_blocks, len(forced))
            rest = np.setdiff1d(np.arange(n), np.fromiter(forced, int, len(forced)))
            extra = g.choice(rest, size=min(budget - len(forced), len(rest)), replace=False)
            sel = np.sort(np.concatenate([np.fromiter(forced, int, len(forced)), extra]))
            row = np.full(width, -1, dtype=np.int32)
            row[:len(sel)] = sel
            if messy:
                k = int(g.integers(0, width + 1))
                row[g.integers(0, width, size=k // 2)] = g.integers(-3, nb_all + 4, size=k // 2)
                row = g.permutation(row)
            out[q, h] = row
    return out, query_pos


def kv_layout(seed: int, lens, page_size: int = 128, spare_pages: int = 2):
    """KV placement of ragged rows: flat starts (rows back to back) and a page table
    of shuffled physical pages (-1 for the spare, unallocated table entries)."""
    g = _streams(seed, 1)[0]
    lens = np.asarray(lens, dtype=np.int64)
    starts = np.zeros(len(lens), dtype=np.int64)
    starts[1:] = np.cumsum(lens)[:-1]
    pages = -(-np.maximum(lens, 0) // page_size)
    ppr = int(pages.max()) + spare_pages if len(lens) else 1
    phys = g.permutation(int(pages.sum()) + 7).astype(np.int32)
    table = np.full((len(lens), ppr), -1, dtype=np.int32)
    at = 0
    for r, n in enumerate(pages):
        table[r, :n] = phys[at:at + n]
        at += n
    return starts, table
