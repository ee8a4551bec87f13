"""Seeded synthetic inputs for MSA prefill (shared by the tests, the benchmark and the
smoke check).  This module draws random numbers and shapes only: it holds none of the
operator's arithmetic, so both the HIP path and the CPU oracle can consume it.

Shapes follow the fixed topology of the operator (MSA pull-request page, "Supported
scope"): 64 query heads, 4 KV heads, 4 index heads, head dim 128, key blocks of 128
tokens, 16 selection slots per (index head, query) with -1 in unused slots.

Recipe (stated once here and in the design notes):
* Tensors: Q [T,64,128], K [T,4,128], V [T,4,128], dO [T,64,128], drawn in that order
  as float32 N(0,1) from ``torch.Generator().manual_seed(tensor_seed)`` and rounded to
  bf16 (round-to-nearest-even, torch's conversion).
* Structure: ``numpy.random.default_rng(structure_seed)``; draw order is document
  lengths (and padding), then q2k index-head-major, token-minor.  Valid slots of a row
  are shuffled, then padded with -1 to 16 (except rule "all", which is ascending).
"""
from __future__ import annotations

import numpy as np

NUM_Q_HEADS = 64
NUM_KV_HEADS = 4
NUM_INDEX_HEADS = 4
HEAD_DIM = 128
BLOCK = 128
TOPK = 16

CONFIGS = {
    0: "single document T=512, all causal blocks selected (dense causal GQA)",
    1: "one packed 16384-token row, document lengths U{512..6000}, 0-5% trailing pad; "
       "diagonal + up to 15 uniform earlier blocks",
    2: "single 16384-token document; diagonal + sink block 0 + 14 uniform causal blocks",
    3: "single 65536-token document; diagonal + 3 local + 12 distance-decaying blocks",
    4: "4 packed 16384-token rows of short documents (15 + Geometric(1/285)); diagonal + "
       "skewed (70% Zipf s=1.2) earlier blocks",
}


# ------------------------------------------------------------------ document lengths
def _lengths_packed_uniform(rng, row_tokens=16384, lo=512, hi=6000, max_pad_frac=0.05):
    pad = int(rng.integers(0, int(max_pad_frac * row_tokens) + 1))
    target = row_tokens - pad
    lens, total = [], 0
    while total < target:
        L = int(rng.integers(lo, hi + 1))
        L = min(L, target - total)
        lens.append(L)
        total += L
    return lens


def _lengths_geometric_rows(rng, rows=4, row_tokens=16384, shift=15, p=1.0 / 285):
    lens = []
    for _ in range(rows):
        total = 0
        while total < row_tokens:
            L = shift + int(rng.geometric(p))
            L = min(L, row_tokens - total)
            lens.append(L)
            total += L
    return lens


def cu_from_lengths(lens):
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return cu


def _token_blocks(cu, blk=BLOCK):
    T = int(cu[-1])
    t = np.arange(T)
    doc = np.searchsorted(cu, t, side="right") - 1
    return (t - cu[doc]) // blk


# ------------------------------------------------------------------ selection rules
def _finish_rows(rng, sel_lists, topk, ascending=False):
    """sel_lists: list of int arrays (valid ids per row) -> int32 [n, topk]."""
    out = np.full((len(sel_lists), topk), -1, dtype=np.int32)
    for r, s in enumerate(sel_lists):
        s = np.asarray(s, dtype=np.int32)
        if not ascending:
            s = s[rng.permutation(len(s))]
        out[r, :len(s)] = s
    return out


def _pick_uniform(rng, lo, hi, k):
    """k distinct ids uniform from [lo, hi) per row (vectorized over rows).
    lo, hi, k: int arrays [n]; returns list of arrays."""
    n = len(lo)
    width = int(np.max(hi - lo)) if n else 0
    if width <= 0:
        return [np.zeros(0, dtype=np.int64) for _ in range(n)]
    keys = rng.random((n, width))
    col = np.arange(width)[None, :]
    keys[col >= (hi - lo)[:, None]] = np.inf
    order = np.argsort(keys, axis=1, kind="stable")
    return [lo[r] + order[r, :k[r]] for r in range(n)]


def _rule_all(rng, blk_t, topk):
    return _finish_rows(rng, [np.arange(b + 1) for b in blk_t], topk, ascending=True)


def _rule_uniform(rng, blk_t, topk):
    k = np.minimum(topk - 1, blk_t)
    picks = _pick_uniform(rng, np.zeros_like(blk_t), blk_t, k)
    return _finish_rows(rng, [np.concatenate([[b], p]) for b, p in zip(blk_t, picks)], topk)


def _rule_sink(rng, blk_t, topk):
    rows = [None] * len(blk_t)
    small = np.nonzero(blk_t < topk)[0]
    big = np.nonzero(blk_t >= topk)[0]
    for r in small:
        rows[r] = np.arange(blk_t[r] + 1)
    if len(big):
        b = blk_t[big]
        picks = _pick_uniform(rng, np.ones_like(b), b, np.full_like(b, topk - 2))
        for n, r in enumerate(big):
            rows[r] = np.concatenate([[blk_t[r], 0], picks[n]])
    return _finish_rows(rng, rows, topk)


def _rule_local_decay(rng, blk_t, topk, n_local=3, chunk=4096):
    rows = [None] * len(blk_t)
    for r in np.nonzero(blk_t < topk)[0]:
        rows[r] = np.arange(blk_t[r] + 1)
    big = np.nonzero(blk_t >= topk)[0]
    n_far = topk - 1 - n_local
    for c0 in range(0, len(big), chunk):
        idx = big[c0:c0 + chunk]
        b = blk_t[idx]
        width = int(b.max()) - n_local  # candidates [0, b - n_local)
        cand = np.arange(width)[None, :]
        w = 1.0 / np.maximum(b[:, None] - cand + 1.0, 1.0)  # masked columns get any w
        u = rng.random((len(idx), width))
        # weighted sampling without replacement: largest log(u)/w keys win
        key = np.log(u) / w
        key[cand >= (b - n_local)[:, None]] = -np.inf
        top = np.argsort(-key, axis=1, kind="stable")[:, :n_far]
        for n, r in enumerate(idx):
            local = blk_t[r] - np.arange(n_local + 1)
            rows[r] = np.concatenate([local, top[n]])
    return _finish_rows(rng, rows, topk)


def _rule_zipf(rng, blk_t, topk, s=1.2, p_zipf=0.7):
    rows = [None] * len(blk_t)
    for r, b in enumerate(blk_t):
        b = int(b)
        if b < topk:
            rows[r] = np.arange(b + 1)
            continue
        pz = (np.arange(b) + 1.0) ** (-s)
        pz /= pz.sum()
        chosen = {b}
        while len(chosen) < topk:
            if rng.random() < p_zipf:
                c = int(rng.choice(b, p=pz))
            else:
                c = int(rng.integers(0, b))
            chosen.add(c)
        lst = [b] + sorted(chosen - {b})
        rows[r] = np.array(lst)
    return _finish_rows(rng, rows, topk)


RULES = {"all": _rule_all, "uniform": _rule_uniform, "sink": _rule_sink,
         "local_decay": _rule_local_decay, "zipf": _rule_zipf}


def make_q2k(rng, cu, rule, num_index_heads=NUM_INDEX_HEADS, topk=TOPK, blk=BLOCK):
    blk_t = _token_blocks(cu, blk)
    return np.stack([RULES[rule](rng, blk_t, topk) for _ in range(num_index_heads)])


def make_structure(cfg: int, seed: int | None = None):
    """(cu_seqlens int32 [N+1], q2k int32 [4, T, 16]) of one of the five workloads."""
    rng = np.random.default_rng(cfg if seed is None else seed)
    if cfg == 0:
        cu, rule = cu_from_lengths([512]), "all"
    elif cfg == 1:
        cu, rule = cu_from_lengths(_lengths_packed_uniform(rng)), "uniform"
    elif cfg == 2:
        cu, rule = cu_from_lengths([16384]), "sink"
    elif cfg == 3:
        cu, rule = cu_from_lengths([65536]), "local_decay"
    elif cfg == 4:
        cu, rule = cu_from_lengths(_lengths_geometric_rows(rng)), "zipf"
    else:
        raise ValueError(cfg)
    return cu, make_q2k(rng, cu, rule)


def make_custom(lengths, rule, seed, num_index_heads=NUM_INDEX_HEADS, topk=TOPK, blk=BLOCK):
    """Small variants for tests: given document lengths and a selection rule."""
    rng = np.random.default_rng(seed)
    cu = cu_from_lengths(lengths)
    return cu, make_q2k(rng, cu, rule, num_index_heads, topk, blk)


def scatter_unused(q2k, seed):
    """Move the -1 slots of every row to random positions (same ids, new slot order)."""
    rng = np.random.default_rng(seed)
    q = np.array(q2k, copy=True)
    keys = rng.random(q.shape)
    order = np.argsort(keys, axis=-1)
    return np.take_along_axis(q, order, axis=-1)


def make_tensors(T, seed, num_heads=NUM_Q_HEADS, num_kv=NUM_KV_HEADS, head_dim=HEAD_DIM,
                 device="cpu"):
    """bf16 Q, K, V, dO (in that draw order) from float32 N(0,1)."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = {}
    for name, h in (("Q", num_heads), ("K", num_kv), ("V", num_kv), ("dO", num_heads)):
        x = torch.randn((T, h, head_dim), generator=g, dtype=torch.float32)
        out[name] = x.to(torch.bfloat16).to(device)
    return out


def make_long_q2k(cu, seed, topk=TOPK, blk=BLOCK, p_unused=0.1):
    """Vectorized q2k for very long documents: per (index head, query) the diagonal block
    and topk - 1 uniform draws from the causal blocks (with replacement, so ids may
    repeat), each slot then set to -1 with probability p_unused."""
    rng = np.random.default_rng(seed)
    blk_t = _token_blocks(np.asarray(cu), blk).astype(np.int64)
    T = len(blk_t)
    q = np.empty((NUM_INDEX_HEADS, T, topk), dtype=np.int32)
    q[:, :, 0] = blk_t
    q[:, :, 1:] = (rng.random((NUM_INDEX_HEADS, T, topk - 1)) * (blk_t[None, :, None] + 1)).astype(np.int32)
    q[rng.random((NUM_INDEX_HEADS, T, topk)) < p_unused] = -1
    return q


def make_index_tensors(T, seed, num_index_heads=NUM_INDEX_HEADS, head_dim=HEAD_DIM, device="cpu"):
    """bf16 index-Q, index-K (in that draw order) from float32 N(0,1): the indexer's
    projections, [T, 4, 128] each."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = {}
    for name in ("IQ", "IK"):
        x = torch.randn((T, num_index_heads, head_dim), generator=g, dtype=torch.float32)
        out[name] = x.to(torch.bfloat16).to(device)
    return out


def make_config(cfg: int, device="cpu"):
    """Full workload: structure and tensors (tensor seed 1000 + cfg)."""
    cu, q2k = make_structure(cfg)
    tens = make_tensors(int(cu[-1]), 1000 + cfg, device=device)
    return cu, q2k, tens
