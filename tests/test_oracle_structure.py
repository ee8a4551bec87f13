"""Pins of the oracle's integer structure (layout, k2q CSR, forward plan, backward task
tables and CTA walk) against brute-force enumeration and the properties the pages
state.  CPU only."""
import json
import os

import numpy as np
import pytest

import workloads as WL
from oracle import oracle as OR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_constants_fixture():
    """tests/golden/page_facts.json holds the operator constants the pages state."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    top = facts["topology"]
    assert (WL.NUM_Q_HEADS, WL.NUM_KV_HEADS, WL.NUM_INDEX_HEADS, WL.HEAD_DIM, WL.BLOCK,
            WL.TOPK) == (top["q_heads"], top["kv_heads"], top["index_heads"], top["head_dim"],
                         top["block"], top["topk"])
    tile = facts["backward_tile"]
    assert OR.TILE_QUERIES * (top["q_heads"] // top["index_heads"]) == tile["rows"]
    assert OR.TILE_QUERIES == tile["queries"]
    assert top["q_heads"] // top["index_heads"] == tile["heads"]


def test_layout_closed_form():
    cu = np.array([0, 1, 129, 258, 258 + 128], dtype=np.int32)  # lengths 1, 128, 129, 128
    cu_ws, W, NB = OR.layout(cu)
    assert list(cu_ws) == [0, 128, 256, 512, 640]
    assert (W, NB) == (640, 5)
    doc, pos, blk = OR.coords(cu)
    assert doc[0] == 0 and doc[1] == 1 and doc[129] == 2 and doc[-1] == 3
    assert pos[128] == 127 and blk[128] == 0 and pos[257] == 128 and blk[257] == 1
    K = np.arange(int(cu[-1]) * 2, dtype=np.float64).reshape(-1, 2)
    Kw = OR.align_kv(K, cu)
    assert Kw.shape == (640, 2)
    assert np.all(Kw[1:128] == 0) and np.all(Kw[128 + 128:256] == 0)
    np.testing.assert_array_equal(OR.gather_ws(Kw, cu), K)


def _brute_csr(q2k, cu, blk):
    HI, T, TOPK = q2k.shape
    cu_ws, W, NB = OR.layout(cu, blk)
    rows = [[] for _ in range(HI * NB)]
    for i in range(HI):
        for t in range(T):
            d = max(k for k in range(len(cu) - 1) if cu[k] <= t)
            pos = t - cu[d]
            seen = set()
            for j in range(TOPK):
                b = int(q2k[i, t, j])
                if b < 0 or b > pos // blk or b in seen:
                    continue
                seen.add(b)
                rows[i * NB + cu_ws[d] // blk + b].append(t)
    return rows


@pytest.mark.parametrize("rule,lengths,seed,topk,blk", [
    ("uniform", [37, 21, 9, 70], 1, 5, 8), ("sink", [130], 2, 6, 8),
    ("zipf", [64, 17, 40, 3], 4, 4, 8), ("all", [40], 5, 5, 8)])
def test_csr_matches_brute_force(rule, lengths, seed, topk, blk):
    cu, q2k = WL.make_custom(lengths, rule, seed, num_index_heads=2, topk=topk, blk=blk)
    q2k = WL.scatter_unused(q2k, seed)
    # plant an out-of-range id and a duplicate; both must be ignored
    q2k[0, 5, -1] = 99
    q2k[1, 7, :2] = q2k[1, 7, 2]
    row_ptr, cols = OR.k2q_csr(q2k, cu, blk)
    rows = _brute_csr(q2k, cu, blk)
    assert row_ptr[0] == 0 and len(row_ptr) == len(rows) + 1
    for r, lst in enumerate(rows):
        assert list(cols[row_ptr[r]:row_ptr[r + 1]]) == sorted(lst)
    assert row_ptr[-1] == OR.member_slots(q2k, cu, blk).sum() == len(cols)


def _brute_tasks(rows, grid, HI):
    meta, qrows = [], []
    for r, lst in enumerate(rows):
        lst = sorted(lst)
        chunks = [lst[k:k + 8] for k in range(0, len(lst), 8)]
        for k, ch in enumerate(chunks):
            meta.append((r, len(ch), int(k == 0) | (2 * int(k == len(chunks) - 1)), k))
            qrows.append(ch + [-1] * (8 - len(ch)))
    return np.array(meta).reshape(-1, 4), np.array(qrows).reshape(-1, 8)


def test_task_member_slots_brute_force():
    """Each task entry's member slot is the first of its query's q2k slots listing the
    bucket's block (duplicates and unused slots planted)."""
    cu, q2k = WL.make_custom([300, 41, 77, 129], "uniform", 9, num_index_heads=3, topk=7, blk=16)
    q2k = WL.scatter_unused(q2k, 9)
    q2k[1, 7, :2] = q2k[1, 7, 2]
    q2k[2, 200, 3] = q2k[2, 200, 5]
    row_ptr, cols = OR.k2q_csr(q2k, cu, 16)
    tk = OR.tasks(row_ptr, cols, cu, 3, 5, blk=16, q2k=q2k)
    cu_ws, W, NB = OR.layout(cu, 16)
    # brute force: first slot of every (index head, query, document-local block)
    first = {}
    for i in range(3):
        for t in range(int(cu[-1])):
            for j in range(q2k.shape[2]):
                first.setdefault((i, t, int(q2k[i, t, j])), j)
    n = 0
    for row in range(tk["R"]):
        r, nv = int(tk["meta"][row, 0]), int(tk["meta"][row, 1])
        i, gb = r // NB, r % NB
        for s_ in range(8):
            t = int(tk["qrows"][row, s_])
            if s_ >= nv:
                assert t == -1 and tk["qslot"][row, s_] == -1
                continue
            d = max(k for k in range(len(cu) - 1) if cu[k] <= t)
            bl = gb - int(cu_ws[d]) // 16
            assert tk["qslot"][row, s_] == first[(i, t, bl)]
            n += 1
    assert n == len(cols)


@pytest.mark.parametrize("grid", [1, 3, 7, 64])
def test_tasks_match_brute_force_and_cover_rows(grid):
    cu, q2k = WL.make_custom([300, 41, 77, 129], "uniform", 8, num_index_heads=3, topk=7, blk=16)
    row_ptr, cols = OR.k2q_csr(q2k, cu, 16)
    tk = OR.tasks(row_ptr, cols, cu, 3, grid, blk=16)
    meta, qrows = _brute_tasks(_brute_csr(q2k, cu, 16), grid, 3)
    np.testing.assert_array_equal(tk["meta"], meta)
    np.testing.assert_array_equal(tk["qrows"], qrows)
    _, pos, _ = OR.coords(cu, 16)
    np.testing.assert_array_equal(tk["qpos"], np.where(qrows >= 0, pos[np.maximum(qrows, 0)], -1))
    counts = np.diff(row_ptr)
    assert tk["R"] == int(np.sum((counts + 7) // 8))
    # exact counts: every tile but the last of its bucket is full
    full = tk["meta"][:, 2] & 2 == 0
    assert np.all(tk["meta"][full, 1] == 8)
    # CTA walk: within each head, contiguous ranges covering each row once
    cover = np.zeros(tk["R"], dtype=int)
    NB = len(counts) // 3
    for i in range(3):
        b = tk["cta"][i]
        assert np.all(np.diff(b) >= 0)
        for c in range(grid):
            cover[b[c]:b[c + 1]] += 1
        head_rows = np.nonzero(tk["meta"][:, 0] // NB == i)[0]
        if len(head_rows):
            assert b[0] == head_rows[0] and b[-1] == head_rows[-1] + 1
        sizes = np.diff(b)
        assert sizes.max() - sizes.min() <= 1
    assert np.all(cover == 1)


@pytest.mark.parametrize("nq", [8, 16, 28, 32])
def test_forward_plan_partitions_queries_and_orders_by_cost(nq):
    cu, q2k = WL.make_custom([300, 41, 77, 129], "uniform", 9, num_index_heads=4, topk=7, blk=16)
    q2k = WL.scatter_unused(q2k, 3)
    q2k[1, 20, 0] = q2k[1, 20, 1]  # a repeated id adds nothing
    items, costs, lists = OR.forward_plan(q2k, cu, nq, blk=16)
    T = int(cu[-1])
    seen = np.zeros((4, T), dtype=int)
    mem = OR.member_slots(q2k, cu, 16).sum(axis=2)
    _, pos, blk = OR.coords(cu, 16)
    for p, (i, t0, n, d) in enumerate(items):
        assert i == p % 4
        assert cu[d] <= t0 and t0 + n <= cu[d + 1] and 1 <= n <= nq
        assert (t0 - cu[d]) % nq == 0
        seen[i, t0:t0 + n] += 1
        assert costs[p] == mem[i, t0:t0 + n].sum()
        # walk list: brute force over the items' queries
        brute = {}
        for u in range(n):
            for b in set(int(x) for x in q2k[i, t0 + u] if 0 <= x <= blk[t0 + u]):
                brute[b] = brute.get(b, 0) | (1 << u)
        got = [(int(b), int(m) & 0xFFFFFFFF) for b, m in lists[p]]  # masks are 32-bit patterns
        assert got == sorted(brute.items())
        assert sum(bin(m).count("1") for _, m in got) == costs[p]
    assert np.all(seen == 1)
    for i in range(4):
        c = costs[i::4]
        assert np.all(np.diff(c) <= 0)
        # ties keep document order
        it = items[i::4]
        for a in range(len(c) - 1):
            if c[a] == c[a + 1]:
                assert it[a][1] < it[a + 1][1]


def test_effective_flops_counts_member_blocks():
    cu, q2k = WL.make_custom([256], "all", 0)
    fwd, bwd, slots = OR.effective_flops(q2k, cu)
    assert slots == 4 * (128 * 1 + 128 * 2)
    assert fwd == 4 * 128 * 128 * 16 * slots and bwd == 2.5 * fwd


def test_config_generators_are_seeded_and_valid():
    for cfg in (0, 2):
        cu1, q1 = WL.make_structure(cfg)
        cu2, q2 = WL.make_structure(cfg)
        np.testing.assert_array_equal(cu1, cu2)
        np.testing.assert_array_equal(q1, q2)
        assert OR.validate(q1, cu1) == 0
    cu, q2k = WL.make_structure(2)
    assert q2k.shape == (4, 16384, 16)
    blk = np.arange(16384) // 128
    big = blk >= 16
    assert np.all((q2k[:, big] >= 0).sum(-1) == 16)
    assert np.all(np.any(q2k[:, big] == 0, axis=-1))
    assert np.all(np.any(q2k == blk[None, :, None], axis=-1))
    t1 = WL.make_tensors(64, 5)
    t2 = WL.make_tensors(64, 5)
    import torch
    assert all(torch.equal(t1[k], t2[k]) for k in t1)
