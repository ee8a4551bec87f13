"""GPU parity at the five workloads' full sizes and on one long document, in the
launch configuration the benchmark times (default grid = one workgroup per CU).  Integer structures are
compared in full; O, LSE and dQ on a seeded sample of query rows the oracle computes
one by one; dK/dV on sampled key blocks whose selecting queries the oracle enumerates
in full; at every row, finiteness and delta = rowsum(dO * O)."""
import functools

import numpy as np
import pytest
import torch

import workloads as WL
from oracle import oracle as OR
from _gpu_util import SCALE, check_close, check_lse, check_structures, run_gpu, say, to_np

pytestmark = pytest.mark.gpu


def _sample_rows(cu, rng, n=40):
    T = int(cu[-1])
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows.update([0, T - 1, int(cu[(len(cu) - 1) // 2])])  # ends and a document start
    mask = np.zeros(T, dtype=bool)
    mask[sorted(rows)] = True
    return mask


def _sample_blocks(cu, q2k, rng, n=2, max_queries=1000):
    """Key tokens of n random workspace blocks that at most max_queries (index head,
    query) pairs select (keeps the oracle's enumeration bounded)."""
    row_ptr, cols = OR.k2q_csr(q2k, cu)
    cu_ws, W, NB = OR.layout(cu)
    counts = np.diff(row_ptr).reshape(4, NB).sum(0)
    ok = np.nonzero((counts > 0) & (counts <= max_queries))[0]
    pick = rng.choice(ok, size=min(n, len(ok)), replace=False)
    T = int(cu[-1])
    doc, pos, _ = OR.coords(cu)
    ws_row = cu_ws[doc] + pos
    mask = np.zeros(T, dtype=bool)
    selectors = np.zeros(T, dtype=bool)
    for gb in pick:
        mask |= (ws_row // 128) == gb
        for i in range(4):
            r = i * NB + gb
            selectors[cols[row_ptr[r]:row_ptr[r + 1]]] = True
    return mask, selectors, pick


def _rows64(x, rows):
    """float64 copy of the given rows of a bf16 tensor, zeros elsewhere (the oracle
    reads only those rows)."""
    out = np.zeros(tuple(x.shape), dtype=np.float64)  # untouched pages stay virtual
    idx = np.nonzero(rows)[0]
    out[idx] = x.index_select(0, torch.from_numpy(idx)).float().numpy()
    return out


# One document of 547 key blocks (past the 512-block point where the plan builder
# switches from its block bitmap to sorting the item's entries) and a short one.
LONG = "long"


def _structure(cfg):
    if cfg == LONG:
        return WL.make_custom([70000, 3000], "uniform", 11), 100
    return WL.make_structure(cfg), cfg


@functools.lru_cache(maxsize=1)
def _case(cfg):
    say("  generating workload", cfg)
    (cu, q2k), seed = _structure(cfg)
    tens = WL.make_tensors(int(cu[-1]), 1000 + seed)
    rng = np.random.default_rng(77 + seed)
    qmask = _sample_rows(cu, rng)
    kmask, selectors, blocks = _sample_blocks(cu, q2k, rng)
    need = qmask | selectors
    say("  oracle: rows", int(qmask.sum()), "key blocks", list(blocks), "rows read", int(need.sum()))
    Q, dO = _rows64(tens["Q"], need), _rows64(tens["dO"], need)
    K, V = (tens[k].float().numpy().astype(np.float64) for k in ("K", "V"))
    rO, rL = OR.forward(Q, K, V, q2k, cu, SCALE, rows=qmask)
    rdQ, rdK, rdV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, SCALE, q_rows=qmask, k_tokens=kmask)
    ref = dict(O=rO, LSE=rL, dQ=rdQ, dK=rdK, dV=rdV)
    return cu, q2k, tens, qmask, kmask, ref


@pytest.mark.parametrize("mode", [3, 2])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, LONG])
def test_full_size_config(cfg, mode):
    say("config", cfg, "dq mode", mode)
    cu, q2k, tens, qmask, kmask, ref = _case(cfg)
    m, out = run_gpu(cu, q2k, tens, mode=mode)
    say("  structures")
    assert check_structures(m, cu, q2k) == 0
    qm = torch.from_numpy(qmask).cuda()
    km = torch.from_numpy(kmask).cuda()
    check_close("O", to_np(out["O"][qm]), ref["O"])
    check_lse(to_np(out["LSE"][qm]), ref["LSE"])
    check_close("dQ", to_np(out["dQ"][qm]), ref["dQ"])
    check_close("dK", to_np(out["dK"][km]), ref["dK"])
    check_close("dV", to_np(out["dV"][km]), ref["dV"])
    for k in ("O", "dQ", "dK", "dV"):
        assert torch.isfinite(out[k].float()).all(), k
    d_ref = (out["O"].float() * tens["dO"].cuda().float()).sum(-1)
    assert torch.allclose(out["delta"], d_ref, rtol=1e-4, atol=1e-4)
