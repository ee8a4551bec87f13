"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (default grid = one workgroup per CU).  Integer structures are
compared in full; O, LSE and dQ on a seeded sample of query rows the oracle computes
one by one; dK/dV on sampled key blocks whose selecting queries the oracle enumerates
in full."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import oracle as OR
from _gpu_util import (SCALE, check_close, check_lse, check_structures, run_gpu, say, to_np)

pytestmark = pytest.mark.gpu


def _sample_rows(cu, rng, n=40):
    T = int(cu[-1])
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows.update([0, T - 1, int(cu[len(cu) // 2])])  # ends and a document start
    mask = np.zeros(T, dtype=bool)
    mask[sorted(rows)] = True
    return mask


def _sample_blocks(cu, q2k, rng, n=2, max_queries=2500):
    """Key tokens of n random (document, block) pairs that at most max_queries
    (index head, query) pairs select (keeps the oracle's enumeration bounded)."""
    row_ptr, _ = OR.k2q_csr(q2k, cu)
    cu_ws, W, NB = OR.layout(cu)
    counts = np.diff(row_ptr).reshape(4, NB).sum(0)
    ok = np.nonzero((counts > 0) & (counts <= max_queries))[0]
    pick = rng.choice(ok, size=min(n, len(ok)), replace=False)
    T = int(cu[-1])
    doc, pos, _ = OR.coords(cu)
    ws_row = cu_ws[doc] + pos
    mask = np.zeros(T, dtype=bool)
    for gb in pick:
        mask |= (ws_row // 128) == gb
    return mask, pick


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_full_size_config(cfg, mode):
    say("config", cfg, "dq mode", mode)
    cu, q2k = WL.make_structure(cfg)
    tens = WL.make_tensors(int(cu[-1]), 1000 + cfg)
    m, out = run_gpu(cu, q2k, tens, mode=mode)
    say("  structures")
    assert check_structures(m, cu, q2k) == 0
    rng = np.random.default_rng(77 + cfg)
    qmask = _sample_rows(cu, rng)
    kmask, blocks = _sample_blocks(cu, q2k, rng)
    say("  oracle rows", int(qmask.sum()), "key blocks", list(blocks))
    Q, K, V, dO = (tens[k].float().numpy().astype(np.float64) for k in ("Q", "K", "V", "dO"))
    rO, rL = OR.forward(Q, K, V, q2k, cu, SCALE, rows=qmask)
    rdQ, rdK, rdV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, SCALE, q_rows=qmask, k_tokens=kmask)
    check_close("O", to_np(out["O"][torch.from_numpy(qmask).cuda()]), rO[qmask])
    check_lse(to_np(out["LSE"][torch.from_numpy(qmask).cuda()]), rL[qmask])
    check_close("dQ", to_np(out["dQ"][torch.from_numpy(qmask).cuda()]), rdQ[qmask])
    km = torch.from_numpy(kmask).cuda()
    check_close("dK", to_np(out["dK"][km]), rdK[kmask])
    check_close("dV", to_np(out["dV"][km]), rdV[kmask])
    # properties at every row: finite outputs, delta = rowsum(dO * O) of the bf16 O
    for k in ("O", "dQ", "dK", "dV"):
        assert torch.isfinite(out[k].float()).all(), k
    d_ref = (out["O"].float() * tens["dO"].cuda().float()).sum(-1)
    assert torch.allclose(out["delta"], d_ref, rtol=1e-4, atol=1e-4)
