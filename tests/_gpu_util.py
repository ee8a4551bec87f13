"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle."""
import math
import sys

import numpy as np
import torch

import workloads as WL
from oracle import oracle as OR

SCALE = 1.0 / math.sqrt(128.0)
REL_L2 = 1e-2          # relative L2 error bound (per tensor)
MAX_ABS_FRAC = 3e-2    # max-abs error bound, as a fraction of max |oracle| (per tensor)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def msa_module():
    import block_sparse_attention_q2k_amd as M
    M.lib()  # fails loudly if the library is not built
    return M


def to_np(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def check_close(name, gpu, ref, rel_l2=REL_L2, max_abs_frac=MAX_ABS_FRAC, mask=None):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        g, r = g[mask], r[mask]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite GPU values" % name
    err = g - r
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(err) / max(nr, 1e-30)
    mx = np.max(np.abs(err)) / max(np.max(np.abs(r)), 1e-30)
    say("  %-6s rel_l2=%.3e max_abs/max|ref|=%.3e" % (name, rel, mx))
    assert rel <= rel_l2, "%s: rel L2 %.3e > %.1e" % (name, rel, rel_l2)
    assert mx <= max_abs_frac, "%s: max-abs %.3e > %.1e" % (name, mx, max_abs_frac)
    return rel, mx


def check_lse(gpu, ref, mask=None):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        g, r = g[mask], r[mask]
    ninf = np.isneginf(r)
    np.testing.assert_array_equal(np.isneginf(g), ninf)
    return check_close("LSE", g[~ninf], r[~ninf])


def run_gpu(cu, q2k, tens, mode=3, grid=None, backward=True, scale=SCALE):
    """Forward (+ backward) of the HIP path on cuda:0.  Returns (msa object, outputs)."""
    M = msa_module()
    dev = "cuda:0"
    m = M.MSA(cu, grid=grid, dq_mode=mode, device=dev)
    Q, K, V, dO = (tens[k].to(dev) for k in ("Q", "K", "V", "dO"))
    q = torch.from_numpy(np.ascontiguousarray(q2k, dtype=np.int32)).to(dev)
    O, LSE = m.forward(Q, K, V, q, scale)
    out = dict(O=O, LSE=LSE)
    if backward:
        dQ, dK, dV = m.backward(Q, dO, O, LSE, scale)
        out.update(dQ=dQ, dK=dK, dV=dV, delta=m.delta)
    torch.cuda.synchronize()
    return m, out


def inputs64(tens):
    return [tens[k].float().numpy().astype(np.float64) for k in ("Q", "K", "V", "dO")]


def check_structures(m, cu, q2k):
    """CSR (after per-row sort), plan and task tables bit-exact against the oracle."""
    rp, cols = m.csr()
    orp, ocols = OR.k2q_csr(q2k, cu)
    np.testing.assert_array_equal(rp, orp)
    for r in range(len(orp) - 1):
        np.testing.assert_array_equal(np.sort(cols[rp[r]:rp[r + 1]]), ocols[orp[r]:orp[r + 1]])
    items, lists = m.plan_items()
    oitems, _, olists = OR.forward_plan(q2k, cu, m.fwd_group)
    np.testing.assert_array_equal(items, oitems)
    assert len(lists) == len(olists)
    for a, b in zip(lists, olists):
        np.testing.assert_array_equal(a, b)
    tk = m.task_tables()
    # the oracle's task builder on the GPU's own CSR order must reproduce the tables
    otk = OR.tasks(rp, cols, cu, 4, m.grid, q2k=q2k)
    assert tk["R"] == otk["R"]
    np.testing.assert_array_equal(tk["head_rows"], otk["head_rows"])
    np.testing.assert_array_equal(tk["cta"], otk["cta"])
    np.testing.assert_array_equal(tk["meta"], otk["meta"])
    np.testing.assert_array_equal(tk["qrows"], otk["qrows"])
    np.testing.assert_array_equal(tk["qpos"], otk["qpos"])
    # stored-dS tile index = (t * 4 + i) * 16 + the oracle's member slot
    head = otk["meta"][:, 0:1] // ((len(orp) - 1) // 4)  # bucket r = i * NB + block
    np.testing.assert_array_equal(tk["qtile"], np.where(otk["qrows"] >= 0,
                                                        (otk["qrows"] * 4 + head) * 16 + otk["qslot"], -1))
    # and the canonical tables (sorted CSR) have the same per-bucket content
    ctk = OR.tasks(orp, ocols, cu, 4, m.grid)
    assert ctk["R"] == tk["R"]
    np.testing.assert_array_equal(ctk["meta"][:, [0, 1, 2, 3]], tk["meta"])
    status = int(m.status[0].item())
    return status
