"""GPU test of msa_build_k2q_csr_noalloc, the CSR entry point that allocates nothing
(its counters live in a device array of the library): called through the C ABI twice in
a row, the second time on a smaller layout, it must produce the same CSR and status word
as msa_build_k2q_csr with a caller-provided scratch buffer (row pointers and status
bit-exact, each row's queries equal after sorting: the fill order of a row is
unspecified)."""
import numpy as np
import pytest
import torch

import workloads as WL
from _gpu_util import msa_module, say

pytestmark = pytest.mark.gpu


def _with_bad_ids(q2k):
    """Plant an out-of-range id and a duplicate (both flagged in the status word)."""
    q = q2k.copy()
    q[0, 5, 15] = 1000   # beyond blk(t)
    j = int(np.nonzero(q[1, 300] >= 0)[0][0])
    q[1, 300, 15 if j != 15 else 14] = q[1, 300, j]  # repeats a listed block
    return q


def _both(M, lens, rule, seed):
    dev = "cuda:0"
    cu, q2k = WL.make_custom(lens, rule, seed)
    q2k = _with_bad_ids(WL.scatter_unused(q2k, seed))
    L = M.Layout(cu, dev)
    q = torch.from_numpy(np.ascontiguousarray(q2k, dtype=np.int32)).to(dev)
    out = []
    for noalloc in (False, True):
        rp = torch.full((4 * L.NB + 1,), -7, dtype=torch.int32, device=dev)
        cols = torch.full((M.msa_csr_cols_capacity(L),), -7, dtype=torch.int32, device=dev)
        st = torch.full((4,), -7, dtype=torch.int32, device=dev)
        if noalloc:
            M.msa_build_k2q_csr_noalloc(q, L, rp, cols, st)
        else:
            scratch = torch.empty(M.msa_csr_scratch_bytes(L), dtype=torch.uint8, device=dev)
            M.msa_build_k2q_csr(q, L, rp, cols, st, scratch)
        torch.cuda.synchronize()
        out.append((rp.cpu().numpy(), cols.cpu().numpy(), int(st[0].item())))
    (rp0, c0, s0), (rp1, c1, s1) = out
    np.testing.assert_array_equal(rp1, rp0)
    assert s1 == s0 == 3, (s0, s1)
    for r in range(len(rp0) - 1):
        np.testing.assert_array_equal(np.sort(c1[rp1[r]:rp1[r + 1]]), np.sort(c0[rp0[r]:rp0[r + 1]]))
    return int(rp0[-1])


def test_noalloc_csr_matches_the_scratch_entry_point_twice():
    M = msa_module()
    say("case", "noalloc csr: 3 documents, 8,700 tokens")
    n1 = _both(M, [5000, 3000, 700], "uniform", 3)
    say("case", "noalloc csr: smaller layout after it, 429 tokens")
    n2 = _both(M, [300, 129], "sink", 4)
    assert n2 < n1
