"""GPU parity of the k2q CSR on a document longer than the CSR kernel's LDS histogram
covers (4,096 blocks = 524,288 tokens): the workgroups whose 256 tokens span more blocks
than that count through global atomics instead.  Checked bit-exact (after a per-row sort)
against the oracle's CSR, with the status word against the oracle's validator."""
import numpy as np
import pytest
import torch

import block_sparse_attention_q2k_amd as M
import workloads as WL
from oracle import oracle as OR
from _gpu_util import say

pytestmark = pytest.mark.gpu


def test_csr_document_beyond_lds_histogram():
    cu = WL.cu_from_lengths([540_000, 300])  # 4,219 blocks, then a short document
    q2k = WL.make_long_q2k(cu, seed=31)
    dev = "cuda:0"
    L = M.Layout(cu, dev)
    say("csr long document: T=%d NB=%d" % (L.T, L.NB))
    row_ptr = torch.empty(4 * L.NB + 1, dtype=torch.int32, device=dev)
    cols = torch.empty(M.msa_csr_cols_capacity(L), dtype=torch.int32, device=dev)
    status = torch.zeros(4, dtype=torch.int32, device=dev)
    scratch = M._bytes(M.msa_csr_scratch_bytes(L), dev)
    M.msa_build_k2q_csr(torch.from_numpy(q2k).to(dev), L, row_ptr, cols, status, scratch)
    torch.cuda.synchronize()
    rp = row_ptr.cpu().numpy()
    cl = cols.cpu().numpy()
    orp, ocols = OR.k2q_csr(q2k, cu)
    np.testing.assert_array_equal(rp, orp)
    for r in range(len(orp) - 1):
        np.testing.assert_array_equal(np.sort(cl[rp[r]:rp[r + 1]]), ocols[orp[r]:orp[r + 1]])
    assert int(status[0].item()) == OR.validate(q2k, cu)
    say("  nnz %d, status %d" % (int(orp[-1]), int(status[0].item())))
