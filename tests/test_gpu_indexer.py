"""GPU parity of the indexer's block selection (msa_index_select through the C ABI)
against the oracle (oracle.index_select, fp64 scores from the same bf16 inputs).

The selection is an integer result decided by floating-point scores: the kernel sums
the 128 products in fp32 in its own order, the oracle in fp64.  Each row is compared
as a set: it must be well formed (ascending, unique, causal, min(16, p // 128 + 1)
entries, -1 after them) and equal to the oracle's, except that a block may be swapped
for another whose oracle score lies within SCORE_TOL of the oracle's 16th-best score
(both are then correct selections up to rounding).  The number of such rows is printed;
no row may differ otherwise."""
import numpy as np
import pytest
import torch

import block_sparse_attention_q2k_amd as M
import workloads as WL
from oracle import oracle as OR
from _gpu_util import say

pytestmark = pytest.mark.gpu

BLK, TOPK = 128, 16
# fp32 accumulation of 128 bf16 products of N(0,1) values: |error| ~ 1e-5; the band
# only has to cover rounding, not a different definition
SCORE_TOL = 1e-3


def _run(cu, IQ, IK, q2k_init=None):
    dev = "cuda:0"
    m = M.MSA(cu, device=dev)
    out = None
    if q2k_init is not None:
        out = torch.full((4, int(cu[-1]), TOPK), q2k_init, dtype=torch.int32, device=dev)
    q2k = m.select(IQ.to(dev), IK.to(dev), out)
    torch.cuda.synchronize()
    return q2k.cpu().numpy()


def _check_rows(cu, IQ, IK, got, queries):
    """Compare the GPU rows of `queries` with the oracle; returns the near-tie row count."""
    want, scores = OR.index_select(IQ.float().numpy(), IK.float().numpy(), cu, queries=queries)
    cu = np.asarray(cu)
    doc_of = np.searchsorted(cu, np.arange(int(cu[-1])), side="right") - 1
    ties = 0
    for t in queries:
        p = t - cu[doc_of[t]]
        nb = p // BLK + 1
        n = min(TOPK, nb)
        for i in range(4):
            g = got[i, t]
            ctx = "head %d token %d (position %d)" % (i, t, p)
            assert (g[n:] == -1).all(), ctx
            sel = g[:n]
            assert (sel >= 0).all() and (sel <= p // BLK).all(), ctx
            assert (np.diff(sel) > 0).all(), ctx
            if (sel == want[i, t, :n]).all():
                continue
            s = scores[(i, int(t))]
            s16 = np.sort(s)[::-1][n - 1]
            extra = set(sel.tolist()) - set(want[i, t, :n].tolist())
            missing = set(want[i, t, :n].tolist()) - set(sel.tolist())
            assert all(s[b] >= s16 - SCORE_TOL for b in extra), (ctx, extra, s16)
            assert all(s[b] <= s16 + SCORE_TOL for b in missing), (ctx, missing, s16)
            ties += 1
    return ties


CASES = {
    # doc lengths: under 16 blocks, exactly 16 blocks, over 16 blocks with a ragged
    # tail, a one-token document, a 2-block document
    "mixed": [300, 2048, 2500, 1, 200],
    "long_ragged": [5000],
    "many_short": [17, 129, 128, 64, 255, 1, 40, 700],
}


@pytest.mark.parametrize("name", list(CASES))
def test_index_select_small(name):
    lens = CASES[name]
    cu = WL.cu_from_lengths(lens)
    T = int(cu[-1])
    tens = WL.make_index_tensors(T, 500 + len(lens))
    say("index_select %s: T=%d docs=%d" % (name, T, len(lens)))
    got = _run(cu, tens["IQ"], tens["IK"], q2k_init=-7)
    ties = _check_rows(cu, tens["IQ"], tens["IK"], got, list(range(T)))
    say("  rows at a score tie: %d of %d" % (ties, 4 * T))


def test_index_select_ties_and_repeat_calls():
    """All-zero index-Q: every score is 0 and the 16 smallest causal ids win; a second
    call on the same output overwrites every row."""
    cu = WL.cu_from_lengths([3000, 130])
    T = int(cu[-1])
    tens = WL.make_index_tensors(T, 77)
    IQ0 = torch.zeros_like(tens["IQ"])
    got = _run(cu, IQ0, tens["IK"], q2k_init=123)
    for t in range(T):
        p = t if t < 3000 else t - 3000
        n = min(TOPK, p // BLK + 1)
        assert got[:, t, :n].tolist() == [list(range(n))] * 4
        assert (got[:, t, n:] == -1).all()
    got2 = _run(cu, tens["IQ"], tens["IK"], q2k_init=-5)
    assert _check_rows(cu, tens["IQ"], tens["IK"], got2, list(range(0, T, 7)) + [T - 1]) >= 0


@pytest.mark.parametrize("layout", ["single_16k", "packed_16k_row", "single_64k"])
def test_index_select_full_size_sampled(layout):
    """Full-size layouts: a 16,384-token document (128 blocks), the packed 16,384-token
    row of several documents, and a 65,536-token document (512 blocks, the longest
    walks).  Every row is checked for form, and about 256 sampled rows (the last
    tokens and document starts included) against the oracle."""
    if layout == "single_16k":
        cu = WL.cu_from_lengths([16384])
    elif layout == "packed_16k_row":
        cu, _ = WL.make_structure(1)
    else:
        cu = WL.cu_from_lengths([65536])
    cu = np.asarray(cu)
    T = int(cu[-1])
    tens = WL.make_index_tensors(T, 901)
    got = _run(cu, tens["IQ"], tens["IK"], q2k_init=-9)
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    p = np.arange(T) - cu[doc]
    n = np.minimum(TOPK, p // BLK + 1)
    for i in range(4):
        sel_ok = np.ones(T, bool)
        for k in range(TOPK):
            col = got[i, :, k]
            sel_ok &= np.where(k < n, (col >= 0) & (col <= p // BLK), col == -1)
        assert sel_ok.all()
    rng = np.random.default_rng(5)
    qs = set(rng.integers(0, T, 240).tolist()) | set(range(T - 8, T)) | set(cu[:-1].tolist())
    qs = sorted(qs)[:300]
    ties = _check_rows(cu, tens["IQ"], tens["IK"], got, qs)
    say("  %s: sampled rows at a score tie: %d of %d" % (layout, ties, 4 * len(qs)))


def test_selection_feeds_the_operator():
    """The path from the indexer on: the GPU selection (checked against the oracle) drives
    the forward and backward, whose outputs match the oracle given the same q2k."""
    from _gpu_util import SCALE, check_close, check_lse, inputs64, run_gpu, to_np
    cu = WL.cu_from_lengths([2600, 300, 129])
    T = int(cu[-1])
    it = WL.make_index_tensors(T, 615)
    q2k = _run(cu, it["IQ"], it["IK"], q2k_init=-3)
    assert _check_rows(cu, it["IQ"], it["IK"], q2k, list(range(T))) >= 0
    tens = WL.make_tensors(T, 616)
    _, out = run_gpu(cu, q2k, tens)
    Qn, Kn, Vn, dOn = inputs64(tens)
    rO, rL = OR.forward(Qn, Kn, Vn, q2k, cu, SCALE)
    rdQ, rdK, rdV, _, _ = OR.backward(Qn, Kn, Vn, dOn, q2k, cu, SCALE)
    check_close("O", to_np(out["O"]), rO)
    check_lse(to_np(out["LSE"]), rL)
    for name, r in (("dQ", rdQ), ("dK", rdK), ("dV", rdV)):
        check_close(name, to_np(out[name]), r)
