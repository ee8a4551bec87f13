"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Integer structures (CSR, plan, task tables) bit-exact; O, LSE, dQ, dK, dV within
relative L2 <= 1e-2 and max-abs <= 3e-2 of the oracle's largest magnitude; delta
(fp32 from the bf16 O) within 1e-5 relative L2 of the fp64 sum over the same O."""
import numpy as np
import pytest
import torch

import block_sparse_attention_q2k_amd as M
import workloads as WL
from oracle import oracle as OR
from _gpu_util import (SCALE, check_close, check_lse, check_structures, inputs64, run_gpu, say,
                       to_np)

pytestmark = pytest.mark.gpu

# small layouts spanning several tiles, ragged tails and several documents
SMALL = {
    "dense_512": ([512], "all", 0),
    "uniform_3docs_ragged": ([700, 300, 129], "uniform", 1),
    "sink_1000": ([1000], "sink", 2),
    "local_decay_2100": ([2100], "local_decay", 3),
    "zipf_many_short": ([300, 17, 129, 128, 64, 255, 1, 40], "zipf", 4),
}


def _small(name, scatter=False):
    lens, rule, seed = SMALL[name]
    cu, q2k = WL.make_custom(lens, rule, seed)
    if scatter:
        q2k = WL.scatter_unused(q2k, seed)
    tens = WL.make_tensors(int(cu[-1]), 100 + seed)
    return cu, q2k, tens


def test_plan_long_document():
    """Walk lists of a 70,000-token document (547 blocks: items past 512 blocks take the
    sorting list builder, the others the per-block mask builder) and a short one, bit-exact
    against the oracle's plan."""
    say("case", "plan_70000_3000")
    cu, q2k = WL.make_custom([70000, 3000], "uniform", 11)
    dev = "cuda:0"
    m = M.MSA(cu, device=dev)
    q = torch.from_numpy(np.ascontiguousarray(q2k, dtype=np.int32)).to(dev)
    M.msa_build_k2q_csr(q, m.layout, m.row_ptr, m.cols, m.status, m.csr_scratch)
    M.msa_plan(m.layout, q, m.plan)
    torch.cuda.synchronize()
    items, lists = m.plan_items()
    oitems, _, olists = OR.forward_plan(q2k, cu, m.fwd_group)
    np.testing.assert_array_equal(items, oitems)
    assert len(lists) == len(olists)
    long_items = 0
    for it, a, b in zip(items, lists, olists):
        np.testing.assert_array_equal(a, b)
        long_items += (int(it[1]) - int(cu[int(it[3])]) + int(it[2]) - 1) // 128 + 1 > 512
    assert long_items > 0


@pytest.mark.parametrize("name", list(SMALL))
def test_structures_small(name):
    say("case", name)
    cu, q2k, tens = _small(name, scatter=True)
    m, _ = run_gpu(cu, q2k, tens, backward=True, grid=37)
    assert check_structures(m, cu, q2k) == 0


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_parity_small(name):
    say("case", name)
    cu, q2k, tens = _small(name)
    m, out = run_gpu(cu, q2k, tens, backward=False)
    Q, K, V, _ = inputs64(tens)
    O, LSE = OR.forward(Q, K, V, q2k, cu, SCALE)
    check_close("O", to_np(out["O"]), O)
    check_lse(to_np(out["LSE"]), LSE)


@pytest.mark.parametrize("mode", [3, 2, 0, 1, 4])
@pytest.mark.parametrize("name", list(SMALL))
def test_backward_parity_small(name, mode):
    say("case", name, "dq mode", mode)
    cu, q2k, tens = _small(name, scatter=(mode != 0))
    m, out = run_gpu(cu, q2k, tens, mode=mode)
    Q, K, V, dO = inputs64(tens)
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, SCALE)
    # delta from the bf16 O the backward consumes, fp32 on the GPU vs fp64 here
    dref = OR.delta(to_np(out["O"]), dO)
    check_close("delta", to_np(out["delta"]), dref, rel_l2=1e-5, max_abs_frac=1e-5)
    check_close("dQ", to_np(out["dQ"]), dQ)
    check_close("dK", to_np(out["dK"]), dK)
    check_close("dV", to_np(out["dV"]), dV)


@pytest.mark.parametrize("grid", [1, 7, 1000])
def test_backward_parity_grids(grid):
    """The KV-parallel walk at other grid sizes: one workgroup per index head walking
    every task row, buckets split between workgroups (their dK/dV parts added
    atomically), and workgroups with empty or one-row ranges."""
    say("case uniform_3docs_ragged grid", grid)
    cu, q2k, tens = _small("uniform_3docs_ragged", scatter=True)
    m, out = run_gpu(cu, q2k, tens, mode=3, grid=grid)
    assert check_structures(m, cu, q2k) == 0
    Q, K, V, dO = inputs64(tens)
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, SCALE)
    check_close("dQ", to_np(out["dQ"]), dQ)
    check_close("dK", to_np(out["dK"]), dK)
    check_close("dV", to_np(out["dV"]), dV)


@pytest.mark.parametrize("seed", range(6))
def test_parity_random_layouts(seed):
    """Seeded random layouts (1-4 documents of 1-1,000 tokens, a random selection rule,
    slots scattered) at a random grid: the forward and the default backward against the
    oracle.  The grid changes how many task rows each workgroup of the KV kernel walks,
    and so which of its ring slots and descriptor rows wrap."""
    rng = np.random.default_rng(7000 + seed)
    lens = [int(v) for v in rng.integers(1, 1001, int(rng.integers(1, 5)))]
    rule = str(rng.choice(["uniform", "sink", "local_decay", "zipf"]))
    grid = int(rng.choice([1, 3, 13, 64, 256, 999]))
    say("case random layout", seed, lens, rule, "grid", grid)
    cu, q2k = WL.make_custom(lens, rule, 7100 + seed)
    q2k = WL.scatter_unused(q2k, 7200 + seed)
    tens = WL.make_tensors(int(cu[-1]), 7300 + seed)
    m, out = run_gpu(cu, q2k, tens, mode=3, grid=grid)
    assert check_structures(m, cu, q2k) == 0
    Q, K, V, dO = inputs64(tens)
    O, LSE = OR.forward(Q, K, V, q2k, cu, SCALE)
    check_close("O", to_np(out["O"]), O)
    check_lse(to_np(out["LSE"]), LSE)
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, SCALE)
    check_close("dQ", to_np(out["dQ"]), dQ)
    check_close("dK", to_np(out["dK"]), dK)
    check_close("dV", to_np(out["dV"]), dV)


@pytest.mark.parametrize("scale", [0.03, 0.3])
def test_parity_other_scales(scale):
    """Softmax scales other than 1/sqrt(128): the scale enters the exponents, the dK
    flush and the dQ epilogue separately."""
    say("case sink_1000 scale", scale)
    cu, q2k, tens = _small("sink_1000", scatter=True)
    m, out = run_gpu(cu, q2k, tens, mode=3, scale=scale)
    Q, K, V, dO = inputs64(tens)
    O, LSE = OR.forward(Q, K, V, q2k, cu, scale)
    check_close("O", to_np(out["O"]), O)
    check_lse(to_np(out["LSE"]), LSE)
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, scale)
    check_close("dQ", to_np(out["dQ"]), dQ)
    check_close("dK", to_np(out["dK"]), dK)
    check_close("dV", to_np(out["dV"]), dV)


def test_invalid_ids_flagged_and_ignored():
    """Out-of-range and repeated ids set the status bits and add no keys."""
    cu, q2k, tens = _small("uniform_3docs_ragged")
    bad = q2k.copy()
    T = int(cu[-1])
    doc = np.searchsorted(cu, np.arange(T), "right") - 1
    blk = (np.arange(T) - cu[doc]) // 128
    for t in range(0, T, 7):
        free = np.nonzero(bad[0, t] == -1)[0]
        if len(free) >= 2:
            bad[0, t, free[0]] = blk[t] + 1 + t % 5  # beyond the causal range
            bad[0, t, free[1]] = bad[0, t, 0]          # repeat
    m, out = run_gpu(cu, bad, tens)
    assert check_structures(m, cu, bad) == 3
    m2, ref = run_gpu(cu, q2k, tens)
    assert torch.equal(out["O"], ref["O"]) and torch.equal(out["LSE"], ref["LSE"])
    for k in ("dQ", "dK", "dV"):  # atomics: equal up to summation order
        check_close(k, to_np(out[k]), to_np(ref[k]), rel_l2=1e-4, max_abs_frac=1e-2)


def test_empty_key_set_rows():
    cu, q2k, tens = _small("sink_1000")
    q2k[1, 5, :] = -1
    q2k[2, 900, :] = -1
    m, out = run_gpu(cu, q2k, tens)
    O, L, dQ = to_np(out["O"]), to_np(out["LSE"]), to_np(out["dQ"])
    assert np.all(O[5, 16:32] == 0) and np.all(np.isneginf(L[5, 16:32]))
    assert np.all(O[900, 32:48] == 0) and np.all(dQ[900, 32:48] == 0)
    Q, K, V, dO = inputs64(tens)
    rO, rL = OR.forward(Q, K, V, q2k, cu, SCALE)
    check_close("O", O, rO)
    check_lse(L, rL)


def test_forward_reference_fallback_rows():
    """Rows whose later blocks score far above their first block (about 115 nats, so
    2^(s - m) against the first block's maximum would overflow fp32) take the exact-max
    second launch of the forward; they and their item neighbours must still match."""
    say("case fallback_rows_384")
    cu, q2k = WL.make_custom([384], "all", 5)
    tens = WL.make_tensors(384, 105)
    u = torch.full((128,), 1.0 / np.sqrt(128.0))
    Q = tens["Q"].float()
    K = tens["K"].float()
    Q[300:310] = 96.0 * u
    K[128:132] = 16.0 * u
    tens = dict(tens, Q=Q.to(torch.bfloat16), K=K.to(torch.bfloat16))
    m, out = run_gpu(cu, q2k, tens, mode=3)
    Q64, K64, V64, dO64 = inputs64(tens)
    O, LSE = OR.forward(Q64, K64, V64, q2k, cu, SCALE)
    check_close("O", to_np(out["O"]), O)
    check_lse(to_np(out["LSE"]), LSE)
    dQ, dK, dV, _, _ = OR.backward(Q64, K64, V64, dO64, q2k, cu, SCALE)
    check_close("dQ", to_np(out["dQ"]), dQ)
    check_close("dK", to_np(out["dK"]), dK)
    check_close("dV", to_np(out["dV"]), dV)


def test_two_calls_reuse_buffers_and_stay_consistent():
    """The same MSA object run twice gives the same structures and close gradients
    (atomics make them not bitwise equal)."""
    cu, q2k, tens = _small("uniform_3docs_ragged")
    m, out1 = run_gpu(cu, q2k, tens)
    Q, K, V, dO = (tens[k].cuda() for k in ("Q", "K", "V", "dO"))
    q = torch.from_numpy(q2k).cuda()
    O, LSE = m.forward(Q, K, V, q, SCALE)
    dQ, dK, dV = m.backward(Q, dO, O, LSE, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(O, out1["O"]) and torch.equal(LSE, out1["LSE"])
    for a, b, n in ((dQ, out1["dQ"], "dQ"), (dK, out1["dK"], "dK"), (dV, out1["dV"], "dV")):
        check_close(n, to_np(a), to_np(b), rel_l2=1e-2, max_abs_frac=1e-2)


@pytest.mark.parametrize("name", ["uniform_3docs_ragged", "zipf_many_short"])
def test_workspace_alignment_bit_exact(name):
    """Kw/Vw hold each document's key rows at its 128-aligned workspace offset (zeros in
    the padding), per (KV head, block) in MFMA row-fragment order; Kt/Vt hold the same
    blocks in transposed-fragment order (the layouts msa.h documents)."""
    cu, q2k, tens = _small(name)
    m, _ = run_gpu(cu, q2k, tens, backward=False)
    for X, Xw, Xt in (("K", m.Kw, m.Kt), ("V", m.Vw, m.Vt)):
        ref = OR.align_kv(tens[X].view(torch.int16).numpy(), cu)  # [W][kv][dim]
        NB = ref.shape[0] // 128
        blk = ref.reshape(NB, 128, 4, 128).transpose(2, 0, 1, 3)  # [kv][gb][key][dim]
        # key = 32 w + l32, dim = 16 ks + 8 hi + e  ->  [kv][gb][w][ks][hi][l32][e]
        rows = blk.reshape(4, NB, 4, 32, 8, 2, 8).transpose(0, 1, 2, 4, 5, 3, 6)
        np.testing.assert_array_equal(Xw.view(torch.int16).cpu().numpy().reshape(rows.shape), rows)
        # key = 32 kk + 8 g + e, dim = 16 dq + l16  ->  [kv][gb][dq][kk][g][l16][e]
        tr = blk.reshape(4, NB, 4, 4, 8, 8, 16).transpose(0, 1, 5, 2, 3, 6, 4)
        np.testing.assert_array_equal(Xt.view(torch.int16).cpu().numpy().reshape(tr.shape), tr)
