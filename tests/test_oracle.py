"""Pins of the fp64 oracle against things other than itself: a hand-derived closed-form
example, textbook dense causal attention (torch SDPA), an independent dense-mask
reformulation with autograd, central finite differences, closed forms and invariants.
CPU only."""
import math

import numpy as np
import pytest
import torch

import workloads as WL
from oracle import oracle as OR


def _tiny_case(lengths, rule, seed, H=8, HKV=2, HI=2, D=16, BLK=8, TOPK=4):
    cu, q2k = WL.make_custom(lengths, rule, seed, num_index_heads=HI, topk=TOPK, blk=BLK)
    T = int(cu[-1])
    rng = np.random.default_rng(seed + 100)
    Q = rng.standard_normal((T, H, D))
    K = rng.standard_normal((T, HKV, D))
    V = rng.standard_normal((T, HKV, D))
    dO = rng.standard_normal((T, H, D))
    return cu, q2k, Q, K, V, dO, BLK


# ------------------------------------------------------------------ hand example
def test_hand_derived_example():
    """One head, D=1, block 2, top-2; every value below is derived by hand.
    Q=1, K=[0, ln2, ln3, 0], V=[6, 0, 12, 5], dO=1, scale 1.
    t0 {blk0}: keys {0}; t1 {blk0}: {0,1}; t2 {blk1, blk0}: {0,1,2}; t3 {blk1}: {2,3}."""
    l2, l3 = math.log(2.0), math.log(3.0)
    Q = np.ones((4, 1, 1))
    K = np.array([0.0, l2, l3, 0.0]).reshape(4, 1, 1)
    V = np.array([6.0, 0.0, 12.0, 5.0]).reshape(4, 1, 1)
    dO = np.ones((4, 1, 1))
    q2k = np.array([[[0, -1], [-1, 0], [1, 0], [1, -1]]], dtype=np.int32)
    cu = np.array([0, 4], dtype=np.int32)
    O, LSE = OR.forward(Q, K, V, q2k, cu, 1.0, blk=2)
    # P rows: [1], [1/3, 2/3], [1/6, 2/6, 3/6], [3/4, 1/4]
    np.testing.assert_allclose(O[:, 0, 0], [6.0, 2.0, 7.0, 10.25], rtol=1e-13)
    np.testing.assert_allclose(LSE[:, 0], [0.0, math.log(3), math.log(6), math.log(4)],
                               rtol=1e-13, atol=1e-15)
    dQ, dK, dV, _, delta = OR.backward(Q, K, V, dO, q2k, cu, 1.0, blk=2)
    # dS = P (dP - delta): t1 [4/3, -4/3]; t2 [-1/6, -7/3, 5/2]; t3 [21/16, -21/16]
    np.testing.assert_allclose(dQ[:, 0, 0], [0.0, -4 / 3 * l2, -7 / 3 * l2 + 2.5 * l3,
                                             21 / 16 * l3], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dK[:, 0, 0], [7 / 6, -11 / 3, 2.5 + 21 / 16, -21 / 16], rtol=1e-12)
    np.testing.assert_allclose(dV[:, 0, 0], [1.5, 1.0, 1.25, 0.25], rtol=1e-12)
    np.testing.assert_allclose(delta[:, 0], [6.0, 2.0, 7.0, 10.25], rtol=1e-13)


# ------------------------------------------------------------------ textbook special case
@pytest.mark.parametrize("shape", [dict(H=8, HKV=2, HI=2, D=16, BLK=8, TOPK=4, T=29),
                                   dict(H=64, HKV=4, HI=4, D=128, BLK=128, TOPK=16, T=300)])
def test_all_causal_blocks_equal_dense_causal_sdpa(shape):
    """Selecting every causal block of a single document is dense causal GQA attention
    (each query head h reads KV head h // (H/HKV))."""
    T, H, HKV, D, BLK = shape["T"], shape["H"], shape["HKV"], shape["D"], shape["BLK"]
    cu, q2k, Q, K, V, dO, _ = _tiny_case([T], "all", 3, H=H, HKV=HKV, HI=shape["HI"], D=D,
                                         BLK=BLK, TOPK=shape["TOPK"])
    scale = 1.0 / math.sqrt(D)
    O, LSE = OR.forward(Q, K, V, q2k, cu, scale, blk=BLK)
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, scale, blk=BLK)
    q = torch.tensor(Q, dtype=torch.float64).permute(1, 0, 2).requires_grad_()
    k = torch.tensor(K, dtype=torch.float64).permute(1, 0, 2).requires_grad_()
    v = torch.tensor(V, dtype=torch.float64).permute(1, 0, 2).requires_grad_()
    rep = H // HKV
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(rep, 0), v.repeat_interleave(rep, 0), is_causal=True, scale=scale)
    out.backward(torch.tensor(dO, dtype=torch.float64).permute(1, 0, 2))
    np.testing.assert_allclose(O, out.detach().permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dQ, q.grad.permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dK, k.grad.permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dV, v.grad.permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)
    # LSE against torch's logsumexp over the causal score matrix
    s = torch.einsum("htd,hsd->hts", torch.tensor(Q).permute(1, 0, 2),
                     torch.tensor(K).permute(1, 0, 2).repeat_interleave(rep, 0)) * scale
    s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(LSE, torch.logsumexp(s, -1).T.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ dense-mask reformulation
def _dense_mask_reference(Q, K, V, dO, q2k, cu, scale, BLK):
    """The pages' generic path: expand the selection into a boolean per-head token mask
    (document-local, causal, key block listed) and run dense masked attention."""
    T, H, D = Q.shape
    HKV, HI = K.shape[1], q2k.shape[0]
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    pos = np.arange(T) - cu[doc]
    mask = np.zeros((HI, T, T), dtype=bool)
    for i in range(HI):
        for t in range(T):
            sel = set(int(b) for b in q2k[i, t] if b >= 0)
            for s_ in range(T):
                mask[i, t, s_] = (doc[s_] == doc[t] and pos[s_] <= pos[t] and pos[s_] // BLK in sel)
    q = torch.tensor(Q).permute(1, 0, 2).requires_grad_()
    k = torch.tensor(K).permute(1, 0, 2).requires_grad_()
    v = torch.tensor(V).permute(1, 0, 2).requires_grad_()
    hm = torch.tensor(mask).repeat_interleave(H // HI, 0)
    s = (q @ k.repeat_interleave(H // HKV, 0).transpose(1, 2)) * scale
    s = s.masked_fill(~hm, float("-inf"))
    lse = torch.logsumexp(s, -1)
    p = torch.where(hm, torch.exp(s - lse.unsqueeze(-1).clamp_min(-1e300)), torch.zeros_like(s))
    out = p @ v.repeat_interleave(H // HKV, 0)
    out.backward(torch.tensor(dO).permute(1, 0, 2))
    return (out.detach().permute(1, 0, 2).numpy(), lse.detach().T.numpy(),
            q.grad.permute(1, 0, 2).numpy(), k.grad.permute(1, 0, 2).numpy(),
            v.grad.permute(1, 0, 2).numpy())


@pytest.mark.parametrize("rule,lengths,seed", [("uniform", [37, 21, 9], 1),
                                               ("sink", [70], 2),
                                               ("local_decay", [90, 5], 3),
                                               ("zipf", [64, 17, 40], 4)])
def test_selection_matches_dense_mask_reformulation(rule, lengths, seed):
    cu, q2k, Q, K, V, dO, BLK = _tiny_case(lengths, rule, seed, TOPK=5)
    q2k = WL.scatter_unused(q2k, seed)  # -1 slots anywhere in the row
    scale = 0.3
    O, LSE = OR.forward(Q, K, V, q2k, cu, scale, blk=BLK)
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, scale, blk=BLK)
    rO, rL, rdQ, rdK, rdV = _dense_mask_reference(Q, K, V, dO, q2k, cu, scale, BLK)
    for a, b in ((O, rO), (LSE, rL), (dQ, rdQ), (dK, rdK), (dV, rdV)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def test_invalid_and_duplicate_ids_add_no_keys():
    """Out-of-range ids and repeated ids do not change the key set (it is a set of
    document-local causal blocks); the validator flags them."""
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([40, 30], "uniform", 7, TOPK=6)
    bad = q2k.copy()
    blk_t = (np.arange(int(cu[-1])) - cu[np.searchsorted(cu, np.arange(int(cu[-1])), "right") - 1]) // BLK
    assert OR.validate(q2k, cu, BLK) == 0
    for i in range(bad.shape[0]):
        for t in range(bad.shape[1]):
            free = np.nonzero(bad[i, t] == -1)[0]
            if len(free) >= 2:
                bad[i, t, free[0]] = blk_t[t] + 1 + (t % 3)  # beyond the causal range
                bad[i, t, free[1]] = bad[i, t, 0]            # duplicate of slot 0
    assert OR.validate(bad, cu, BLK) == 3
    a = OR.backward(Q, K, V, dO, q2k, cu, 0.25, blk=BLK)
    b = OR.backward(Q, K, V, dO, bad, cu, 0.25, blk=BLK)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)
    neg = q2k.copy()
    neg[0, 0, -1] = -5
    assert OR.validate(neg, cu, BLK) & 1


# ------------------------------------------------------------------ finite differences
def test_gradients_match_central_finite_differences():
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([13, 9], "uniform", 11, H=4, HKV=1, HI=1, D=8,
                                           BLK=4, TOPK=3)
    scale = 0.7
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, scale, blk=BLK)

    def loss(Q_, K_, V_):
        O, _ = OR.forward(Q_, K_, V_, q2k, cu, scale, blk=BLK)
        return float(np.sum(O * dO))

    rng = np.random.default_rng(5)
    h = 1e-6
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = {"Q": (Xp, K, V), "K": (Q, Xp, V), "V": (Q, K, Xp)}[name]
            args_m = {"Q": (Xm, K, V), "K": (Q, Xm, V), "V": (Q, K, Xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-6 * max(1.0, abs(G[idx])), (name, idx, fd, G[idx])


# ------------------------------------------------------------------ closed forms
def test_zero_query_gives_uniform_attention():
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([33, 20], "uniform", 21)
    Q[:] = 0.0
    O, LSE = OR.forward(Q, K, V, q2k, cu, 0.5, blk=BLK)
    T, H, D = Q.shape
    HI, HKV = q2k.shape[0], K.shape[1]
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    for t in range(T):
        pos = t - cu[doc[t]]
        for h in range(H):
            i = h // (H // HI)
            keys = [cu[doc[t]] + p for p in range(pos + 1) if p // BLK in set(q2k[i, t][q2k[i, t] >= 0])]
            assert abs(LSE[t, h] - math.log(len(keys))) < 1e-12
            np.testing.assert_allclose(O[t, h], V[keys, i // (HI // HKV)].mean(0), rtol=1e-11, atol=1e-12)


def test_first_token_of_document_closed_form():
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([17, 25, 8], "uniform", 23)
    scale = 0.9
    O, LSE = OR.forward(Q, K, V, q2k, cu, scale, blk=BLK)
    dQ, _, _, _, _ = OR.backward(Q, K, V, dO, q2k, cu, scale, blk=BLK)
    H, HKV = Q.shape[1], K.shape[1]
    for t in cu[:-1]:
        for h in range(H):
            kv = h // (H // HKV)
            np.testing.assert_allclose(O[t, h], V[t, kv], rtol=1e-13)
            assert abs(LSE[t, h] - scale * np.dot(Q[t, h], K[t, kv])) < 1e-12
            np.testing.assert_allclose(dQ[t, h], 0.0, atol=1e-14)


def test_constant_values_give_constant_output_and_zero_qk_grads():
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([45, 12], "sink", 29)
    V[:] = 1.75
    O, _ = OR.forward(Q, K, V, q2k, cu, 0.4, blk=BLK)
    dQ, dK, _, _, _ = OR.backward(Q, K, V, dO, q2k, cu, 0.4, blk=BLK)
    np.testing.assert_allclose(O, 1.75, rtol=1e-13)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-12)
    np.testing.assert_allclose(dK, 0.0, atol=1e-12)


def test_empty_key_set_row():
    """A row whose slots are all -1 has no keys: O = 0, LSE = -inf, no gradient."""
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([20], "uniform", 31)
    q2k[0, 11, :] = -1
    O, LSE = OR.forward(Q, K, V, q2k, cu, 0.5, blk=BLK)
    dQ, dK, dV, _, _ = OR.backward(Q, K, V, dO, q2k, cu, 0.5, blk=BLK)
    hpi = Q.shape[1] // q2k.shape[0]
    assert np.all(O[11, :hpi] == 0.0) and np.all(np.isneginf(LSE[11, :hpi]))
    assert np.all(dQ[11, :hpi] == 0.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(dK)) and np.all(np.isfinite(dV))


# ------------------------------------------------------------------ invariants
def test_slot_order_and_unused_slot_placement_do_not_matter():
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([50, 31], "uniform", 41, TOPK=6)
    a = OR.backward(Q, K, V, dO, q2k, cu, 0.3, blk=BLK)
    b = OR.backward(Q, K, V, dO, WL.scatter_unused(q2k, 9), cu, 0.3, blk=BLK)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def test_documents_do_not_leak():
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([30, 26, 19], "uniform", 43)
    a = OR.backward(Q, K, V, dO, q2k, cu, 0.3, blk=BLK)
    fa = OR.forward(Q, K, V, q2k, cu, 0.3, blk=BLK)
    sl = slice(int(cu[1]), int(cu[2]))  # perturb document 1 only
    Q2, K2, V2, dO2 = Q.copy(), K.copy(), V.copy(), dO.copy()
    for X in (Q2, K2, V2, dO2):
        X[sl] += 3.0
    b = OR.backward(Q2, K2, V2, dO2, q2k, cu, 0.3, blk=BLK)
    fb = OR.forward(Q2, K2, V2, q2k, cu, 0.3, blk=BLK)
    keep = np.ones(int(cu[-1]), dtype=bool)
    keep[sl] = False
    for x, y in list(zip(a, b)) + list(zip(fa, fb)):
        np.testing.assert_array_equal(x[keep], y[keep])


def test_key_and_value_shifts():
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([41, 22], "zipf", 47)
    scale = 0.6
    O, LSE = OR.forward(Q, K, V, q2k, cu, scale, blk=BLK)
    c = np.random.default_rng(1).standard_normal(K.shape[1:])  # per KV head
    O2, LSE2 = OR.forward(Q, K + c[None], V, q2k, cu, scale, blk=BLK)
    H, HKV = Q.shape[1], K.shape[1]
    shift = scale * np.einsum("thd,hd->th", Q, np.repeat(c, H // HKV, axis=0))
    np.testing.assert_allclose(O2, O, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(LSE2, LSE + shift, rtol=1e-11, atol=1e-11)
    O3, _ = OR.forward(Q, K, V + c[None], q2k, cu, scale, blk=BLK)
    np.testing.assert_allclose(O3, O + np.repeat(c, H // HKV, axis=0)[None], rtol=1e-11, atol=1e-11)


def test_frobenius_identities():
    """<dQ,Q> = <dK,K> (both equal sum dS*s) and <dV,V> = sum delta."""
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([60, 35], "sink", 53)
    dQ, dK, dV, _, delta = OR.backward(Q, K, V, dO, q2k, cu, 0.45, blk=BLK)
    assert abs(np.sum(dQ * Q) - np.sum(dK * K)) < 1e-9 * max(1.0, abs(np.sum(dQ * Q)))
    assert abs(np.sum(dV * V) - np.sum(delta)) < 1e-9 * max(1.0, abs(np.sum(delta)))


def test_delta_closed_form():
    rng = np.random.default_rng(3)
    dO = rng.standard_normal((5, 3, 8))
    O = np.zeros((5, 3, 8))
    O[:, :, 2] = 1.0  # basis vector: delta picks one column
    np.testing.assert_array_equal(OR.delta(O, dO), dO[:, :, 2])


def test_masked_subsets_equal_full_results():
    """Row/block subsets (used at full sizes) agree exactly with the full computation."""
    cu, q2k, Q, K, V, dO, BLK = _tiny_case([70, 33], "uniform", 59)
    T = int(cu[-1])
    full = OR.backward(Q, K, V, dO, q2k, cu, 0.3, blk=BLK)
    rng = np.random.default_rng(2)
    qr = rng.random(T) < 0.3
    kt = np.zeros(T, dtype=bool)
    kt[8:16] = True  # one key block of document 0
    sub = OR.backward(Q, K, V, dO, q2k, cu, 0.3, q_rows=qr, k_tokens=kt, blk=BLK)
    np.testing.assert_array_equal(sub[0], full[0][qr])
    np.testing.assert_allclose(sub[1], full[1][kt], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sub[2], full[2][kt], rtol=1e-13, atol=1e-14)
    fo, fl = OR.forward(Q, K, V, q2k, cu, 0.3, blk=BLK)
    so, sl = OR.forward(Q, K, V, q2k, cu, 0.3, rows=qr, blk=BLK)
    np.testing.assert_array_equal(so, fo[qr])
    np.testing.assert_array_equal(sl, fl[qr])
