"""Pins of the oracle's indexer selection (oracle.index_select) against facts that do
not come from the oracle itself: hand-built scores with a known top-16, the truncated
case, causality, document locality, tie order, invariances and a second, dense
formulation of the same definition.

The pages state what the indexer produces (a document-local top-16 q2k per index head
and query, truncated when fewer blocks exist; pull-request page, Design and Supported
scope) but not its scoring rule; the rule tested here is the reading the oracle's
docstring states (block score = best visible key's dot product)."""
import numpy as np
import pytest

from oracle import oracle as O

BLK = 128


def _unit_case(n_blocks=20, top=(0, 2, 3, 5, 6, 7, 9, 10, 11, 12, 13, 15, 16, 17, 18, 19)):
    """One document of n_blocks blocks; index-Q = e0 for every query and head; in block b
    the key at offset 5 has index-K = v_b e0 (v_b = 100 for the blocks in `top`, 1 for the
    others) and every other key is 0."""
    T = n_blocks * BLK
    IQ = np.zeros((T, 4, 128))
    IQ[:, :, 0] = 1.0
    IK = np.zeros((T, 4, 128))
    for b in range(n_blocks):
        IK[b * BLK + 5, :, 0] = 100.0 if b in top else 1.0
    return IQ, IK, [0, T]


def test_hand_built_top16():
    IQ, IK, cu = _unit_case()
    t = 19 * BLK + 50  # sees key 5 of its own block
    q2k, _ = O.index_select(IQ, IK, cu, queries=[t])
    want = [0, 2, 3, 5, 6, 7, 9, 10, 11, 12, 13, 15, 16, 17, 18, 19]
    for i in range(4):
        assert q2k[i, t].tolist() == want


def test_causal_keys_of_the_diagonal_block_are_invisible():
    IQ, IK, cu = _unit_case()
    t = 19 * BLK + 2  # key 19*128+5 lies after the query: block 19 scores 0
    q2k, s = O.index_select(IQ, IK, cu, queries=[t])
    # block 19 drops out; the best of the score-1 blocks {1, 4, 8, 14} by id joins
    assert q2k[0, t].tolist() == [0, 1, 2, 3, 5, 6, 7, 9, 10, 11, 12, 13, 15, 16, 17, 18]
    assert s[(0, t)][19] == 0.0
    t = 19 * BLK + 5  # the query's own key: visible
    q2k, _ = O.index_select(IQ, IK, cu, queries=[t])
    assert q2k[3, t].tolist() == [0, 2, 3, 5, 6, 7, 9, 10, 11, 12, 13, 15, 16, 17, 18, 19]


def test_truncated_rows_pad_with_minus_one():
    IQ, IK, cu = _unit_case()
    for t, nb in ((0, 1), (BLK - 1, 1), (3 * BLK + 7, 4), (15 * BLK, 16)):
        q2k, _ = O.index_select(IQ, IK, cu, queries=[t])
        row = q2k[2, t].tolist()
        assert row == list(range(nb)) + [-1] * (16 - nb)


def test_ties_go_to_the_smaller_block_id():
    T = 30 * BLK
    IQ = np.zeros((T, 4, 128))  # every score 0
    IK = np.ones((T, 4, 128))
    q2k, _ = O.index_select(IQ, IK, [0, T], queries=[T - 1])
    assert q2k[1, T - 1].tolist() == list(range(16))


def test_document_locality_and_future_keys():
    rng = np.random.default_rng(7)
    cu = [0, 1000, 3300, 3400]
    T = cu[-1]
    IQ = rng.standard_normal((T, 4, 128))
    IK = rng.standard_normal((T, 4, 128))
    qs = [1000, 1127, 1128, 2000, 3299, 3300, 3399]
    base, _ = O.index_select(IQ, IK, cu, queries=qs)
    IK2 = IK.copy()
    IK2[:1000] *= 50.0        # another document's keys
    IK2[3300:] *= 50.0
    for t in qs[:5]:
        IK3 = IK2.copy()
        IK3[t + 1:3300] = 1e3 * np.abs(IK3[t + 1:3300])  # keys after the query
        got, _ = O.index_select(IQ, IK3, cu, queries=[t])
        assert (got[:, t] == base[:, t]).all(), t


def test_positive_scale_and_other_heads_do_not_change_a_head():
    rng = np.random.default_rng(3)
    cu = [0, 2900]
    IQ = rng.standard_normal((2900, 4, 128))
    IK = rng.standard_normal((2900, 4, 128))
    qs = [2899, 2500, 1700]
    a, _ = O.index_select(IQ, IK, cu, queries=qs)
    IQ2 = IQ * 3.7
    IK2 = IK.copy()
    IK2[:, 1:] = rng.standard_normal((2900, 3, 128))
    b, _ = O.index_select(IQ2, IK2, cu, queries=qs)
    assert (a[0, qs] == b[0, qs]).all()


@pytest.mark.parametrize("seed", [0, 1])
def test_dense_formulation_agrees(seed):
    """The same definition written densely: all scores of a document as one product,
    a causal mask, per-block maxima by reshaping, then a lexicographic ranking."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 700, 700 + 2500])
    T = int(cu[-1])
    IQ = rng.standard_normal((T, 4, 128)).astype(np.float32).astype(np.float64)
    IK = rng.standard_normal((T, 4, 128)).astype(np.float32).astype(np.float64)
    qs = list(range(0, T, 37)) + [T - 1, 699, 700]
    got, _ = O.index_select(IQ, IK, cu, queries=qs)
    for d in range(len(cu) - 1):
        c0, L = int(cu[d]), int(cu[d + 1] - cu[d])
        nbd = -(-L // BLK)
        for i in range(4):
            S = IQ[c0:c0 + L, i] @ IK[c0:c0 + L, i].T          # [L, L]
            S = np.where(np.tril(np.ones((L, L), bool)), S, -np.inf)
            Sp = np.full((L, nbd * BLK), -np.inf)
            Sp[:, :L] = S
            B = Sp.reshape(L, nbd, BLK).max(axis=2)              # [L, nbd]
            for t in qs:
                if not (c0 <= t < c0 + L):
                    continue
                p = t - c0
                nb = p // BLK + 1
                ids = np.arange(nb)
                rank = np.lexsort((ids, -B[p, :nb]))[:16]
                want = sorted(rank.tolist()) + [-1] * (16 - min(16, nb))
                assert got[i, t].tolist() == want, (d, i, t)
