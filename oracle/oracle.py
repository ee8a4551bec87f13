"""Plain CPU oracle for MiniMax Sparse Attention (MSA) prefill forward and backward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It shares no
code with the HIP library (``block_sparse_attention_q2k_amd``) and never imports it.

Floating point: ``msa_oracle.c`` (fp64, OpenMP), loaded through ctypes.  Integer
structure (layout, k2q CSR, forward plan, backward task tables): numpy here, written as
the plain definitions.  Citations name the page and its section:

* [PR] -- "feat(minimax-m3): add SM100 MSA sparse attention with custom backward"
  (NVIDIA-NeMo Automodel pull request 3809), sections Design / Supported scope /
  Custom kernel / Attention-operator benchmark.
* [BWD] -- API page of ``kernels.msa_backward_sm100`` (module summary, class
  constants, ``run_backward``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libmsa_oracle.so")

# Fixed topology of the operator ([PR] Supported scope): 64 query heads, 4 KV heads,
# 4 index heads, head dim 128, key block 128, top-k 16.
TILE_QUERIES = 8  # queries per backward task row: 8 queries x 16 heads = 128 rows ([BWD] summary)


def build(force: bool = True) -> str:
    """Compile msa_oracle.c with gcc (fp64, OpenMP) into oracle/_build."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i32, dbl, ptr = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.msa_oracle_forward.argtypes = [i32] * 8 + [ptr] * 5 + [dbl, ptr, ptr, ptr]
        lib.msa_oracle_backward.argtypes = [i32] * 8 + [ptr] * 6 + [dbl] + [ptr] * 7
        lib.msa_oracle_delta.argtypes = [i32, i32, i32, ptr, ptr, ptr]
        lib.msa_oracle_validate.argtypes = [i32] * 5 + [ptr, ptr]
        for f in (lib.msa_oracle_forward, lib.msa_oracle_backward, lib.msa_oracle_delta,
                  lib.msa_oracle_validate):
            f.restype = ctypes.c_int
        _lib_handle = lib
    return _lib_handle


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    a = np.asarray(a, dtype=np.float64)
    return np.ascontiguousarray(a)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# --------------------------------------------------------------------------------------
# Packed-document layout ([PR] Design: documents padded to a multiple of 128 tokens in
# the attention K/V workspace; [BWD] run_backward: W a positive multiple of 128).
# --------------------------------------------------------------------------------------
def layout(cu_seqlens, blk: int = 128):
    """Return (cu_ws, W, NB): workspace offsets of each document (each document padded
    to a multiple of ``blk`` rows), the workspace length and its block count."""
    cu = _i32(cu_seqlens)
    lens = np.diff(cu)
    padded = ((lens + blk - 1) // blk) * blk
    cu_ws = np.zeros(len(cu), dtype=np.int32)
    cu_ws[1:] = np.cumsum(padded)
    W = int(cu_ws[-1])
    return cu_ws, W, W // blk


def coords(cu_seqlens, blk: int = 128):
    """Per compact token t: (doc(t), pos(t), blk(t)) ([PR] Design: the layout carries
    document offsets and token coordinates)."""
    cu = _i32(cu_seqlens)
    T = int(cu[-1])
    t = np.arange(T)
    doc = np.searchsorted(cu, t, side="right") - 1
    pos = t - cu[doc]
    return doc.astype(np.int64), pos.astype(np.int64), (pos // blk).astype(np.int64)


def align_kv(X, cu_seqlens, blk: int = 128):
    """Place compact K or V rows [T, ...] into the 128-aligned workspace [W, ...]; rows
    past each document's end are zero ([PR] Design; [BWD] run_backward)."""
    cu_ws, W, _ = layout(cu_seqlens, blk)
    doc, pos, _ = coords(cu_seqlens, blk)
    out = np.zeros((W,) + X.shape[1:], dtype=X.dtype)
    out[cu_ws[doc] + pos] = X
    return out


def gather_ws(Xw, cu_seqlens, blk: int = 128):
    """Inverse of align_kv: workspace rows of the real tokens, in compact order."""
    cu_ws, _, _ = layout(cu_seqlens, blk)
    doc, pos, _ = coords(cu_seqlens, blk)
    return Xw[cu_ws[doc] + pos]


def member_slots(q2k, cu_seqlens, blk: int = 128):
    """Boolean [HI, T, TOPK]: slot j of (i, t) names a member of Sel(i, t) that can hold
    keys, i.e. an id in [0, blk(t)] not listed in an earlier slot of the same row
    (-1 marks unused slots; [PR] Design)."""
    q = _i32(q2k)
    _, _, blk_t = coords(cu_seqlens, blk)
    ok = (q >= 0) & (q <= blk_t[None, :, None])
    topk = q.shape[2]
    first = np.ones_like(ok)
    for j in range(1, topk):
        first[:, :, j] = ~np.any(q[:, :, :j] == q[:, :, j:j + 1], axis=2)
    return ok & first


def validate(q2k, cu_seqlens, blk: int = 128) -> int:
    """Precondition flags of q2k: 1 = id outside [-1, blk(t)], 2 = id repeated in a row.
    (Plain C loop in msa_oracle.c.)"""
    cu = _i32(cu_seqlens)
    q = _i32(q2k)
    HI, T, TOPK = q.shape
    return int(_lib().msa_oracle_validate(T, HI, blk, TOPK, len(cu) - 1, _p(cu), _p(q)))


# --------------------------------------------------------------------------------------
# k2q CSR: inversion of query->key-block lists into key-block->query lists ([PR] Design:
# forward CSR/schedule; bindings page: build_k2q_csr).
# --------------------------------------------------------------------------------------
def k2q_csr(q2k, cu_seqlens, blk: int = 128):
    """Row r = i*NB + gb with gb = cu_ws[doc(t)]/blk + b the workspace block of
    document-local block b.  Returns (row_ptr [HI*NB+1], cols [nnz]) with each row's
    query ids ascending (the canonical order)."""
    q = _i32(q2k)
    HI, T, TOPK = q.shape
    cu_ws, W, NB = layout(cu_seqlens, blk)
    doc, _, _ = coords(cu_seqlens, blk)
    mem = member_slots(q, cu_seqlens, blk)
    i_idx, t_idx, j_idx = np.nonzero(mem)  # lexicographic (i, t, j)
    gb = cu_ws[doc[t_idx]] // blk + q[i_idx, t_idx, j_idx]
    rows = i_idx.astype(np.int64) * NB + gb
    order = np.argsort(rows, kind="stable")  # stable: t ascending within a row
    cols = t_idx[order].astype(np.int32)
    counts = np.bincount(rows, minlength=HI * NB)
    row_ptr = np.zeros(HI * NB + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr, cols


# --------------------------------------------------------------------------------------
# Forward plan: the query-parallel forward's work list.
# --------------------------------------------------------------------------------------
def forward_plan(q2k, cu_seqlens, nq: int, blk: int = 128):
    """Work items {i, t0, n, doc}: each document is cut into groups of ``nq``
    consecutive queries (last one shorter); every index head i has the same groups.
    Each head's groups are ordered by cost = number of member slots, descending, ties
    by document order; the heads are interleaved (item p belongs to head p % HI and is
    that head's (p // HI)-th item).  Each item also carries its walk list: the member
    blocks of its queries in ascending order, each with the bit mask of the queries
    (bit u = query t0 + u) that list it.  Returns (items int32 [HI*G, 4], costs
    [HI*G], lists: list of int32 [len, 2] arrays (block, mask))."""
    q = _i32(q2k)
    HI = q.shape[0]
    cu = _i32(cu_seqlens)
    mem = member_slots(q, cu, blk)
    per_tok = mem.sum(axis=2)  # [HI, T]
    groups = []
    for d in range(len(cu) - 1):
        for t0 in range(int(cu[d]), int(cu[d + 1]), nq):
            groups.append((t0, min(nq, int(cu[d + 1]) - t0), d))
    G = len(groups)
    items = np.zeros((HI * G, 4), dtype=np.int32)
    costs = np.zeros(HI * G, dtype=np.int32)
    lists = [None] * (HI * G)
    for i in range(HI):
        c = np.array([per_tok[i, t0:t0 + n].sum() for (t0, n, _) in groups], dtype=np.int64)
        order = sorted(range(G), key=lambda g: (-c[g], g))
        for rank, g in enumerate(order):
            p = rank * HI + i
            t0, n, d = groups[g]
            items[p] = (i, t0, n, d)
            costs[p] = c[g]
            masks = {}
            for u in range(n):
                for j in np.nonzero(mem[i, t0 + u])[0]:
                    b = int(q[i, t0 + u, j])
                    masks[b] = masks.get(b, 0) | (1 << u)
            # masks are 32-bit patterns: bit 31 is stored as the int32 sign bit
            lists[p] = (np.array(sorted(masks.items()), dtype=np.int64).reshape(-1, 2)
                        .astype(np.uint32).view(np.int32))
    return items, costs, lists


# --------------------------------------------------------------------------------------
# Backward task tables + CTA walk ([BWD] summary: task rows of 8 queries x 16 heads,
# bucketed by (index head, key block); [PR] Changelog: exact counts, CTA scheduling).
# --------------------------------------------------------------------------------------
def tasks(row_ptr, cols, cu_seqlens, num_index_heads: int, grid: int, blk: int = 128, q2k=None):
    """Task rows in ascending bucket order r; bucket r holds ceil(count_r / 8) rows and
    row k of it carries cols[row_ptr[r] + 8k : +8] (-1 padded).  Returns a dict:
    meta int32 [R, 4] = (r, n_valid, flags, k) with flags bit0 = first row of its
    bucket, bit1 = last; qrows int32 [R, 8]; qpos int32 [R, 8] (document-local
    positions, -1 padded); R; per-head row counts; cta [HI, grid+1] row bounds: in
    index head i, workgroup c walks rows [cta[i, c], cta[i, c+1]), with
    cta[i, c] = off_i + floor(c * R_i / grid).  With q2k given, also qslot int32 [R, 8]:
    the first of the 16 q2k slots of (index head, query) that lists the bucket's
    document-local block (-1 padded)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    _, pos, _ = coords(cu_seqlens, blk)
    nrows = len(row_ptr) - 1
    NB = nrows // num_index_heads
    meta, qrows, qpos, qslot = [], [], [], []
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ws = np.concatenate([[0], np.cumsum((np.diff(cu) + blk - 1) // blk * blk)])
    for r in range(nrows):
        c0, c1 = int(row_ptr[r]), int(row_ptr[r + 1])
        ntile = (c1 - c0 + TILE_QUERIES - 1) // TILE_QUERIES
        for k in range(ntile):
            ids = cols[c0 + TILE_QUERIES * k: min(c1, c0 + TILE_QUERIES * (k + 1))]
            flags = (1 if k == 0 else 0) | (2 if k == ntile - 1 else 0)
            meta.append((r, len(ids), flags, k))
            pad = TILE_QUERIES - len(ids)
            qrows.append(list(ids) + [-1] * pad)
            qpos.append([int(pos[t]) for t in ids] + [-1] * pad)
            if q2k is not None:
                i, gb = r // NB, r % NB
                d = int(np.searchsorted(ws, gb * blk, side="right") - 1)  # document of block gb
                bl = gb - int(ws[d]) // blk
                sl = []
                for t in ids:
                    sel = [int(x) for x in q2k[i, t]]
                    sl.append(sel.index(bl))
                qslot.append(sl + [-1] * pad)
    R = len(meta)
    meta = np.array(meta, dtype=np.int32).reshape(R, 4)
    qrows = np.array(qrows, dtype=np.int32).reshape(R, TILE_QUERIES)
    qpos = np.array(qpos, dtype=np.int32).reshape(R, TILE_QUERIES)
    head_rows = np.array([np.sum(meta[:, 0] // NB == i) for i in range(num_index_heads)],
                         dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(head_rows)])
    cta = np.zeros((num_index_heads, grid + 1), dtype=np.int64)
    for i in range(num_index_heads):
        for c in range(grid + 1):
            cta[i, c] = off[i] + (c * head_rows[i]) // grid
    out = dict(meta=meta, qrows=qrows, qpos=qpos, R=R, head_rows=head_rows, cta=cta)
    if q2k is not None:
        out["qslot"] = np.array(qslot, dtype=np.int32).reshape(R, TILE_QUERIES)
    return out


# --------------------------------------------------------------------------------------
# Floating point: forward / backward / delta in fp64 (msa_oracle.c).
# --------------------------------------------------------------------------------------
def _dims(Q, K, q2k):
    T, H, D = Q.shape
    HKV = K.shape[1]
    HI, _, TOPK = q2k.shape
    return T, H, HKV, HI, D, TOPK


def forward(Q, K, V, q2k, cu_seqlens, scale, rows=None, blk: int = 128):
    """O [T,H,D] (fp64) and LSE [T,H] (natural log, scale included) of the exact
    forward.  ``rows``: optional boolean [T]; then only those rows are computed and
    (O[rows], LSE[rows]) are returned, in ascending row order."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    q = _i32(q2k)
    cu = _i32(cu_seqlens)
    T, H, HKV, HI, D, TOPK = _dims(Q, K, q)
    # untouched pages of np.empty are never materialised
    O = np.empty((T, H, D))
    LSE = np.empty((T, H))
    mask = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.uint8))
    rc = _lib().msa_oracle_forward(T, H, HKV, HI, D, blk, TOPK, len(cu) - 1, _p(cu), _p(Q),
                                   _p(K), _p(V), _p(q), float(scale), _p(mask), _p(O), _p(LSE))
    if rc:
        raise RuntimeError("msa_oracle_forward failed (%d)" % rc)
    if rows is None:
        return O, LSE
    idx = np.nonzero(np.asarray(rows, dtype=bool))[0]
    return O[idx], LSE[idx]


def backward(Q, K, V, dO, q2k, cu_seqlens, scale, q_rows=None, k_tokens=None, blk: int = 128):
    """Exact fp64 gradients (dQ [T,H,D], dK [T,HKV,D], dV [T,HKV,D]) of the exact
    forward, plus its LSE and delta [T,H].  ``q_rows`` selects dQ rows, ``k_tokens``
    the key tokens whose dK/dV rows are wanted (boolean [T] each; None = all); with a
    selection, dQ[q_rows] / dK[k_tokens] / dV[k_tokens] are returned in ascending token
    order, and LSE/delta are valid only on rows the selection needed."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    q = _i32(q2k)
    cu = _i32(cu_seqlens)
    T, H, HKV, HI, D, TOPK = _dims(Q, K, q)
    dQ = np.empty((T, H, D))
    dK = np.empty((T, HKV, D))
    dV = np.empty((T, HKV, D))
    LSE = np.empty((T, H))
    dl = np.empty((T, H))
    qm = None if q_rows is None else np.ascontiguousarray(np.asarray(q_rows, dtype=np.uint8))
    km = None if k_tokens is None else np.ascontiguousarray(np.asarray(k_tokens, dtype=np.uint8))
    rc = _lib().msa_oracle_backward(T, H, HKV, HI, D, blk, TOPK, len(cu) - 1, _p(cu), _p(Q),
                                    _p(K), _p(V), _p(dO), _p(q), float(scale), _p(qm), _p(km),
                                    _p(dQ), _p(dK), _p(dV), _p(LSE), _p(dl))
    if rc:
        raise RuntimeError("msa_oracle_backward failed (%d)" % rc)
    if q_rows is not None:
        dQ = dQ[np.nonzero(np.asarray(q_rows, dtype=bool))[0]]
    if k_tokens is not None:
        kidx = np.nonzero(np.asarray(k_tokens, dtype=bool))[0]
        dK, dV = dK[kidx], dV[kidx]
    return dQ, dK, dV, LSE, dl


def delta(O, dO):
    """delta[t,h] = sum_c dO[t,h,c] O[t,h,c] ([PR] Custom kernel: delta preprocessing)."""
    O, dO = _f64(O), _f64(dO)
    T, H, D = O.shape
    out = np.empty((T, H))
    _lib().msa_oracle_delta(T, H, D, _p(O), _p(dO), _p(out))
    return out


# --------------------------------------------------------------------------------------
# Work accounting (block-granular effective FLOPs: every member block counts all its
# 128 keys; 4*D flops per (query-head row, key) forward, 10*D backward).
# --------------------------------------------------------------------------------------
def effective_flops(q2k, cu_seqlens, num_heads: int = 64, head_dim: int = 128, blk: int = 128):
    mem = member_slots(q2k, cu_seqlens, blk)
    HI = mem.shape[0]
    slots = int(mem.sum())
    rows_per_slot = num_heads // HI
    fwd = 4.0 * head_dim * blk * rows_per_slot * slots
    bwd = 10.0 * head_dim * blk * rows_per_slot * slots
    return fwd, bwd, slots


def index_select(IQ, IK, cu_seqlens, topk: int = 16, blk: int = 128, queries=None):
    """Document-local top-k block selection of the indexer: the q2k the operator consumes.

    [PR] Design: the indexer selects a document-local q2k for every (index head, query)
    and may align index-K like the attention K; [PR] Supported scope: 4 index heads,
    head dim 128, block 128, top-k 16; [PR] Testing: truncated top-16 support.  The pages
    do not give the scoring rule.  The reading taken here: the score of document-local
    block b for index head i and the query at document position p is the largest
    <IQ[t, i], IK[j, i]> over the keys j of block b the query can see (j <= p); the
    selection is the min(16, p // 128 + 1) causal blocks of highest score, ties going to
    the smaller block id, listed in ascending id order with -1 in the unused slots.

    IQ, IK: [T, 4, 128] (any float dtype; computed in fp64).  queries: optional compact
    token ids to evaluate (default all).  Returns (q2k int32 [4, T, topk] with -1 rows
    for tokens not evaluated, scores dict (i, t) -> fp64 block scores of t's causal
    blocks) -- the scores let a caller judge near-ties at the selection boundary.
    """
    IQ = np.asarray(IQ, dtype=np.float64)
    IK = np.asarray(IK, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, HI, _ = IQ.shape
    q2k = np.full((HI, T, topk), -1, dtype=np.int32)
    scores = {}
    want = np.arange(T) if queries is None else np.asarray(queries, dtype=np.int64)
    doc_of = np.searchsorted(cu, np.arange(T), side="right") - 1
    for t in want:
        d = doc_of[t]
        c0 = cu[d]
        p = t - c0
        nb = p // blk + 1
        for i in range(HI):
            s = np.empty(nb, dtype=np.float64)
            for b in range(nb):
                keys = IK[c0 + b * blk:c0 + min(b * blk + blk, p + 1), i, :]
                s[b] = np.max(keys @ IQ[t, i, :])
            order = sorted(range(nb), key=lambda b: (-s[b], b))[:topk]
            sel = sorted(order)
            q2k[i, t, :len(sel)] = sel
            scores[(i, int(t))] = s
    return q2k, scores
