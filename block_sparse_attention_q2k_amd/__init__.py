"""Python binding of libmsa, the MI355X (gfx950) MSA prefill forward/backward library.

Argument marshalling only: every step of the operator runs in the HIP kernels behind
the C ABI declared in ``include/msa.h``.  PyTorch provides device memory and streams.
The functions below carry the C names; ``MSA`` bundles one layout's buffers and runs
the call sequence (forward: CSR, plan, K/V alignment, forward; backward: preprocess,
task tables, backward).  If the library is not built, loading fails loudly -- there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB as _LIB_PATH

NUM_Q_HEADS, NUM_KV_HEADS, NUM_INDEX_HEADS, HEAD_DIM, BLOCK, TOPK = 64, 4, 4, 128, 128, 16
PLAN_MAX_LIST = 16 * 16
TILE_QUERIES, FWD_GROUP = 8, 16
DQ_ACCUM_FP32, DQ_ACCUM_BF16X2, DQ_RECOMPUTE, DQ_STORED, DQ_ACCUM_F16X2 = 0, 1, 2, 3, 4
Q2K_OUT_OF_RANGE, Q2K_DUPLICATE = 1, 2
PLAN_HEADER_WORDS, TASKS_HEADER_WORDS = 16, 64


class MSAError(RuntimeError):
    def __init__(self, fn, rc, text):
        super().__init__("%s failed: %d (%s)" % (fn, rc, text))
        self.rc = rc


class _Layout(ctypes.Structure):
    _fields_ = [("num_docs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("num_ws_tokens", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p),
                ("cu_ws", ctypes.c_void_p)]


_lib = None
EXPORTS = ["msa_layout_host", "msa_csr_scratch_bytes", "msa_csr_cols_capacity", "msa_plan_bytes",
           "msa_tasks_bytes", "msa_bwd_scratch_bytes", "msa_default_grid", "msa_align_kv",
           "msa_build_k2q_csr", "msa_plan", "msa_forward", "msa_backward_preprocess",
           "msa_tasks_meta_offset", "msa_build_tasks", "msa_backward", "msa_status_string",
           "msa_set_timing_events", "msa_build_k2q_csr_noalloc", "msa_index_select"]


def lib():
    """Load libmsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch bundles its own HIP runtime (soname libamdhip64.so.7) and its libraries
        # request it by the unversioned name; loading it first makes libmsa bind to
        # that same runtime instead of a second copy (which would crash the process).
        import torch  # noqa: F401
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmsa.so is not built (%s); run block_sparse_attention_q2k_amd.build"
                               % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        P, I, Z, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        LP = ctypes.POINTER(_Layout)
        sig = {
            "msa_layout_host": (I, [P, I, P, P]),
            "msa_csr_scratch_bytes": (Z, [LP]),
            "msa_csr_cols_capacity": (Z, [LP]),
            "msa_plan_bytes": (Z, [LP]),
            "msa_tasks_bytes": (Z, [LP, I]),
            "msa_bwd_scratch_bytes": (Z, [LP, I]),
            "msa_default_grid": (I, []),
            "msa_align_kv": (I, [P, P, LP, P, P, P, P, P]),
            "msa_build_k2q_csr": (I, [P, LP, P, P, P, P, Z, P]),
            "msa_build_k2q_csr_noalloc": (I, [P, LP, P, P, P, P]),
            "msa_index_select": (I, [P, P, LP, P, P]),
            "msa_plan": (I, [LP, P, P, Z, P]),
            "msa_forward": (I, [P, P, P, LP, P, F, P, P, P]),
            "msa_backward_preprocess": (I, [P, P, I, P, P]),
            "msa_tasks_meta_offset": (Z, [I]),
            "msa_build_tasks": (I, [LP, P, P, P, I, P, Z, P]),
            "msa_backward": (I, [P, P, P, P, P, P, P, P, P, P, I, LP, F, I, P, P, P, P, Z, P]),
            "msa_status_string": (ctypes.c_char_p, [I]),
            "msa_set_timing_events": (None, [P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(fn, rc):
    if rc != 0:
        raise MSAError(fn, rc, lib().msa_status_string(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(fn, name, t, dtype, shape=None, min_numel=None):
    """The C ABI sees only pointers, so a tensor of the wrong size would be read or written
    past its end on the GPU: require a contiguous tensor of this dtype and exact shape (or at
    least min_numel elements).  (The device is checked by _gpu, after all of these.)"""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: %s must be a torch tensor" % (fn, name))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s: %s has dtype %s, expected %s" % (fn, name, t.dtype, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s: %s has shape %s, expected %s" % (fn, name, tuple(t.shape), tuple(shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s: %s has %d elements, needs at least %d" % (fn, name, t.numel(), min_numel))
    if not t.is_contiguous():
        raise ValueError("%s: %s is not contiguous" % (fn, name))


def _gpu(fn, **tensors):
    """After the structural checks: every tensor argument must live on a GPU."""
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError("%s: %s is not on a GPU" % (fn, name))


def _dt():
    import torch
    return torch.bfloat16, torch.float32, torch.int32, torch.uint8


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def msa_layout_host(cu_seqlens):
    """(cu_ws int32 numpy [N+1], W) for host document offsets; raises on bad offsets."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    cu_ws = np.zeros_like(cu)
    W = ctypes.c_int32(0)
    _check("msa_layout_host", lib().msa_layout_host(cu.ctypes.data_as(ctypes.c_void_p), len(cu) - 1,
                                                   cu_ws.ctypes.data_as(ctypes.c_void_p),
                                                   ctypes.byref(W)))
    return cu_ws, int(W.value)


class Layout:
    """Packed-document layout: host offsets plus their device copies."""

    def __init__(self, cu_seqlens, device="cuda"):
        import torch
        self.cu_host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        self.cu_ws_host, self.W = msa_layout_host(self.cu_host)
        self.num_docs = len(self.cu_host) - 1
        self.T = int(self.cu_host[-1])
        self.NB = self.W // BLOCK
        self.cu = torch.from_numpy(self.cu_host).to(device)
        self.cu_ws = torch.from_numpy(self.cu_ws_host).to(device)
        self.c = _Layout(self.num_docs, self.T, self.W, self.cu.data_ptr(), self.cu_ws.data_ptr())

    def ref(self):
        return ctypes.byref(self.c)


def msa_csr_scratch_bytes(layout):
    return lib().msa_csr_scratch_bytes(layout.ref())


def msa_csr_cols_capacity(layout):
    return lib().msa_csr_cols_capacity(layout.ref())


def msa_plan_bytes(layout):
    return lib().msa_plan_bytes(layout.ref())


def msa_tasks_bytes(layout, grid):
    return lib().msa_tasks_bytes(layout.ref(), grid)


def msa_bwd_scratch_bytes(layout, mode):
    return lib().msa_bwd_scratch_bytes(layout.ref(), mode)


def msa_default_grid():
    return lib().msa_default_grid()


def msa_tasks_meta_offset(grid):
    return lib().msa_tasks_meta_offset(grid)


def msa_align_kv(K, V, layout, Kw, Vw, Kt, Vt, stream=None):
    bf, _, _, _ = _dt()
    for n, t in (("K", K), ("V", V)):
        _need("msa_align_kv", n, t, bf, (layout.T, NUM_KV_HEADS, HEAD_DIM))
    for n, t in (("Kw", Kw), ("Vw", Vw), ("Kt", Kt), ("Vt", Vt)):
        _need("msa_align_kv", n, t, bf, min_numel=layout.W * NUM_KV_HEADS * HEAD_DIM)
    _gpu("msa_align_kv", K=K, V=V, Kw=Kw, Vw=Vw, Kt=Kt, Vt=Vt)
    _check("msa_align_kv", lib().msa_align_kv(_ptr(K), _ptr(V), layout.ref(), _ptr(Kw), _ptr(Vw),
                                              _ptr(Kt), _ptr(Vt), _stream(stream)))


def _need_q2k(fn, q2k, layout):
    _need(fn, "q2k", q2k, _dt()[2], (NUM_INDEX_HEADS, layout.T, TOPK))


def msa_build_k2q_csr(q2k, layout, row_ptr, cols, status, scratch, stream=None):
    _, _, i32, _ = _dt()
    fn = "msa_build_k2q_csr"
    _need_q2k(fn, q2k, layout)
    _need(fn, "row_ptr", row_ptr, i32, min_numel=NUM_INDEX_HEADS * layout.NB + 1)
    _need(fn, "cols", cols, i32, min_numel=msa_csr_cols_capacity(layout))
    _need(fn, "status", status, i32, min_numel=1)
    _need(fn, "scratch", scratch, None)
    _gpu(fn, q2k=q2k, row_ptr=row_ptr, cols=cols, status=status, scratch=scratch)
    _check("msa_build_k2q_csr", lib().msa_build_k2q_csr(
        _ptr(q2k), layout.ref(), _ptr(row_ptr), _ptr(cols), _ptr(status), _ptr(scratch),
        scratch.numel() * scratch.element_size(), _stream(stream)))


def msa_build_k2q_csr_noalloc(q2k, layout, row_ptr, cols, status, stream=None):
    """msa_build_k2q_csr without a scratch argument: the library's own device array holds
    the counters (for callers that cannot allocate; calls on one GPU must not overlap)."""
    _, _, i32, _ = _dt()
    fn = "msa_build_k2q_csr_noalloc"
    _need_q2k(fn, q2k, layout)
    _need(fn, "row_ptr", row_ptr, i32, min_numel=NUM_INDEX_HEADS * layout.NB + 1)
    _need(fn, "cols", cols, i32, min_numel=msa_csr_cols_capacity(layout))
    _need(fn, "status", status, i32, min_numel=1)
    _gpu(fn, q2k=q2k, row_ptr=row_ptr, cols=cols, status=status)
    _check(fn, lib().msa_build_k2q_csr_noalloc(_ptr(q2k), layout.ref(), _ptr(row_ptr), _ptr(cols),
                                               _ptr(status), _stream(stream)))


def msa_index_select(IQ, IK, layout, q2k, stream=None):
    """The indexer's block selection: q2k int32 [4, T, 16] from index-Q / index-K bf16
    [T, 4, 128] (top-16 document-local causal blocks by their best visible key)."""
    bf, _, i32, _ = _dt()
    fn = "msa_index_select"
    for n, t in (("IQ", IQ), ("IK", IK)):
        _need(fn, n, t, bf, (layout.T, NUM_INDEX_HEADS, HEAD_DIM))
    _need(fn, "q2k", q2k, i32, (NUM_INDEX_HEADS, layout.T, TOPK))
    _gpu(fn, IQ=IQ, IK=IK, q2k=q2k)
    _check(fn, lib().msa_index_select(_ptr(IQ), _ptr(IK), layout.ref(), _ptr(q2k), _stream(stream)))


def msa_plan(layout, q2k, plan, stream=None):
    _need_q2k("msa_plan", q2k, layout)
    _need("msa_plan", "plan", plan, None)
    _gpu("msa_plan", q2k=q2k, plan=plan)
    _check("msa_plan", lib().msa_plan(layout.ref(), _ptr(q2k), _ptr(plan),
                                      plan.numel() * plan.element_size(), _stream(stream)))


def msa_forward(Q, Kw, Vt, layout, plan, scale, O, LSE, stream=None):
    bf, f32, _, _ = _dt()
    fn = "msa_forward"
    for n, t in (("Q", Q), ("O", O)):
        _need(fn, n, t, bf, (layout.T, NUM_Q_HEADS, HEAD_DIM))
    for n, t in (("Kw", Kw), ("Vt", Vt)):
        _need(fn, n, t, bf, min_numel=layout.W * NUM_KV_HEADS * HEAD_DIM)
    _need(fn, "LSE", LSE, f32, (layout.T, NUM_Q_HEADS))
    _need(fn, "plan", plan, None, min_numel=msa_plan_bytes(layout) // plan.element_size())
    _gpu(fn, Q=Q, Kw=Kw, Vt=Vt, plan=plan, O=O, LSE=LSE)
    _check("msa_forward", lib().msa_forward(_ptr(Q), _ptr(Kw), _ptr(Vt), layout.ref(), _ptr(plan),
                                            float(scale), _ptr(O), _ptr(LSE), _stream(stream)))


def msa_backward_preprocess(O, dO, num_tokens, delta, stream=None):
    bf, f32, _, _ = _dt()
    fn = "msa_backward_preprocess"
    for n, t in (("O", O), ("dO", dO)):
        _need(fn, n, t, bf, (int(num_tokens), NUM_Q_HEADS, HEAD_DIM))
    _need(fn, "delta", delta, f32, (int(num_tokens), NUM_Q_HEADS))
    _gpu(fn, O=O, dO=dO, delta=delta)
    _check("msa_backward_preprocess", lib().msa_backward_preprocess(
        _ptr(O), _ptr(dO), int(num_tokens), _ptr(delta), _stream(stream)))


def msa_build_tasks(layout, row_ptr, cols, q2k, grid, tasks, stream=None):
    _, _, i32, _ = _dt()
    fn = "msa_build_tasks"
    _need(fn, "row_ptr", row_ptr, i32, min_numel=NUM_INDEX_HEADS * layout.NB + 1)
    _need(fn, "cols", cols, i32, min_numel=msa_csr_cols_capacity(layout))
    _need_q2k(fn, q2k, layout)
    _need(fn, "tasks", tasks, None)
    _gpu(fn, row_ptr=row_ptr, cols=cols, q2k=q2k, tasks=tasks)
    _check("msa_build_tasks", lib().msa_build_tasks(layout.ref(), _ptr(row_ptr), _ptr(cols), _ptr(q2k),
                                                    int(grid), _ptr(tasks), tasks.numel() * tasks.element_size(),
                                                    _stream(stream)))


def msa_backward(Q, Kw, Vw, Kt, dO, LSE, delta, q2k, plan, tasks, grid, layout, scale, mode, dQ, dK,
                 dV, scratch, stream=None):
    bf, f32, _, _ = _dt()
    fn = "msa_backward"
    for n, t in (("Q", Q), ("dO", dO), ("dQ", dQ)):
        _need(fn, n, t, bf, (layout.T, NUM_Q_HEADS, HEAD_DIM))
    for n, t in (("Kw", Kw), ("Vw", Vw), ("Kt", Kt)):
        _need(fn, n, t, bf, min_numel=layout.W * NUM_KV_HEADS * HEAD_DIM)
    for n, t in (("dK", dK), ("dV", dV)):
        _need(fn, n, t, bf, (layout.T, NUM_KV_HEADS, HEAD_DIM))
    for n, t in (("LSE", LSE), ("delta", delta)):
        _need(fn, n, t, f32, (layout.T, NUM_Q_HEADS))
    _need_q2k(fn, q2k, layout)
    _need(fn, "plan", plan, None, min_numel=msa_plan_bytes(layout) // plan.element_size())
    _need(fn, "tasks", tasks, None, min_numel=msa_tasks_bytes(layout, int(grid)) // tasks.element_size())
    _need(fn, "scratch", scratch, None)
    _gpu(fn, Q=Q, Kw=Kw, Vw=Vw, Kt=Kt, dO=dO, LSE=LSE, delta=delta, q2k=q2k, plan=plan, tasks=tasks,
         dQ=dQ, dK=dK, dV=dV, scratch=scratch)
    _check("msa_backward", lib().msa_backward(
        _ptr(Q), _ptr(Kw), _ptr(Vw), _ptr(Kt), _ptr(dO), _ptr(LSE), _ptr(delta), _ptr(q2k),
        _ptr(plan), _ptr(tasks), int(grid),
        layout.ref(), float(scale), int(mode), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(scratch),
        scratch.numel() * scratch.element_size(), _stream(stream)))


TIMING_EVENTS = 6


def msa_set_timing_events(events):
    """events: TIMING_EVENTS torch.cuda.Event objects (already recorded once, so that
    the HIP events exist), or None to turn the hook off."""
    if events is None:
        lib().msa_set_timing_events(None)
        return
    assert len(events) == TIMING_EVENTS
    arr = (ctypes.c_void_p * TIMING_EVENTS)(*[e.cuda_event for e in events])
    lib().msa_set_timing_events(arr)


def _bytes(n, device):
    import torch
    return torch.empty(max(16, (int(n) + 15) // 16 * 16), dtype=torch.uint8, device=device)


class MSA:
    """Buffers of one layout plus the forward and backward call sequences."""

    def __init__(self, cu_seqlens, grid=None, dq_mode=DQ_STORED, device="cuda"):
        import torch
        self.layout = L = Layout(cu_seqlens, device)
        self.device = device
        self.grid = int(grid) if grid else msa_default_grid()
        self.fwd_group = FWD_GROUP
        self.dq_mode = dq_mode
        self.row_ptr = torch.empty(NUM_INDEX_HEADS * L.NB + 1, dtype=torch.int32, device=device)
        self.cols = torch.empty(msa_csr_cols_capacity(L), dtype=torch.int32, device=device)
        self.status = torch.zeros(4, dtype=torch.int32, device=device)
        self.csr_scratch = _bytes(msa_csr_scratch_bytes(L), device)
        self.plan = _bytes(msa_plan_bytes(L), device)
        self.tasks = _bytes(msa_tasks_bytes(L, self.grid), device)
        self.bwd_scratch = _bytes(msa_bwd_scratch_bytes(L, dq_mode), device)
        self.Kw = torch.empty((L.W, NUM_KV_HEADS, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.Vw = torch.empty_like(self.Kw)
        self.Kt = torch.empty_like(self.Kw)  # [4][W/128][128][128] transposed blocks
        self.Vt = torch.empty_like(self.Kw)
        self.delta = torch.empty((L.T, NUM_Q_HEADS), dtype=torch.float32, device=device)

    def select(self, IQ, IK, q2k=None, stream=None):
        """The indexer's block selection for this layout.  Returns q2k int32 [4, T, 16]."""
        import torch
        if q2k is None:
            q2k = torch.empty((NUM_INDEX_HEADS, self.layout.T, TOPK), dtype=torch.int32, device=self.device)
        msa_index_select(IQ, IK, self.layout, q2k, stream)
        return q2k

    def forward(self, Q, K, V, q2k, scale, O=None, LSE=None, stream=None):
        """CSR + plan + K/V alignment + forward.  Returns (O, LSE)."""
        import torch
        L = self.layout
        if O is None:
            O = torch.empty_like(Q)
        if LSE is None:
            LSE = torch.empty((L.T, NUM_Q_HEADS), dtype=torch.float32, device=self.device)
        msa_build_k2q_csr(q2k, L, self.row_ptr, self.cols, self.status, self.csr_scratch, stream)
        msa_plan(L, q2k, self.plan, stream)
        msa_align_kv(K, V, L, self.Kw, self.Vw, self.Kt, self.Vt, stream)
        msa_forward(Q, self.Kw, self.Vt, L, self.plan, scale, O, LSE, stream)
        self.q2k = q2k
        return O, LSE

    def backward(self, Q, dO, O, LSE, scale, dQ=None, dK=None, dV=None, stream=None):
        """Preprocess + task tables + backward (uses the CSR, plan, q2k and K/V workspace
        of the last forward).  Returns (dQ, dK, dV) in compact order."""
        import torch
        L = self.layout
        if dQ is None:
            dQ = torch.empty_like(Q)
        if dK is None:
            dK = torch.empty((L.T, NUM_KV_HEADS, HEAD_DIM), dtype=torch.bfloat16, device=self.device)
        if dV is None:
            dV = torch.empty_like(dK)
        if not hasattr(self, "q2k"):
            raise RuntimeError("MSA.backward needs the CSR, plan and workspace of a forward call first")
        msa_backward_preprocess(O, dO, L.T, self.delta, stream)
        msa_build_tasks(L, self.row_ptr, self.cols, self.q2k, self.grid, self.tasks, stream)
        msa_backward(Q, self.Kw, self.Vw, self.Kt, dO, LSE, self.delta, self.q2k, self.plan,
                     self.tasks, self.grid, L, scale, self.dq_mode, dQ, dK, dV, self.bwd_scratch,
                     stream)
        return dQ, dK, dV

    # ---- views of the integer structures (for checks)
    def csr(self):
        rp = self.row_ptr.cpu().numpy()
        return rp, self.cols[: int(rp[-1])].cpu().numpy()

    def plan_items(self):
        """(items int32 [n, 4] = {i, t0, n, doc}, walk lists [(block, mask)] per item)."""
        L = self.layout
        w = self.plan.view(torch_int32()).cpu().numpy()
        ni = 4 * ((L.T + FWD_GROUP - 1) // FWD_GROUP + L.num_docs)
        n = int(w[0])
        items = w[PLAN_HEADER_WORDS: PLAN_HEADER_WORDS + 4 * n].reshape(-1, 4)
        lens = w[PLAN_HEADER_WORDS + 4 * ni: PLAN_HEADER_WORDS + 4 * ni + n]
        base = PLAN_HEADER_WORDS + 4 * ni + (ni + 3) // 4 * 4
        lists = [w[base + 2 * PLAN_MAX_LIST * p: base + 2 * PLAN_MAX_LIST * p + 2 * int(lens[p])].reshape(-1, 2)
                 for p in range(n)]
        return items, lists

    def task_tables(self):
        w = self.tasks.view(torch_int32()).cpu().numpy()
        R, grid = int(w[0]), int(w[9])
        rmax = int(w[10])
        mo = msa_tasks_meta_offset(grid)
        meta = w[mo: mo + 4 * rmax].reshape(-1, 4)[:R]
        qrows = w[mo + 4 * rmax: mo + 12 * rmax].reshape(-1, 8)[:R]
        qpos = w[mo + 12 * rmax: mo + 20 * rmax].reshape(-1, 8)[:R]
        qtile = w[mo + 20 * rmax: mo + 28 * rmax].reshape(-1, 8)[:R]
        cta = w[TASKS_HEADER_WORDS: TASKS_HEADER_WORDS + 4 * (grid + 1)].reshape(4, grid + 1)
        return dict(R=R, head_rows=w[1:5].copy(), head_first=w[5:9].copy(), grid=grid, meta=meta,
                    qrows=qrows, qpos=qpos, qtile=qtile, cta=cta)


def torch_int32():
    import torch
    return torch.int32
