"""Host-side checks of the C ABI (no GPU needed): every symbol declared in
include/msa.h is exported by libmsa.so; layout and size queries; argument errors are
returned before anything touches a device."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def M():
    import block_sparse_attention_q2k_amd as M
    if not os.path.exists(M._LIB_PATH):
        from block_sparse_attention_q2k_amd import build
        build.build()
    M.lib()
    return M


def declared_functions():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(M):
    names = declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(M._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(M.EXPORTS)


def test_layout_host(M):
    cu_ws, W = M.msa_layout_host([0, 1, 129, 258, 386])
    assert list(cu_ws) == [0, 128, 256, 512, 640] and W == 640
    for bad in ([1, 5], [0, 5, 5], [0, 7, 3]):
        with pytest.raises(M.MSAError):
            M.msa_layout_host(bad)


class FakeLayout:
    """A layout struct whose device pointers are aligned host addresses: only valid for
    calls that must fail before any device access."""

    def __init__(self, M, T=1000, W=1024, N=1):
        self.buf = np.zeros(64, dtype=np.int32)
        p = (self.buf.ctypes.data + 15) // 16 * 16
        self.c = M._Layout(N, T, W, p, p)

    def ref(self):
        return ctypes.byref(self.c)


def test_size_queries(M):
    L = FakeLayout(M, T=16384, W=16384)
    assert M.msa_csr_scratch_bytes(L) == 4 * 128 * 4
    assert M.msa_csr_cols_capacity(L) == 4 * 16384 * 16
    assert M.msa_plan_bytes(L) > 4 * 4 * (16384 // 16)
    assert M.msa_tasks_bytes(L, 512) > M.msa_tasks_bytes(L, 256) > 0
    assert M.msa_tasks_bytes(L, 0) == 0
    f32 = M.msa_bwd_scratch_bytes(L, 0)
    b16 = M.msa_bwd_scratch_bytes(L, 1)
    rec = M.msa_bwd_scratch_bytes(L, 2)
    assert f32 - b16 == 16384 * 64 * 128 * 2
    assert rec == 2 * 16384 * 4 * 128 * 4
    assert M.msa_bwd_scratch_bytes(L, 7) == 0
    bad = FakeLayout(M, T=1000, W=1000)  # W not a multiple of 128
    assert M.msa_plan_bytes(bad) == 0


def test_argument_errors_return_before_device_use(M):
    lib = M.lib()
    L = FakeLayout(M)
    buf = np.zeros(4096, dtype=np.uint8)
    a = ctypes.c_void_p((buf.ctypes.data + 15) // 16 * 16)
    mis = ctypes.c_void_p(a.value + 4)
    null = None
    E = dict(NULL=1, ALIGN=2, SHAPE=3, SCRATCH=4, MODE=5, GRID=6)
    assert lib.msa_align_kv(a, a, L.ref(), a, null, a, a, None) == E["NULL"]
    assert lib.msa_align_kv(a, a, L.ref(), a, mis, a, a, None) == E["ALIGN"]
    assert lib.msa_build_k2q_csr(a, L.ref(), a, a, a, a, 1, None) == E["SCRATCH"]
    assert lib.msa_plan(L.ref(), a, a, 16, None) == E["SCRATCH"]
    assert lib.msa_forward(a, a, a, L.ref(), a, ctypes.c_float(-1.0), a, a, None) == E["SHAPE"]
    assert lib.msa_backward_preprocess(a, a, 0, a, None) == E["SHAPE"]
    assert lib.msa_build_tasks(L.ref(), a, a, a, 0, a, 1 << 30, None) == E["GRID"]
    bw = lambda grid, mode, nbytes: lib.msa_backward(a, a, a, a, a, a, a, a, a, a, grid, L.ref(),
                                                     ctypes.c_float(0.1), mode, a, a, a, a, nbytes, None)
    assert bw(256, 9, 1 << 40) == E["MODE"]
    assert bw(0, 2, 1 << 40) == E["GRID"]
    assert bw(256, 0, 16) == E["SCRATCH"]
    assert bw(256, 2, 16) == E["SCRATCH"]
    # the softmax scale must be finite and positive (checked before the device)
    for sc in (0.0, -0.5, float("nan"), float("inf")):
        assert lib.msa_forward(a, a, a, L.ref(), a, ctypes.c_float(sc), a, a, None) == E["SHAPE"], sc
        assert lib.msa_backward(a, a, a, a, a, a, a, a, a, a, 256, L.ref(), ctypes.c_float(sc), 2, a, a, a, a,
                                1 << 40, None) == E["SHAPE"], sc
    assert lib.msa_index_select(a, null, L.ref(), a, None) == E["NULL"]
    assert lib.msa_index_select(a, a, L.ref(), mis, None) == E["ALIGN"]
    assert lib.msa_index_select(a, a, None, a, None) == E["NULL"]
    bad = FakeLayout(M, T=1000, W=1000)
    assert lib.msa_align_kv(a, a, bad.ref(), a, a, a, a, None) == E["SHAPE"]
    assert lib.msa_index_select(a, a, bad.ref(), a, None) == E["SHAPE"]
    assert lib.msa_status_string(4) == b"buffer smaller than its size query"


def test_binding_refuses_tensors_the_kernels_would_overrun(M):
    """The binding checks dtype, shape, contiguity and device before any pointer reaches the
    library (which sees only pointers)."""
    import torch
    L = M.Layout([0, 300, 700], device="cpu")
    T, W = L.T, L.W
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    Q = torch.zeros((T, 64, 128), dtype=bf)
    Kw = torch.zeros((W, 4, 128), dtype=bf)
    q2k = torch.full((4, T, 16), -1, dtype=i32)
    plan = torch.zeros(M.msa_plan_bytes(L), dtype=torch.uint8)
    LSE = torch.zeros((T, 64), dtype=f32)
    call = lambda **kw: M.msa_forward(**{**dict(Q=Q, Kw=Kw, Vt=Kw, layout=L, plan=plan, scale=0.1,
                                                O=Q, LSE=LSE), **kw})
    with pytest.raises(ValueError, match="dtype"):
        call(Q=Q.float())
    with pytest.raises(ValueError, match="shape"):
        call(O=torch.zeros((T - 1, 64, 128), dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        call(LSE=torch.zeros((T, 32), dtype=f32))
    with pytest.raises(ValueError, match="at least"):
        call(Kw=torch.zeros((W - 128, 4, 128), dtype=bf))
    with pytest.raises(ValueError, match="contiguous"):
        call(Q=torch.zeros((64, T, 128), dtype=bf).transpose(0, 1))
    with pytest.raises(ValueError, match="not on a GPU"):
        call()
    with pytest.raises(TypeError):
        call(LSE=np.zeros((T, 64), dtype=np.float32))
    with pytest.raises(ValueError, match="shape"):
        M.msa_backward_preprocess(Q, Q, T, torch.zeros((T, 63), dtype=f32))
    IQ = torch.zeros((T, 4, 128), dtype=bf)
    with pytest.raises(ValueError, match="shape"):
        M.msa_index_select(IQ, torch.zeros((T, 4, 64), dtype=bf), L, q2k)
    with pytest.raises(ValueError, match="dtype"):
        M.msa_index_select(IQ, IQ, L, q2k.to(torch.int64))
    with pytest.raises(ValueError, match="not on a GPU"):
        M.msa_index_select(IQ, IQ, L, q2k)
    m = M.MSA([0, 300, 700], grid=8, device="cpu")
    with pytest.raises(RuntimeError, match="forward"):
        m.backward(Q, Q, Q, LSE, 0.1)


def test_product_path_has_no_oracle_dependency():
    """The package neither imports nor loads anything under oracle/."""
    pkg = os.path.join(ROOT, "block_sparse_attention_q2k_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.lower(), f


def test_bench_traffic_digest_covers_existing_sources():
    """bench.py reports recorded HBM traffic only for the build it was measured on; every
    file of that digest must exist (a renamed source would otherwise break the bench)."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    for f in bench.TRAFFIC_SOURCES:
        assert os.path.exists(os.path.normpath(os.path.join(root, "block_sparse_attention_q2k_amd", "csrc", f))), f
    assert len(bench.sources_digest()) == 64
