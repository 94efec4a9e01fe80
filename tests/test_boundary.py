"""The C ABI on the CPU: the library loads, exports what include/splr.h declares, and rejects bad
arguments before any HIP call (so these run without a GPU; no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from sparse_rank_linear_prune24_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, DTYPE, ALIGN, HIP, WORKSPACE, SCRATCH = range(8)
A = 0x10000          # an aligned, never dereferenced address
MIS = 0x10008        # misaligned


def header_functions():
    text = open(os.path.join(ROOT, "include", "splr.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\**(splr_[a-z0-9_]+)\(", text, re.M)))


def test_exports_match_header():
    declared = header_functions()
    assert set(declared) == set(binding.EXPORTS), declared
    lib = binding.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert binding.version().count(".") == 2


def test_status_strings():
    lib = binding.lib()
    for code in range(8):
        assert lib.splr_status_string(code).decode().startswith(binding.STATUS[code])
    assert lib.splr_status_string(99) == b"SPLR_ERR_UNKNOWN"


def test_pack_validation():
    f = binding.lib().splr_prune24_pack
    assert f(None, 4, 64, 1, A, A, None) == NULL
    assert f(A, 4, 64, 1, None, A, None) == NULL
    assert f(A, 0, 64, 1, A, A, None) == SHAPE
    assert f(A, 4, 48, 1, A, A, None) == SHAPE
    assert f(A, 4, 0, 1, A, A, None) == SHAPE
    assert f(A, -1, 64, 1, A, A, None) == SHAPE
    assert f(A, 1 << 25, 64, 1, A, A, None) == SHAPE
    assert f(A, 4, 64, 2, A, A, None) == DTYPE
    assert f(MIS, 4, 64, 1, A, A, None) == ALIGN
    assert f(A, 4, 64, 0, A, MIS, None) == ALIGN


def test_prune_nm_pack_validation():
    f = binding.lib().splr_prune_nm_pack
    assert f(None, 4, 64, 2, 8, 1, A, A, None) == NULL
    assert f(A, 4, 64, 2, 8, 1, None, A, None) == NULL
    assert f(A, 0, 64, 2, 8, 1, A, A, None) == SHAPE
    assert f(A, 4, 48, 2, 8, 1, A, A, None) == SHAPE
    for n, m in [(0, 4), (3, 4), (3, 8), (4, 8), (2, 6), (2, 32), (1, 2)]:
        assert f(A, 4, 64, n, m, 1, A, A, None) == SHAPE, (n, m)
    assert f(A, 4, 64, 2, 8, 2, A, A, None) == DTYPE
    assert f(MIS, 4, 64, 2, 8, 1, A, A, None) == ALIGN
    assert f(A, 4, 64, 1, 16, 0, A, MIS, None) == ALIGN


def test_pack_scaled_validation():
    f = binding.lib().splr_prune24_pack_scaled
    assert f(None, A, 4, 64, 1, A, A, None) == NULL
    assert f(A, None, 4, 64, 1, A, A, None) == NULL
    assert f(A, A, 4, 64, 1, None, A, None) == NULL
    assert f(A, A, 0, 64, 1, A, A, None) == SHAPE
    assert f(A, A, 4, 48, 1, A, A, None) == SHAPE
    assert f(A, A, 4, 64, 2, A, A, None) == DTYPE
    assert f(A, MIS, 4, 64, 1, A, A, None) == ALIGN
    assert f(MIS, A, 4, 64, 1, A, A, None) == ALIGN


def test_pack_residual_validation():
    f = binding.lib().splr_prune24_pack_residual
    assert f(None, A, A, 4, 64, 16, 1, A, A, None) == NULL
    assert f(A, None, A, 4, 64, 16, 1, A, A, None) == NULL
    assert f(A, A, None, 4, 64, 16, 1, A, A, None) == NULL
    assert f(A, A, A, 4, 64, 16, 1, None, A, None) == NULL
    assert f(A, A, A, 4, 64, -1, 1, A, A, None) == SHAPE
    assert f(A, A, A, 4, 64, 1025, 1, A, A, None) == SHAPE
    assert f(A, A, A, 4, 48, 16, 1, A, A, None) == SHAPE
    assert f(A, A, A, 0, 64, 16, 1, A, A, None) == SHAPE
    assert f(A, A, A, 4, 64, 16, 3, A, A, None) == DTYPE
    assert f(MIS, A, A, 4, 64, 16, 1, A, A, None) == ALIGN
    assert f(A, MIS, A, 4, 64, 16, 1, A, A, None) == ALIGN
    assert f(A, None, None, 4, 64, 0, 1, MIS, A, None) == ALIGN


def test_linear_ex_validation():
    import ctypes
    f = binding.lib().splr_linear_ex
    wsb = binding.lib().splr_linear_workspace_bytes(16, 32, 64, 16, 1)
    args = lambda yd, Y=A: (A, 16, 64, A, A, 32, A, A, 16, 1, yd, Y, A, wsb, None)
    assert f(*args(2)) == DTYPE
    assert f(*args(-1)) == DTYPE
    assert f(*args(1, None)) == NULL
    assert f(*args(1, MIS)) == ALIGN
    assert f(A, 16, 64, A, A, 32, A, A, 16, 1, 1, A, A, ctypes.c_size_t(0), None) == 6  # workspace too small


def test_packed_bytes():
    import ctypes
    f = binding.lib().splr_packed_bytes
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    assert f(17, 96, 1, ctypes.byref(vb), ctypes.byref(mb)) == OK
    assert (vb.value, mb.value) == (2 * 2 * 512 * 2, 2 * 1 * 1024)   # 2 tile rows x 1 metadata block of 1 KiB
    assert f(4096, 4096, 0, ctypes.byref(vb), ctypes.byref(mb)) == OK
    assert (vb.value, mb.value) == (4096 * 4096 // 2 * 4, 4096 * 4096 // 8)
    assert f(16, 48, 1, ctypes.byref(vb), ctypes.byref(mb)) == SHAPE
    assert f(16, 64, 9, ctypes.byref(vb), ctypes.byref(mb)) == DTYPE
    assert f(16, 64, 1, None, ctypes.byref(mb)) == NULL


def test_linear_validation():
    f = binding.lib().splr_linear
    ws = binding.lib().splr_linear_workspace_bytes
    good = dict(X=A, M=16, n_in=64, values=A, meta=A, n_out=32, U=A, V=A, r=16, dt=1, Y=A, ws=A,
                wsb=1 << 30, stream=None)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["X"], a["M"], a["n_in"], a["values"], a["meta"], a["n_out"], a["U"], a["V"], a["r"], a["dt"],
                 a["Y"], a["ws"], a["wsb"], a["stream"])

    assert call(X=None) == NULL
    assert call(Y=None) == NULL
    assert call(U=None) == NULL
    assert call(M=0) == SHAPE
    assert call(n_out=0) == SHAPE
    assert call(n_in=80) == SHAPE
    assert call(r=8) == SHAPE
    assert call(r=-16) == SHAPE
    assert call(r=2048) == SHAPE
    assert call(dt=7) == DTYPE
    assert call(X=MIS) == ALIGN
    assert call(V=MIS) == ALIGN
    assert call(Y=MIS) == ALIGN
    assert call(ws=None) == WORKSPACE
    assert call(wsb=ws(16, 32, 64, 16, 1) - 1) == WORKSPACE
    # r == 0: U, V may be NULL (this case would pass validation, so only the size query is checked)
    assert ws(16, 32, 64, 0, 1) == 0
    assert ws(16, 32, 64, 16, 1) > 0 and ws(2048, 4096, 4096, 64, 1) % 256 == 0
    assert ws(0, 32, 64, 16, 1) == 0


def test_stage_validation():
    lib = binding.lib()
    s1, s2 = lib.splr_linear_stage1, lib.splr_linear_stage2
    wsb = lib.splr_linear_workspace_bytes(16, 32, 64, 16, 1)
    # stage 1: X, V, workspace
    assert s1(None, 16, 64, A, 16, 1, A, wsb, None) == NULL
    assert s1(A, 16, 64, None, 16, 1, A, wsb, None) == NULL
    assert s1(A, 16, 40, A, 16, 1, A, wsb, None) == SHAPE
    assert s1(A, 0, 64, A, 16, 1, A, wsb, None) == SHAPE
    assert s1(A, 16, 64, A, 24, 1, A, wsb, None) == SHAPE
    assert s1(A, 16, 64, A, 16, 3, A, wsb, None) == DTYPE
    assert s1(A, 16, 64, MIS, 16, 1, A, wsb, None) == ALIGN
    assert s1(A, 16, 64, A, 16, 1, None, wsb, None) == WORKSPACE
    assert s1(A, 16, 64, A, 16, 1, A, wsb - 1, None) == WORKSPACE
    # stage 2: X, values, meta, U, Y, workspace (V is not an argument)
    assert s2(A, 16, 64, None, A, 32, A, 16, 1, A, A, wsb, None) == NULL
    assert s2(A, 16, 64, A, A, 32, None, 16, 1, A, A, wsb, None) == NULL
    assert s2(A, 16, 64, A, A, 32, A, 16, 1, None, A, wsb, None) == NULL
    assert s2(A, 16, 64, A, A, 0, A, 16, 1, A, A, wsb, None) == SHAPE
    assert s2(A, 16, 64, A, A, 32, A, 16, 1, A, MIS, wsb, None) == ALIGN
    assert s2(A, 16, 64, A, A, 32, MIS, 16, 1, A, A, wsb, None) == ALIGN
    assert s2(A, 16, 64, A, A, 32, A, 16, 1, A, None, wsb, None) == WORKSPACE

def test_stage2_dense_validation():
    """splr_linear_stage2_dense: stage 2's checks, and bfloat16 only."""
    lib = binding.lib()
    d = lib.splr_linear_stage2_dense
    wsb = lib.splr_linear_workspace_bytes(16, 32, 64, 16, 1)
    assert d(None, 16, 64, A, A, 32, A, 16, 1, A, A, wsb, None) == NULL
    assert d(A, 16, 64, None, A, 32, A, 16, 1, A, A, wsb, None) == NULL
    assert d(A, 16, 64, A, A, 32, None, 16, 1, A, A, wsb, None) == NULL
    assert d(A, 16, 64, A, A, 32, A, 16, 1, None, A, wsb, None) == NULL
    assert d(A, 16, 40, A, A, 32, A, 16, 1, A, A, wsb, None) == SHAPE
    assert d(A, 16, 64, A, A, 0, A, 16, 1, A, A, wsb, None) == SHAPE
    assert d(A, 16, 64, A, A, 32, A, 24, 1, A, A, wsb, None) == SHAPE
    assert d(A, 16, 64, A, A, 32, A, 16, 1, A, MIS, wsb, None) == ALIGN
    assert d(A, 16, 64, A, A, 32, A, 16, 1, A, None, wsb, None) == WORKSPACE
    assert d(A, 16, 64, A, A, 32, A, 16, 3, A, A, wsb, None) == DTYPE
    wsf = lib.splr_linear_workspace_bytes(16, 32, 64, 16, 0)
    assert d(A, 16, 64, A, A, 32, A, 16, 0, A, A, wsf, None) == DTYPE


def test_group_validation():
    """splr_linear_group / splr_linear_stage2_group: the count, the pointer arrays, and every layer's
    arguments as splr_linear checks them, all before any HIP call."""
    lib = binding.lib()
    g, g2 = lib.splr_linear_group, lib.splr_linear_stage2_group
    arr = lambda *p: (ctypes.c_void_p * len(p))(*p)
    wsb = lib.splr_linear_workspace_bytes(128, 512, 64, 16, 1)
    two = arr(A, A)
    # count
    for c in (0, -1, binding.GROUP_MAX + 1):
        assert g(c, two, 128, 64, two, two, 512, two, two, 16, 1, two, two, wsb, None) == SHAPE
        assert g2(c, two, 128, 64, two, two, 512, two, 16, 1, two, two, wsb, None) == SHAPE
    # missing arrays
    assert g(2, None, 128, 64, two, two, 512, two, two, 16, 1, two, two, wsb, None) == NULL
    assert g(2, two, 128, 64, two, two, 512, two, None, 16, 1, two, two, wsb, None) == NULL
    assert g(2, two, 128, 64, two, two, 512, two, two, 16, 1, two, None, wsb, None) == NULL
    assert g2(2, two, 128, 64, two, None, 512, two, 16, 1, two, two, wsb, None) == NULL
    assert g2(2, two, 128, 64, two, two, 512, None, 16, 1, two, two, wsb, None) == NULL
    # a missing or misaligned entry of the second layer
    assert g2(2, two, 128, 64, two, arr(A, None), 512, two, 16, 1, two, two, wsb, None) == NULL
    assert g2(2, two, 128, 64, two, two, 512, two, 16, 1, arr(A, MIS), two, wsb, None) == ALIGN
    assert g(2, two, 128, 64, two, two, 512, two, arr(A, MIS), 16, 1, two, two, wsb, None) == ALIGN
    # shapes, type and workspace, shared by the layers
    assert g2(2, two, 128, 40, two, two, 512, two, 16, 1, two, two, wsb, None) == SHAPE
    assert g2(2, two, 128, 64, two, two, 512, two, 24, 1, two, two, wsb, None) == SHAPE
    assert g2(2, two, 128, 64, two, two, 512, two, 16, 3, two, two, wsb, None) == DTYPE
    assert g2(2, two, 128, 64, two, two, 512, two, 16, 1, two, two, wsb - 1, None) == WORKSPACE
    assert g2(2, two, 128, 64, two, two, 512, two, 16, 1, two, arr(A, None), wsb, None) == WORKSPACE


def test_reconstruct_validation():
    f = binding.lib().splr_dense_reconstruct
    assert f(None, A, A, A, 4, 64, 16, 1, A, None) == NULL
    assert f(A, A, None, A, 4, 64, 16, 1, A, None) == NULL
    assert f(A, A, A, A, 4, 40, 16, 1, A, None) == SHAPE
    assert f(A, A, A, A, 4, 64, 17, 1, A, None) == SHAPE
    assert f(A, A, A, A, 4, 64, 16, 5, A, None) == DTYPE
    assert f(A, A, A, A, 4, 64, 16, 1, MIS, None) == ALIGN


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        binding.prune24_pack(torch.zeros((4, 64), dtype=torch.bfloat16))


def test_version_names_the_sources():
    """splr_version() carries the hash of the sources the library was built from."""
    from sparse_rank_linear_prune24_amd import build
    assert binding.version() == "0.2.0+" + build.source_hash()


NO_GPU = not os.path.exists("/dev/kfd")


@pytest.mark.skipif(not NO_GPU, reason="reaches a kernel launch with placeholder pointers: only without a GPU")
def test_largest_sizes_pass_validation():
    """The largest sizes the ABI accepts pass every check, including the dispatch limits of each
    launch (grids of up to 2^24 rows or tokens): with no GPU present the call then fails at the
    launch (SPLR_ERR_HIP), not in validation. One step beyond a limit is SPLR_ERR_SHAPE."""
    lib = binding.lib()
    rows, cols = 1 << 24, 4096              # rows * cols = 2^36 elements, the largest matrix
    big = 1 << 40
    for dt in (0, 1):
        assert lib.splr_prune24_pack(A, rows, cols, dt, A, A, None) == HIP
        assert lib.splr_prune24_pack(A, rows + 1, cols, dt, A, A, None) == SHAPE
        assert lib.splr_prune24_pack(A, rows, cols + 32, dt, A, A, None) == SHAPE
        assert lib.splr_prune24_pack_scaled(A, A, rows, cols, dt, A, A, None) == HIP
        assert lib.splr_prune_nm_pack(A, rows, cols, 2, 8, dt, A, A, None) == HIP
        assert lib.splr_prune24_pack_residual(A, A, A, rows, cols, 1024, dt, A, A, None) == HIP
        assert lib.splr_dense_reconstruct(A, A, A, A, rows, cols, 1024, dt, A, None) == HIP
        assert lib.splr_dense_reconstruct(A, A, A, A, rows, cols + 32, 1024, dt, A, None) == SHAPE
        # tokens x outputs = 2^36, rank 1024 (float32: M * r = 2^34 first-stage outputs)
        for M, n_out in ((rows, cols), (cols, rows), (16, rows), (64, rows)):
            assert lib.splr_linear(A, M, cols, A, A, n_out, A, A, 1024, dt, A, A, big, None) == HIP, (dt, M, n_out)
            assert lib.splr_linear_stage1(A, M, cols, A, 1024, dt, A, big, None) == HIP
            assert lib.splr_linear_stage2(A, M, cols, A, A, n_out, A, 1024, dt, A, A, big, None) == HIP
            if dt == 1:
                assert lib.splr_linear_stage2_dense(A, M, cols, A, A, n_out, A, 1024, dt, A, A, big, None) == HIP
        assert lib.splr_linear(A, rows, cols, A, A, cols + 16, A, A, 1024, dt, A, A, big, None) == SHAPE


def test_linear_noalloc_validation():
    f = binding.lib().splr_linear_noalloc
    args = dict(X=A, M=16, n_in=64, values=A, meta=A, n_out=32, U=A, V=A, r=16, dt=1, Y=A, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["X"], a["M"], a["n_in"], a["values"], a["meta"], a["n_out"], a["U"], a["V"], a["r"], a["dt"],
                 a["Y"], a["stream"])

    assert call(X=None) == NULL
    assert call(V=None) == NULL
    assert call(n_in=48) == SHAPE
    assert call(r=8) == SHAPE
    assert call(dt=4) == DTYPE
    assert call(Y=MIS) == ALIGN
    # the built-in workspace holds 32 MiB: 16384 tokens at rank 1024 need more (checked before any HIP call)
    ws = binding.lib().splr_linear_workspace_bytes
    assert ws(16384, 4096, 4096, 1024, 1) > 32 << 20 and ws(16384, 4096, 4096, 1024, 0) > 32 << 20
    assert call(M=16384, n_in=4096, n_out=4096, r=1024) == SCRATCH
    assert call(M=16384, n_in=4096, n_out=4096, r=1024, dt=0) == SCRATCH


def test_cholqr_validation():
    lib = binding.lib()
    assert lib.splr_gram_workspace_bytes(4096, 80) == 128 * 80 * 80 * 8
    assert lib.splr_gram_workspace_bytes(33, 5) % 256 == 0 and lib.splr_gram_workspace_bytes(33, 5) >= 2 * 25 * 8
    assert lib.splr_gram_workspace_bytes(0, 8) == 0 and lib.splr_gram_workspace_bytes(8, 193) == 0
    g = lib.splr_gram_f64
    need = lib.splr_gram_workspace_bytes(64, 8)
    assert g(None, 64, 8, A, A, need, None) == NULL
    assert g(A, 64, 8, None, A, need, None) == NULL
    assert g(A, 0, 8, A, A, need, None) == SHAPE
    assert g(A, 64, 0, A, A, need, None) == SHAPE
    assert g(A, 64, 193, A, A, need, None) == SHAPE
    assert g(A, 64, 8, A, None, need, None) == WORKSPACE
    assert g(A, 64, 8, A, A, need - 1, None) == WORKSPACE
    assert g(A + 2, 64, 8, A, A, need, None) == ALIGN
    assert g(A, 64, 8, A + 4, A, need, None) == ALIGN
    c = lib.splr_chol_rinv
    assert c(None, 8, A, None) == NULL
    assert c(A, 8, None, None) == NULL
    assert c(A, 0, A, None) == SHAPE
    assert c(A, 193, A, None) == SHAPE
    assert c(A + 4, 8, A, None) == ALIGN
    assert c(A, 8, A + 2, None) == ALIGN
