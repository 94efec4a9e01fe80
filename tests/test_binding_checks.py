"""The Python binding checks every tensor against the sizes it passes to the C ABI, before the call.

The ABI sees only pointers, so a tensor of the wrong shape or type would be read or written out of
bounds by a kernel. These tests run on the CPU: the binding's device test is replaced so that host
tensors stand in for device tensors, and every case must raise ValueError before the library is
called (a call that got through would fail at its launch here, with no GPU). They are skipped where
a GPU is present, since a missed check would then hand host pointers to a kernel."""
import os

import pytest
import torch

from sparse_rank_linear_prune24_amd import binding

pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host tensors stand in for device tensors")


class _Stream:
    cuda_stream = 0


S = _Stream()
bf, f32 = torch.bfloat16, torch.float32


@pytest.fixture(autouse=True)
def host_as_device(monkeypatch):
    monkeypatch.setattr(binding, "_is_device", lambda t: True)


def layer(M=32, n_in=128, n_out=48, r=16, dt=bf):
    TR, TK = binding.tiles(n_out, n_in)
    return dict(X=torch.zeros(M, n_in, dtype=dt), values=torch.zeros(TR, TK, 64, 8, dtype=dt),
                meta=torch.zeros(binding.meta_shape(n_out, n_in), dtype=torch.int32), U=torch.zeros(n_out, r, dtype=dt),
                V=torch.zeros(r, n_in, dtype=dt), Y=torch.zeros(M, n_out, dtype=f32),
                ws=torch.zeros(1 << 20, dtype=torch.uint8), n_out=n_out)


def lin(d, **kw):
    a = dict(d, **kw)
    return binding.linear(a["X"], a["values"], a["meta"], a["U"], a["V"], n_out=a["n_out"], out=a["Y"],
                          workspace=a["ws"], stream=S)


def test_correct_shapes_reach_the_library():
    # with no GPU the call fails at its launch, after every check passed
    with pytest.raises(binding.SplrError, match="SPLR_ERR_HIP"):
        lin(layer())


@pytest.mark.parametrize("bad", [
    dict(V=torch.zeros(16, 96, dtype=bf)),                 # V columns != n_in
    dict(V=torch.zeros(32, 128, dtype=bf)),                # V rows != U's rank
    dict(U=torch.zeros(40, 16, dtype=bf)),                 # U rows != n_out
    dict(U=torch.zeros(48, 16, dtype=f32)),                # U dtype != X dtype
    dict(V=None),                                          # U without V
    dict(values=torch.zeros(3, 2, 64, 4, dtype=bf)),       # values too small for the tile grid
    dict(values=torch.zeros(3, 2, 64, 8, dtype=f32)),      # values dtype != X dtype
    dict(meta=torch.zeros(3, 1, 64, 2, dtype=torch.int32)),  # metadata too small
    dict(meta=torch.zeros(3, 1, 64, 4, dtype=torch.int64)),  # metadata not 32-bit
    dict(Y=torch.zeros(32, 48, dtype=bf)),                 # float32 Y expected
    dict(Y=torch.zeros(32, 32, dtype=f32)),                # Y too small
    dict(Y=torch.zeros(48, 32, dtype=f32).t()),            # not contiguous
    dict(X=torch.zeros(32, 128, dtype=torch.float16)),     # unsupported dtype
    dict(X=torch.zeros(32, 128, 1, dtype=bf)),             # not a matrix
])
def test_linear_rejects(bad):
    with pytest.raises((ValueError, TypeError)):
        lin(layer(), **bad)


def test_linear_ex_output_type():
    d = layer()
    with pytest.raises(ValueError):   # bf16 requested, float32 buffer given
        binding.linear_ex(d["X"], d["values"], d["meta"], d["U"], d["V"], y_dtype=bf, n_out=48, out=d["Y"],
                          workspace=d["ws"], stream=S)


def test_stages_reject():
    d = layer()
    with pytest.raises(ValueError):
        binding.linear_stage1(d["X"], torch.zeros(16, 64, dtype=bf), d["ws"], stream=S)
    with pytest.raises(ValueError):
        binding.linear_stage2(d["X"], d["values"], d["meta"], torch.zeros(47, 16, dtype=bf), d["ws"], n_out=48,
                              out=d["Y"], stream=S)
    with pytest.raises(ValueError):
        binding.linear_stage2(d["X"], d["values"], d["meta"], d["U"], d["ws"], n_out=48,
                              out=torch.zeros(32, 47, dtype=f32), stream=S)


def test_packs_reject():
    R = torch.zeros(48, 128, dtype=bf)
    d = layer()
    with pytest.raises(ValueError):
        binding.prune24_pack(R, torch.zeros(3, 2, 64, 4, dtype=bf), d["meta"], stream=S)
    with pytest.raises(ValueError):
        binding.prune24_pack(R, d["values"], torch.zeros(3, 1, 32, 4, dtype=torch.int32), stream=S)
    with pytest.raises(ValueError):
        binding.prune_nm_pack(R, 2, 8, d["values"].float(), d["meta"], stream=S)
    with pytest.raises(ValueError):
        binding.prune24_pack_scaled(R, torch.zeros(64), d["values"], d["meta"], stream=S)
    with pytest.raises(ValueError):
        binding.prune24_pack_residual(R, d["U"], torch.zeros(16, 64, dtype=bf), d["values"], d["meta"], stream=S)
    with pytest.raises(ValueError):
        binding.prune24_pack_residual(R, d["U"], None, d["values"], d["meta"], stream=S)


def test_reconstruct_rejects():
    d = layer()
    with pytest.raises(ValueError):
        binding.dense_reconstruct(d["values"], d["meta"], d["U"], d["V"], out=torch.zeros(48, 64), stream=S)
    with pytest.raises(ValueError):
        binding.dense_reconstruct(d["values"], d["meta"], d["U"], torch.zeros(16, 64, dtype=bf), stream=S)
