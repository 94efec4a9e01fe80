"""GPU parity of the grouped layer product (splr_linear_group, splr_linear_stage2_group).

Each layer's Y must equal its own splr_linear call bit for bit: the arithmetic of an output element
does not depend on which tile takes it or which layers share the grid. Every layer is also compared
with the float64 oracle (all token rows on small shapes, sampled rows on large ones) to the bar of
the single-layer tests: max|Y_gpu - Y_ref| <= tau * rms(Y_ref), tau = 1e-2 for bfloat16 and 1e-5 for
float32 inputs, and TIGHT = 2e-4 for bfloat16 (float32 accumulation).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, inputs
from tests._helpers import TAU, from_dev, meta_from_dev, rel_err, to_dev
from tests.test_gpu_linear import TIGHT, sampled_rows

pytestmark = pytest.mark.gpu


def _layers(count, M, n_in, n_out, r, dtype, seed):
    return [inputs.random_case(M, n_in, n_out, r, dtype, seed=seed + 101 * i, n_outliers=2) for i in range(count)]


def _device(L, dtype):
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    U = to_dev(L.U, dtype) if L.r else None
    V = to_dev(L.V, dtype) if L.r else None
    return dict(X=to_dev(L.X, dtype), values=vd, meta=md, U=U, V=V)


def _check_oracle(L, d, Y, dtype, tag, rows):
    v, m = from_dev(d["values"], dtype), meta_from_dev(d["meta"])
    U, V = (L.U, L.V) if L.r else (None, None)
    ref = oracle.linear(L.X, v, m, L.n_out, U, V, dtype, rows=rows)
    got = Y if rows is None else Y[rows]
    err = rel_err(got, ref)
    print(f"[group] {tag}: max|dY|/rms = {err:.3e}", flush=True)
    assert err <= TAU[dtype], f"{tag}: {err:.3e}"
    if dtype == "bf16":
        assert err <= TIGHT, f"{tag}: {err:.3e}"


# (layers, M, n_in, n_out, r): which kernel and tile the group takes
CASES = [
    (2, 2000, 4128, 4000, 64),   # alone 256-row tiles (128 of 512 rows), together 512-row tiles; ragged M, rows, K tail
    (4, 4096, 96, 1024, 0),      # 4 x 64 tiles of 512 rows: the 512-row tile; no low-rank part
    (3, 1100, 320, 700, 192),    # 256-row tiles either way; rank blocks after the main loop
    (2, 40, 512, 300, 32),       # decode-sized: the layers run one after the other
    (1, 300, 256, 200, 16),      # a group of one
]


@pytest.mark.parametrize("count,M,n_in,n_out,r", CASES)
def test_group_bitwise_and_oracle(count, M, n_in, n_out, r):
    dtype = "bf16"
    tag = f"{count} x {M}x{n_in}->{n_out} r{r}"
    print(f"[group] {tag}", flush=True)
    Ls = _layers(count, M, n_in, n_out, r, dtype, seed=M + n_in + r)
    ds = [_device(L, dtype) for L in Ls]
    single = [binding.linear(d["X"], d["values"], d["meta"], d["U"], d["V"], n_out=n_out) for d in ds]
    grouped = binding.linear_group([d["X"] for d in ds], [d["values"] for d in ds], [d["meta"] for d in ds],
                                   [d["U"] for d in ds] if r else None, [d["V"] for d in ds] if r else None,
                                   n_out=n_out)
    # stage 1 per layer, then the grouped stage 2 on the workspaces it left
    wss = [binding.new_workspace(M, n_out, n_in, r, torch.bfloat16) for _ in ds]
    for d, ws in zip(ds, wss):
        if r:
            binding.linear_stage1(d["X"], d["V"], ws)
    staged = binding.linear_stage2_group([d["X"] for d in ds], [d["values"] for d in ds], [d["meta"] for d in ds],
                                         [d["U"] for d in ds] if r else None, wss if r else None, n_out=n_out)
    torch.cuda.synchronize()
    rows = None if M * n_out * n_in <= (1 << 28) else sampled_rows(M, 3)
    for i, (L, d) in enumerate(zip(Ls, ds)):
        y1, yg, ys = (t.cpu().numpy() for t in (single[i], grouped[i], staged[i]))
        assert np.array_equal(y1.view(np.uint32), yg.view(np.uint32)), f"{tag}: layer {i} differs from its own call"
        assert np.array_equal(y1.view(np.uint32), ys.view(np.uint32)), f"{tag}: layer {i} (stage 2 group) differs"
        _check_oracle(L, d, yg, dtype, f"{tag} layer {i}", rows)


def test_group_attention_kv_full_size():
    """The benchmark's grouped call: k_proj and v_proj of the 8192-token, rank-128 block (two
    1024-output layers, 512-row tiles only together), against their own calls and the oracle on one
    token row in every 128-token tile."""
    Ls = [inputs.make_layer("C5", 1), inputs.make_layer("C5", 2)]
    ds = [_device(L, "bf16") for L in Ls]
    M, n_out = Ls[0].M, Ls[0].n_out
    single = [binding.linear(d["X"], d["values"], d["meta"], d["U"], d["V"], n_out=n_out) for d in ds]
    grouped = binding.linear_group([d["X"] for d in ds], [d["values"] for d in ds], [d["meta"] for d in ds],
                                   [d["U"] for d in ds], [d["V"] for d in ds], n_out=n_out)
    torch.cuda.synchronize()
    rows = sampled_rows(M, 4)
    for i, (L, d) in enumerate(zip(Ls, ds)):
        y1, yg = single[i].cpu().numpy(), grouped[i].cpu().numpy()
        assert np.array_equal(y1.view(np.uint32), yg.view(np.uint32)), f"{L.name} differs from its own call"
        _check_oracle(L, d, yg, "bf16", f"C5 group {L.name}", rows)


def test_group_fp32():
    """float32 layers run one after the other; each equals its own call."""
    Ls = _layers(2, 32, 512, 512, 16, "fp32", seed=9)
    ds = [_device(L, "fp32") for L in Ls]
    single = [binding.linear(d["X"], d["values"], d["meta"], d["U"], d["V"]) for d in ds]
    grouped = binding.linear_group([d["X"] for d in ds], [d["values"] for d in ds], [d["meta"] for d in ds],
                                   [d["U"] for d in ds], [d["V"] for d in ds])
    for i, (L, d) in enumerate(zip(Ls, ds)):
        y1, yg = single[i].cpu().numpy(), grouped[i].cpu().numpy()
        assert np.array_equal(y1.view(np.uint32), yg.view(np.uint32))
        _check_oracle(L, d, yg, "fp32", f"fp32 layer {i}", None)


def test_group_rejects_mixed_shapes():
    Ls = [inputs.random_case(128, 64, 32, 16, "bf16", seed=1), inputs.random_case(128, 64, 48, 16, "bf16", seed=2)]
    ds = [_device(L, "bf16") for L in Ls]
    with pytest.raises(ValueError):
        binding.linear_group([d["X"] for d in ds], [d["values"] for d in ds], [d["meta"] for d in ds],
                             [d["U"] for d in ds], [d["V"] for d in ds])
