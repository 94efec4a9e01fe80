"""GPU parity of splr_linear_stage2_dense (S expanded to dense bfloat16 on chip, dense MFMA) against
the float64 oracle, and against the structured-sparse stage 2.

Bar: as for splr_linear (max|Y_gpu - Y_ref| <= 1e-2 rms(Y_ref) for bfloat16 inputs, and the tighter
float32-accumulation bound TIGHT = 2e-4); small-integer inputs make every sum exact, so there the
result must equal the oracle bit for bit. Shapes cover both tile forms of the dense kernel (512 rows
and eight waves when that gives every CU a tile, else 256 rows and four waves), ragged rows, tokens
and K, rank 0 and rank blocks before and after the main loop, and token counts of the decode range.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, configs, inputs
from tests._helpers import TAU, rel_err, to_dev
from tests.test_gpu_linear import TIGHT, sampled_rows

pytestmark = pytest.mark.gpu


def dense_call(Xd, vd, md, Ud, Vd, M, n_in, n_out, r):
    ws = binding.new_workspace(M, n_out, n_in, r, Xd.dtype, Xd.device)
    binding.linear_stage1(Xd, Vd, ws)
    return binding.linear_stage2_dense(Xd, vd, md, Ud, ws, n_out=n_out), ws


def check_dense(L, tag, rows=None):
    print(f"[dense] {tag} M={L.M} n_in={L.n_in} n_out={L.n_out} r={L.r}", flush=True)
    dtype = "bf16"
    Xd, Ud, Vd = to_dev(L.X, dtype), to_dev(L.U if L.r else None, dtype), to_dev(L.V if L.r else None, dtype)
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    Y, ws = dense_call(Xd, vd, md, Ud, Vd, L.M, L.n_in, L.n_out, L.r)
    Y_sparse = binding.linear_stage2(Xd, vd, md, Ud, ws, n_out=L.n_out)
    torch.cuda.synchronize()
    Y, Y_sparse = Y.cpu().numpy(), Y_sparse.cpu().numpy()
    v_ref, m_ref = oracle.prune24_pack(L.R, dtype)
    U, V = (L.U, L.V) if L.r else (None, None)
    Y_ref = oracle.linear(L.X, v_ref, m_ref, L.n_out, U, V, dtype, rows=rows)
    Yg = Y if rows is None else Y[rows]
    assert np.all(np.isfinite(Yg))
    err = rel_err(Yg, Y_ref)
    print(f"[dense] {tag}: max|dY|/rms = {err:.3e}", flush=True)
    assert err <= TAU[dtype] and err <= TIGHT, f"{tag}: {err:.3e}"
    # same products, summed in another order: the two stage-2 paths agree to float32 rounding
    assert rel_err(Y, Y_sparse.astype(np.float64)) <= TIGHT


SHAPES = [
    (1, 64, 16, 16), (17, 96, 33, 16), (64, 320, 64, 0), (65, 1024, 129, 64), (257, 512, 513, 128),
    (200, 2080, 300, 64), (1024, 1024, 384, 64), (128, 4096, 256, 192), (96, 512, 80, 1024),
]


@pytest.mark.parametrize("M,n_in,n_out,r", SHAPES)
def test_dense_shapes(M, n_in, n_out, r):
    L = inputs.random_case(M, n_in, n_out, r, "bf16", seed=3 * M + n_in + n_out + r, n_outliers=2)
    check_dense(L, f"{M}x{n_in}->{n_out} r{r}")


# the second and the last: Y above 96 MiB (non-temporal token-row stores); the last with ragged tokens and outputs
WIDE = [(4100, 2080, 4100, 80), (4096, 448, 8192, 0), (4160, 544, 4096, 144), (8200, 96, 6150, 16)]


@pytest.mark.parametrize("M,n_in,n_out,r", WIDE)
def test_dense_wide_tile(M, n_in, n_out, r):
    assert -(-n_out // 512) * -(-M // 128) >= 256
    L = inputs.random_case(M, n_in, n_out, r, "bf16", seed=M + n_in + n_out + r + 1, n_outliers=2)
    check_dense(L, f"wide {M}x{n_in}->{n_out} r{r}", rows=sampled_rows(M, 21))


def test_dense_named_c2():
    """The 2048-token q_proj layer in full (the dense kernel's 256-row form)."""
    L = inputs.make_layer("C2", 0)
    check_dense(L, "C2")


def test_dense_named_c5_q():
    """C5's q_proj layer (8192 tokens, rank 128, the 512-row form), sampled rows."""
    c = configs.get("C5")
    L = inputs.make_layer("C5", 0)
    check_dense(L, "C5/q_proj", rows=sampled_rows(c.M, c.config_id))


@pytest.mark.parametrize("M,n_out,r", [(256, 160, 16), (4096, 4096, 144)])
def test_dense_integer_exact_bitwise(M, n_out, r):
    """Small integers (every product and partial sum exact in float32): the dense path equals the
    oracle and the structured-sparse path bit for bit, in both tile forms."""
    dtype, n_in = "bf16", 544
    print(f"[dense] integer M={M} n_out={n_out} r={r}", flush=True)
    X = inputs.small_integers((M, n_in), -4, 4, dtype, seed=M + r, tensor_id=0)
    U = inputs.small_integers((n_out, r), -2, 2, dtype, seed=M + r, tensor_id=2)
    V = inputs.small_integers((r, n_in), -2, 2, dtype, seed=M + r, tensor_id=3)
    R = inputs.small_integers((n_out, n_in), -4, 4, dtype, seed=M + r, tensor_id=1)
    rows = sampled_rows(M, 13) if M > 1024 else None
    v_ref, m_ref = oracle.prune24_pack(R, dtype)
    ref = oracle.linear(X, v_ref, m_ref, n_out, U, V, dtype, rows=rows)
    vd, md = binding.prune24_pack(to_dev(R, dtype))
    Xd, Ud, Vd = to_dev(X, dtype), to_dev(U, dtype), to_dev(V, dtype)
    Y, ws = dense_call(Xd, vd, md, Ud, Vd, M, n_in, n_out, r)
    Y2 = binding.linear_stage2_dense(Xd, vd, md, Ud, ws, n_out=n_out)
    Ys = binding.linear_stage2(Xd, vd, md, Ud, ws, n_out=n_out)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    assert torch.equal(Y.view(torch.int32), Ys.view(torch.int32))
    Y = Y.cpu().numpy()
    assert np.array_equal((Y if rows is None else Y[rows]).astype(np.float64), ref)


def test_dense_rejects_fp32():
    L = inputs.random_case(32, 64, 16, 16, "fp32", seed=1)
    Xd, Ud = to_dev(L.X, "fp32"), to_dev(L.U, "fp32")
    vd, md = binding.prune24_pack(to_dev(L.R, "fp32"))
    ws = binding.new_workspace(32, 16, 64, 16, Xd.dtype, Xd.device)
    with pytest.raises(binding.SplrError) as e:
        binding.linear_stage2_dense(Xd, vd, md, Ud, ws, n_out=16)
    assert e.value.status == 3
