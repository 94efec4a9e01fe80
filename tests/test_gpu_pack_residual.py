"""GPU parity of splr_prune24_pack_residual (R = W - U V formed in the kernel with the pinned
binary32 fused multiply-add order, then 2:4 projection + pack): values and metadata bit-identical
to the oracle's, for ragged shapes, ranks 0 / below one register block / several blocks with a
partial last one, special values (NaN canonicalisation), and the 4096 x 4096 rank-64 layer of the
prefill workload."""
import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, inputs
from tests._helpers import from_dev, meta_from_dev, to_dev

pytestmark = pytest.mark.gpu
BITS = {"fp32": np.uint32, "bf16": np.uint16}


def assert_residual_equal(W, U, V, dtype, tag=""):
    print(f"[pack_residual] {tag} dtype={dtype} W={W.shape} r={0 if U is None else U.shape[1]}", flush=True)
    v_ref, m_ref = oracle.prune24_pack_residual(W, U, V, dtype)
    v, m = binding.prune24_pack_residual(to_dev(W, dtype), to_dev(U, dtype) if U is not None else None,
                                         to_dev(V, dtype) if V is not None else None)
    torch.cuda.synchronize()
    v, m = from_dev(v, dtype), meta_from_dev(m)
    assert np.array_equal(m, m_ref), f"{tag}: metadata differs at {np.argwhere(m != m_ref)[:5]}"
    assert np.array_equal(v.view(BITS[dtype]), v_ref.view(BITS[dtype])), f"{tag}: values differ"


def case(n_out, n_in, r, dtype, seed):
    W = inputs.gaussian((n_out, n_in), 0.02, dtype, seed=seed, config_id=3200, tensor_id=1)
    if r == 0:
        return W, None, None
    U = inputs.gaussian((n_out, r), 0.02 / np.sqrt(r), dtype, seed=seed, config_id=3200, tensor_id=2)
    V = inputs.gaussian((r, n_in), 0.02 / np.sqrt(r), dtype, seed=seed, config_id=3200, tensor_id=3)
    return W, U, V


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_out,n_in,r", [(1, 32, 1), (17, 96, 5), (64, 512, 0), (40, 1056, 64), (129, 4128, 64),
                                          (50, 320, 80), (33, 1024, 130), (16, 256, 256)])
def test_shapes(dtype, n_out, n_in, r):
    W, U, V = case(n_out, n_in, r, dtype, seed=n_out + n_in + r)
    assert_residual_equal(W, U, V, dtype, f"{n_out}x{n_in} r={r}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_special_values(dtype):
    W, U, V = case(48, 256, 16, dtype, seed=9)
    b = BITS[dtype]
    Wb, Ub, Vb = W.view(b).copy(), U.view(b).copy(), V.view(b).copy()
    inf, nan = (0x7F800000, 0xFFC00123) if dtype == "fp32" else (0x7F80, 0xFFC1)
    Wb[3, 5] = nan            # NaN weight
    Wb[4, 7] = inf            # inf weight, finite terms
    Ub[5, 2] = inf            # inf factor: inf * V terms (and inf - inf where V < 0 meets W = inf ...)
    Vb[2, 9] = 0              # inf * 0 -> NaN in row 5, column 9
    Wb[6, :] = 0              # exact zeros: the residual is -U V
    assert_residual_equal(Wb.view(W.dtype), Ub.view(U.dtype), Vb.view(V.dtype), dtype, "specials")


def test_prefill_layer_full():
    """The q_proj layer of the prefill workload: W, U, V as stored, rank 64."""
    L = inputs.make_layer("C2", 0, with_x=False)
    assert_residual_equal(L.W, L.U, L.V, L.dtype, "C2 q_proj")
