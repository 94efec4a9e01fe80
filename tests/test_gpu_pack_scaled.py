"""GPU parity of splr_prune24_pack_scaled (activation-aware 2:4 projection + pack): values and
metadata bit-identical to the oracle's, for Gaussian residuals with column scales from synthetic
calibration activations (outlier columns x20), ragged shapes, dense ties, zero scales and special
values, and the 4096 x 4096 layer of the prefill workload."""
import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, configs, inputs
from tests._helpers import from_dev, meta_from_dev, to_dev

pytestmark = pytest.mark.gpu
NP = {"fp32": np.float32, "bf16": np.uint16}
BITS = {"fp32": np.uint32, "bf16": np.uint16}


def assert_scaled_equal(R, d, dtype, tag=""):
    print(f"[pack_scaled] {tag} dtype={dtype} shape={R.shape}", flush=True)
    v_ref, m_ref = oracle.prune24_pack_scaled(R, d, dtype)
    v, m = binding.prune24_pack_scaled(to_dev(R, dtype), torch.from_numpy(np.ascontiguousarray(d)).cuda())
    torch.cuda.synchronize()
    v, m = from_dev(v, dtype), meta_from_dev(m)
    assert np.array_equal(m, m_ref), f"{tag}: metadata differs at {np.argwhere(m != m_ref)[:5]}"
    assert np.array_equal(v.view(BITS[dtype]), v_ref.view(BITS[dtype])), f"{tag}: values differ"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_out,n_in", [(1, 32), (3, 96), (17, 64), (129, 4128), (1000, 320)])
def test_ragged_shapes(dtype, n_out, n_in):
    R = inputs.gaussian((n_out, n_in), 0.02, dtype, seed=n_out + 3 * n_in, config_id=3100)
    X = inputs.activations(64, n_in, dtype, max(1, n_in // 512), 20.0, seed=n_in, config_id=3101, layer_id=0)
    assert_scaled_equal(R, inputs.column_scales(X, dtype), dtype, f"gaussian {n_out}x{n_in}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ties_zero_scales_and_special_values(dtype):
    g = np.random.default_rng(7)
    b = BITS[dtype]
    R = inputs.from_f64(g.integers(-2, 3, size=(64, 256)).astype(np.float64), dtype).view(b).copy()
    specials = ([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x00000001, 0x80000002, 0x7F7FFFFF, 0x80000000]
                if dtype == "fp32" else [0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8002, 0x7F7F, 0x8000])
    idx = g.integers(0, R.size, size=1500)
    R.reshape(-1)[idx] = np.array(specials, dtype=b)[g.integers(0, len(specials), size=idx.size)]
    # scales: small integers with repeats (exact ties), zeros, negatives, one infinity, one NaN, and
    # subnormals
    d = g.choice(np.array([0.0, 1.0, 2.0, 0.5, -1.0, 3.0], np.float32), size=256)
    d[17] = np.inf
    d[40] = np.nan
    d[[3, 99]] = np.array([1e-40, 3e-42], np.float32)
    assert_scaled_equal(R.view(NP[dtype]), d, dtype, "ties+specials")


def test_unit_scales_match_plain_pack():
    R = inputs.gaussian((256, 1024), 0.02, "bf16", seed=4, config_id=3102)
    Rd = to_dev(R, "bf16")
    v1, m1 = binding.prune24_pack(Rd)
    v2, m2 = binding.prune24_pack_scaled(Rd, torch.ones(1024, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16)) and torch.equal(m1, m2)


def test_prefill_layer_full():
    """The 4096 x 4096 residual of the prefill workload, scales from its 2048-token activations."""
    L = inputs.make_layer("C2", 0)
    d = inputs.column_scales(L.X, L.dtype)
    assert_scaled_equal(L.R, d, L.dtype, "C2 q_proj")
