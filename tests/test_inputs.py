"""The seeded input generator: rounding, determinism, and the workload recipe."""
import json
import os

import numpy as np
import pytest
import torch

from sparse_rank_linear_prune24_amd import configs, inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    a = np.concatenate([
        g.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-42, 3.4e38, -3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                 dtype=np.float32),
        # exact halfway cases between two bf16 values (ties to even)
        (np.arange(1, 2000, dtype=np.uint32) << 15 | np.uint32(0x3F800000)).view(np.float32),
    ])
    ours = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_bits_to_f32(ours), torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_golden_hashes():
    with open(os.path.join(HERE, "golden", "input_hashes.json")) as fh:
        golden = json.load(fh)
    for key, want in golden.items():
        cfg, layer = key.split("/")
        L = inputs.make_layer(cfg, int(layer))
        assert inputs.layer_hashes(L) == want, key


def test_recipe_statistics():
    L = inputs.make_layer("C2", 0, M=256)
    c = configs.get("C2")
    W = inputs.to_f64(L.W, "bf16")
    assert abs(W.std() / 0.02 - 1) < 0.01
    U = inputs.to_f64(L.U, "bf16")
    assert abs(U.std() / (0.02 / 8) - 1) < 0.02
    X = inputs.to_f64(L.X, "bf16")
    col_std = X.std(axis=0)
    outliers = np.flatnonzero(col_std > 5)
    assert len(outliers) == c.n_outliers
    assert np.all(np.abs(col_std[outliers] / 20 - 1) < 0.2)
    # the decode workload reuses the prefill layer bit for bit, with its own activations
    L3 = inputs.make_layer("C3", 0)
    assert np.array_equal(L3.W, L.W) and np.array_equal(L3.R, L.R)
    assert L3.X.shape == (16, 4096)
    assert not np.array_equal(L3.X, L.X[:16])


def test_residual_is_w_minus_uv():
    L = inputs.make_layer("C1", 0)
    R = L.W.astype(np.float64) - L.U.astype(np.float64) @ L.V.astype(np.float64)
    assert np.array_equal(L.R, R.astype(np.float32))


def test_workload_sizes():
    # dense-equivalent FLOP of the named workloads (2 M n_out n_in summed over layers)
    assert configs.get("C2").dense_equiv_flop() == 68_719_476_736
    assert configs.get("C4").dense_equiv_flop() == 1_443_109_011_456
    assert configs.get("C5").dense_equiv_flop() == 3_573_412_790_272
    with pytest.raises(KeyError):
        configs.get("C9")
