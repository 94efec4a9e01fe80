"""Pins of the oracle's data-free alternating minimisation (oracle/am.py).

The loop alternates the exact sparse update (2:4 hard thresholding, HASSLE-free page, §4.1.1) and
the exact low-rank update (rank-r truncated SVD, §4.2.1, best by Eckart-Young, §3). Pins:
  * the truncated SVD on matrices with prescribed singular values: the error is the tail energy
    (Eckart-Young) and the kept singular values are the prescribed ones;
  * the dense view of the packed S equals the oracle's C reconstruction;
  * r = 0: one step is the plain projection, whose error is the energy of the two smallest entries
    of every group (closed form);
  * each step minimises exactly over one block, so the objective never increases (up to the
    rounding of the stored factors);
  * a weight of rank r is fitted by L_0 alone: the first objective is at rounding level.
"""
import numpy as np
import pytest

import oracle
import oracle.am as am
from sparse_rank_linear_prune24_amd import inputs


def orthonormal(n, k, seed):
    q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((n, k)))
    return q


def test_truncated_svd_eckart_young():
    s = np.array([9.0, 7.5, 5.0, 4.0, 2.5, 1.0, 0.5, 0.25])
    Z = orthonormal(40, 8, 1) @ np.diag(s) @ orthonormal(30, 8, 2).T
    for r in (0, 1, 3, 8):
        u, sr, vt = am.truncated_svd(Z, r)
        assert np.allclose(sr, s[:r], rtol=1e-12, atol=1e-12)
        err = np.linalg.norm(Z - (u * sr) @ vt) ** 2
        assert err == pytest.approx(float(np.sum(s[r:] ** 2)), rel=1e-10, abs=1e-20)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_dense_view_matches_reconstruction(dtype):
    W = inputs.gaussian((33, 96), 0.02, dtype, seed=3)
    values, meta = oracle.prune24_pack(W, dtype)
    assert np.array_equal(am.dense_sparse(values, meta, 33, 96, dtype),
                          oracle.dense_reconstruct(values, meta, 33, 96, None, None, dtype))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rank_zero_is_one_projection(dtype):
    W = inputs.gaussian((32, 128), 0.02, dtype, seed=4)
    values, meta, U, V, obj = am.alternating_minimization(W, 0, 3, dtype)
    v0, m0 = oracle.prune24_pack(W, dtype)
    assert U is None and np.array_equal(meta, m0) and np.array_equal(values.view(np.uint8), v0.view(np.uint8))
    g = np.sort(np.abs(inputs.to_f64(W, dtype)).reshape(32, -1, 4), axis=2)
    dropped = float(np.sqrt(np.sum(g[:, :, :2] ** 2)))
    assert obj == pytest.approx([dropped] * 3, rel=1e-12)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_objective_never_increases(dtype):
    W = inputs.gaussian((64, 128), 0.02, dtype, seed=5)
    _, _, _, _, obj = am.alternating_minimization(W, 8, 12, dtype)
    slack = 1e-6 if dtype == "fp32" else 2e-3   # rounding of the stored factors
    assert all(b <= a * (1 + slack) for a, b in zip(obj, obj[1:])), obj
    assert obj[-1] < obj[0]


def test_rank_r_weight_is_fitted_by_the_start():
    A = inputs.gaussian((48, 6), 0.1, "fp32", seed=6, tensor_id=1)
    B = inputs.gaussian((6, 96), 0.1, "fp32", seed=6, tensor_id=2)
    W = (A.astype(np.float64) @ B.astype(np.float64)).astype(np.float32)
    _, _, _, _, obj = am.alternating_minimization(W, 6, 2, "fp32")
    assert obj[0] < 1e-5 * np.linalg.norm(W.astype(np.float64))


def test_storage_rounding_helpers():
    """The alternating minimisation's own conversions: exact widening, and round to nearest even
    at the bfloat16 boundary (hand-written cases: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 and
    goes to the even 1; 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 and goes to 1 + 2^-6;
    just above a halfway point rounds up)."""
    from oracle import am as oam
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -2.5, 0.0, -0.0])
    b = oam._from_f64(x, "bf16")
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000]
    assert oam._to_f64(b, "bf16").tolist() == [1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -2.5, 0.0, -0.0]
    f = oam._from_f64(np.array([1 + 2.0 ** -30, 3.0]), "fp32")
    assert f.dtype == np.float32 and f.tolist() == [1.0, 3.0]
