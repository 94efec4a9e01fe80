"""Cholesky QR building blocks of the low-rank step (splr_gram_f64, splr_chol_rinv) against numpy:
the Gram matrix of float32 columns in float64 (every product exact, so only the summation order
differs) and the inverse Cholesky factor, which is unique for a positive definite G (R upper
triangular with a positive diagonal)."""
import numpy as np
import pytest
import torch

from sparse_rank_linear_prune24_amd import binding

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("n,k", [(1, 1), (33, 5), (100, 192), (4096, 80), (14336, 144), (5000, 67)])
def test_gram_f64(n, k):
    print(f"[gram] n={n} k={k}", flush=True)
    rng = np.random.default_rng(n * 1000 + k)
    Y = rng.standard_normal((n, k)).astype(np.float32) * rng.uniform(0.01, 10.0, size=k).astype(np.float32)
    G = binding.gram_f64(torch.from_numpy(Y).to(DEV)).cpu().numpy()
    y = Y.astype(np.float64)
    ref = y.T @ y
    # float64 sums of n exact products: |error| <= n * 2^-53 * sum |y_i y_j|
    bound = n * 2.0 ** -52 * (np.abs(y).T @ np.abs(y))
    assert np.all(np.abs(G - ref) <= bound + 1e-300)
    assert np.array_equal(G, G.T)


@pytest.mark.parametrize("k", [1, 2, 4, 5, 17, 80, 144, 192])
def test_chol_rinv(k):
    print(f"[chol_rinv] k={k}", flush=True)
    rng = np.random.default_rng(k)
    A = rng.standard_normal((2 * k + 7, k)) * rng.uniform(0.1, 10.0, size=k)
    G = A.T @ A
    Rinv = binding.chol_rinv(torch.from_numpy(G).to(DEV)).cpu().numpy()
    ref = np.linalg.inv(np.linalg.cholesky(G).T)
    assert np.all(np.tril(Rinv, -1) == 0.0)
    # float64 factorisation, float32 output: the rounding of the output dominates unless G is badly
    # conditioned; the float64 part is bounded by cond(G) * 2^-50 relative to |R^-1|
    cond = np.linalg.cond(G)
    tol = (2.0 ** -23 + cond * 2.0 ** -50) * np.abs(ref).max()
    assert np.abs(Rinv - ref).max() <= tol, (np.abs(Rinv - ref).max(), tol)


def test_cholqr_orthonormalises():
    """Y R^-1 has orthonormal columns for a well-conditioned float32 Y (the use in the low-rank step)."""
    rng = np.random.default_rng(7)
    Y = torch.from_numpy(rng.standard_normal((4096, 80)).astype(np.float32)).to(DEV)
    Q = Y @ binding.chol_rinv(binding.gram_f64(Y))
    E = (Q.double().T @ Q.double()).cpu().numpy() - np.eye(80)
    assert np.abs(E).max() < 1e-5
