"""Data-free alternating minimisation W ~ S + U V on the GPU (HASSLE-free page, §4).

Each step solves the two subproblems in turn: the sparse update is the 2:4 projection of the
residual W - U V (hard thresholding, §4.1.1), run by the fused residual + pack kernel
(splr_prune24_pack_residual); the low-rank update is the rank-r truncated SVD C_r(W - S) (§4.2.1).
The pages run 80 steps at rank 64 (§5.2, §5.3).

Readings where the pages are silent (the same as the CPU oracle's): the loop starts from
L_0 = C_r(W), the weight's leading singular components (LoSparse page, §3.2); L is kept as balanced
thin factors U = U_r sqrt(Sigma_r), V = sqrt(Sigma_r) V_r^T in the storage type (rounded to
nearest); the objective is ||W - S - U V||_F of the stored S, U, V.

C_r is computed by subspace iteration (float32 matrix products from torch; Cholesky QR with the
k x k factors in float64 on the host; the small projected matrix decomposed through a k x k
symmetric eigenproblem, float64, host), warm-started from the previous step's right singular basis:
after a few steps of the loop it agrees with the exact truncated SVD to the working precision on
matrices whose r-th and (r+1)-th singular values are separated. The matrix products and the small
factorisations are library calls (torch, numpy); the projection and the reconstruction of S are
this library's kernels.
"""
from __future__ import annotations

import time
from typing import Callable, Dict, List, Optional

import numpy as np
import torch

from . import binding


def _gram(Y: torch.Tensor) -> np.ndarray:
    """Y^T Y in float64 for Y [n, k] (k small), as the sum of per-chunk products of up to 32 row
    chunks (a batched product keeps many workgroups busy where one k x k product over all n rows
    would run on a single one)."""
    n, k = Y.shape
    chunks = 32 if n % 32 == 0 and n >= 32 * k else 1
    Yd = Y.double().reshape(chunks, n // chunks, k)
    return torch.bmm(Yd.transpose(1, 2).contiguous(), Yd).sum(0).cpu().numpy()


def _orthonormalize(Y: torch.Tensor) -> torch.Tensor:
    """Orthonormal basis of the columns of Y [n, k] (k small) by Cholesky QR, twice: the Gram
    matrix is formed in float64 on the GPU, its k x k Cholesky factor inverted in float64 on the
    host, and Y multiplied by the inverse."""
    for _ in range(2):
        G = _gram(Y)
        Rinv = np.linalg.inv(np.linalg.cholesky(G).T)
        Y = Y @ torch.from_numpy(Rinv).to(device=Y.device, dtype=torch.float32)
    return Y


def _low_rank(Z: torch.Tensor, r: int, basis: Optional[torch.Tensor], power_iters: int, oversample: int,
              gen: torch.Generator):
    """Approximate C_r(Z) for float32 Z [n_out, n_in]: (U, V) balanced float32 factors and the right
    basis [n_in, k] to warm-start the next call. Subspace iteration; the projected k x n_in matrix
    B = Q^T Z is decomposed through the eigenvectors of B B^T (float64, on the host)."""
    n_out, n_in = Z.shape
    k = min(r + oversample, n_out, n_in)
    B = basis if basis is not None else torch.randn(n_in, k, generator=gen, device=Z.device, dtype=torch.float32)
    B = _orthonormalize(B)
    for _ in range(power_iters):
        Q = _orthonormalize(Z @ B)
        B = _orthonormalize(Z.T @ Q)
    Q = _orthonormalize(Z @ B)
    small = Q.T @ Z                                   # [k, n_in]
    lam, vec = np.linalg.eigh(_gram(small.T.contiguous()))
    order = np.argsort(lam)[::-1][:k]
    lam, vec = np.maximum(lam[order], 0.0), vec[:, order]
    s = np.sqrt(lam)
    Wv = torch.from_numpy(vec).to(device=Z.device, dtype=torch.float64)
    right = (small.double().T @ Wv) / torch.from_numpy(np.where(s > 0, s, 1.0)).to(Z.device)[None, :]  # [n_in, k]
    root = torch.from_numpy(np.sqrt(s[:r])).to(device=Z.device, dtype=torch.float64)
    U = ((Q.double() @ Wv[:, :r]) * root[None, :]).float()
    V = (root[:, None] * right[:, :r].T).float()
    return U, V, right.float().contiguous()


def alternating_minimization(W: torch.Tensor, r: int, iters: int, *, power_iters: int = 2, start_iters: int = 6,
                             oversample: int = 16, seed: int = 0, X: Optional[torch.Tensor] = None,
                             track: bool = True, on_step: Optional[Callable[[Dict], None]] = None) -> Dict:
    """Run `iters` steps on W [n_out, n_in] (bfloat16 or float32, on the GPU).

    Returns dict(values, meta, U, V, objective, layer_rel_error, seconds): the packed S and factors
    after the last step; objective[t] = ||W - S_t - U_t V_t||_F after step t (when `track`); with
    activations X [M, n_in], layer_rel_error[t] = ||X W^T - splr_linear(X)||_F / ||X W^T||_F.
    `on_step`, if given, is called after every step with dict(step, U_in, V_in: the stored factors
    the projection used; values, meta: the packed S it produced; U32, V32: the float32 factors of
    the low-rank step, before rounding to storage) -- device tensors, valid during the call."""
    n_out, n_in = W.shape
    dtype = W.dtype
    gen = torch.Generator(device=W.device)
    gen.manual_seed(seed)
    W32 = W.float()
    basis = None
    U = V = None
    t0 = time.perf_counter()
    if r > 0:
        U32, V32, basis = _low_rank(W32, r, None, start_iters, oversample, gen)
        U, V = U32.to(dtype).contiguous(), V32.to(dtype).contiguous()
    objective: List[float] = []
    layer_err: List[float] = []
    ref = X.float() @ W32.T if X is not None else None
    values = meta = None
    for step in range(iters):
        U_in, V_in = U, V
        values, meta = binding.prune24_pack_residual(W, U, V, values, meta)
        S = binding.dense_reconstruct(values, meta, None, None, n_out=n_out, n_in=n_in)
        Z = W32 - S
        if r > 0:
            U32, V32, basis = _low_rank(Z, r, basis, power_iters, oversample, gen)
            U, V = U32.to(dtype).contiguous(), V32.to(dtype).contiguous()
        if on_step is not None:
            on_step(dict(step=step, U_in=U_in, V_in=V_in, values=values, meta=meta,
                         U32=U32 if r > 0 else None, V32=V32 if r > 0 else None))
        if track:
            L = U.float() @ V.float() if r > 0 else 0.0
            objective.append(float(torch.linalg.norm(Z - L)))
        if ref is not None:
            Y = binding.linear(X, values, meta, U, V, n_out=n_out)
            layer_err.append(float(torch.linalg.norm(Y - ref) / torch.linalg.norm(ref)))
    torch.cuda.synchronize()
    return dict(values=values, meta=meta, U=U, V=V, objective=objective, layer_rel_error=layer_err,
                seconds=time.perf_counter() - t0)
