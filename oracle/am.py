"""Data-free alternating minimisation of W ~ S + U V -- TEST INFRASTRUCTURE ONLY (oracle).

The decomposition alternates an exact sparse update and an exact low-rank update (HASSLE-free page,
§4): with an identity Hessian the sparse subproblem is solved by hard thresholding onto the 2:4 set
(§4.1.1) and the low-rank subproblem by the rank-r truncated SVD C_r (§4.2.1; C_r is the best
rank-r approximation by the Eckart-Young theorem, §3). The pages run 80 steps at rank 64 (§5.2,
§5.3). Readings where the pages are silent:
  * start: L_0 = C_r(W), the leading singular components of the weight (LoSparse page, §3.2);
  * storage: L is kept as thin factors in the storage type, balanced as U = U_r sqrt(Sigma_r),
    V = sqrt(Sigma_r) V_r^T, each rounded to nearest; every sparse step projects the residual
    W - U V of the stored factors with the fused pack's pinned arithmetic
    (oracle.prune24_pack_residual);
  * objective: ||W - S - U V||_F of the stored S, U, V, in float64.
The truncated SVD is numpy's (LAPACK, float64).
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from . import prune24_pack_residual, unpack


# ---- storage-type conversions (this module's own; the oracle imports nothing from the product)

def _to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array: float32 values, or bfloat16 bit patterns (uint16),
    which are the upper 16 bits of a float32."""
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _from_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 to the storage type: to the nearest float32 (ties to even), then for bfloat16
    to the nearest bfloat16 (ties to even: add 0x7FFF plus the lowest kept bit, drop 16 bits).
    The factors rounded here are finite."""
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    if dtype == "fp32":
        return a32
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    if not np.all(np.isfinite(a32)):
        raise ValueError("non-finite factor")
    u = a32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def truncated_svd(Z: np.ndarray, r: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """C_r(Z) as (U_r, s_r, V_r^T): the r leading singular triplets of the float64 matrix Z."""
    u, s, vt = np.linalg.svd(Z, full_matrices=False)
    return u[:, :r], s[:r], vt[:r]


def balanced_factors(Z: np.ndarray, r: int, dtype: str) -> Tuple[Optional[np.ndarray], Optional[np.ndarray]]:
    """Stored thin factors of C_r(Z): U = U_r sqrt(s), V = sqrt(s) V_r^T, rounded to the storage type."""
    if r == 0:
        return None, None
    u, s, vt = truncated_svd(Z, r)
    root = np.sqrt(s)
    return _from_f64(u * root, dtype), _from_f64(root[:, None] * vt, dtype)


def dense_sparse(values, meta, n_out: int, n_in: int, dtype: str) -> np.ndarray:
    """The packed S as a dense float64 matrix (stored entries at their columns, zeros elsewhere)."""
    kept, nib = unpack(values, meta, n_out, n_in, dtype)
    k = _to_f64(kept, dtype)
    S = np.zeros((n_out, n_in))
    groups = n_in // 4
    a = (nib & 3).astype(np.int64)
    b = (nib >> 2).astype(np.int64)
    rows = np.arange(n_out)[:, None]
    base = 4 * np.arange(groups)[None, :]
    S[rows, base + a] = k[:, 0::2]
    S[rows, base + b] = k[:, 1::2]
    return S


def alternating_minimization(W: np.ndarray, r: int, iters: int, dtype: str):
    """Returns (values, meta, U, V, objectives) after `iters` steps; objectives[t] is
    ||W - S_t - U_t V_t||_F after step t (each step: S from the current factors, then new factors)."""
    n_out, n_in = W.shape
    w = _to_f64(W, dtype)
    U, V = balanced_factors(w, r, dtype)
    objectives: List[float] = []
    values = meta = None
    for _ in range(iters):
        values, meta = prune24_pack_residual(W, U, V, dtype)
        S = dense_sparse(values, meta, n_out, n_in, dtype)
        U, V = balanced_factors(w - S, r, dtype)
        L = 0.0 if U is None else _to_f64(U, dtype) @ _to_f64(V, dtype)
        objectives.append(float(np.linalg.norm(w - S - L)))
    return values, meta, U, V, objectives
