"""Data-free alternating minimisation W ~ S + U V on the GPU (HASSLE-free page, §4).

Each step solves the two subproblems in turn: the sparse update is the 2:4 projection of the
residual W - U V (hard thresholding, §4.1.1), run by the fused residual + pack kernel
(splr_prune24_pack_residual); the low-rank update is the rank-r truncated SVD C_r(W - S) (§4.2.1).
The pages run 80 steps at rank 64 (§5.2, §5.3).

Readings where the pages are silent (the same as the CPU oracle's): the loop starts from
L_0 = C_r(W), the weight's leading singular components (LoSparse page, §3.2); L is kept as balanced
thin factors U = U_r sqrt(Sigma_r), V = sqrt(Sigma_r) V_r^T in the storage type (rounded to
nearest); the objective is ||W - S - U V||_F of the stored S, U, V.

C_r is computed by subspace iteration on a k-column basis (k = r + oversampling), warm-started from
the previous step's right singular basis: float32 matrix products (torch); the basis kept
orthonormal after each application of Z^T Z by one Cholesky QR pass whose float64 Gram matrix and triangular inverse are this
library's kernels (splr_gram_f64, splr_chol_rinv), so they stay on the device; the last basis Y is
not orthonormalised: its Gram matrix Y^T Y and that of the projected matrix Z^T Y go to the host
together, once per step, where one k x k symmetric-definite eigenproblem (float64, LAPACK through
scipy) gives the Rayleigh-Ritz rotation of the orthonormalised basis Y R^-1 in one go. After a few steps of
the loop this agrees with the exact truncated SVD to the working precision on matrices whose r-th
and (r+1)-th singular values are separated. The projection and the reconstruction of S are this
library's kernels.
"""
from __future__ import annotations

import time
from typing import Callable, Dict, List, Optional

import numpy as np
import scipy.linalg
import torch
from threadpoolctl import ThreadpoolController

from . import binding

_threadpools: Optional[ThreadpoolController] = None


def _blas_one_thread():
    """Context limiting the host BLAS to one thread (the controller is built once: building it
    scans the loaded libraries)."""
    global _threadpools
    if _threadpools is None:
        _threadpools = ThreadpoolController()
    return _threadpools.limit(limits=1, user_api="blas")


class _Buffers:
    """Device scratch reused across the steps of one loop, and direct calls of the Cholesky QR
    entry points on tensors this module made itself (contiguous float32 / float64 on one device;
    the library still checks sizes and alignment)."""

    def __init__(self):
        self.lib = binding.lib()
        self.ws: Optional[torch.Tensor] = None

    def gram(self, Y: torch.Tensor) -> torch.Tensor:
        assert Y.dtype == torch.float32 and Y.is_contiguous() and Y.dim() == 2
        n, k = Y.shape
        need = int(self.lib.splr_gram_workspace_bytes(n, k))
        if need == 0:
            raise ValueError(f"basis of shape {(n, k)} is out of range for splr_gram_f64")
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=Y.device)
        G = torch.empty((k, k), dtype=torch.float64, device=Y.device)
        binding._check("splr_gram_f64", self.lib.splr_gram_f64(Y.data_ptr(), n, k, G.data_ptr(), self.ws.data_ptr(),
                                                               self.ws.numel(), binding._stream(None)))
        return G

    def rinv(self, G: torch.Tensor) -> torch.Tensor:
        k = G.shape[0]
        out = torch.empty((k, k), dtype=torch.float32, device=G.device)
        binding._check("splr_chol_rinv", self.lib.splr_chol_rinv(G.data_ptr(), k, out.data_ptr(), binding._stream(None)))
        return out


def _orthonormalize(Y: torch.Tensor, buf: _Buffers) -> torch.Tensor:
    """Y R^-1 for Y^T Y = R^T R (one Cholesky QR pass, no host round trip): columns orthonormal up
    to float32 rounding times cond(Y)."""
    return Y @ buf.rinv(buf.gram(Y))


def _device_part(W: torch.Tensor, W32: torch.Tensor, U, V, values, meta, basis, r: int, k: int, power_iters: int,
                 buf: _Buffers):
    """The step up to its host round trip, all on the device: the projection S of W - U V, Z = W - S,
    the subspace iteration on Z from `basis`, Y = Z B, P = Z^T Y and the two k x k Gram matrices
    M = Y^T Y, P^T P stacked as MG [2, k, k] (float64). Returns values, meta, Z, Y, P, MG (the last
    three None when r == 0)."""
    n_out, n_in = W.shape
    values, meta = binding.prune24_pack_residual(W, U, V, values, meta)
    S = binding.dense_reconstruct(values, meta, None, None, n_out=n_out, n_in=n_in)
    Z = W32 - S
    if r == 0:
        return values, meta, Z, None, None, None
    Y, P, MG = _project(Z, basis, power_iters, buf)
    return values, meta, Z, Y, P, MG


def _project(Z: torch.Tensor, B: torch.Tensor, power_iters: int, buf: _Buffers):
    for _ in range(power_iters):
        # one orthonormalisation per application of Z^T Z: the float32 product keeps the directions
        # down to sqrt(float32 epsilon) sigma_1, far below the ones kept here
        B = _orthonormalize(Z.T @ (Z @ B), buf)
    Y = Z @ B                                          # [n_out, k]
    P = Z.T @ Y                                        # [n_in, k] = (Y^T Z)^T
    return Y, P, torch.stack([buf.gram(Y), buf.gram(P)])


def _ritz(MG: np.ndarray, r: int, k: int) -> np.ndarray:
    """Host part: from M = Y^T Y = R^T R and P^T P, the symmetric-definite pencil (P^T P, M) gives
    T with T^T M T = I and P^T P T = M T diag(s^2) (T = R^-1 W for the eigenvectors W of
    R^-T P^T P R^-1), s descending. Returns the coefficient matrix [k, k + 2r] = [T / s | T_r sqrt(s_r)
    / s_r | T_r sqrt(s_r)] of the next basis, V^T and U."""
    if not np.isfinite(MG).all():
        raise FloatingPointError("low-rank step: non-finite Gram matrix (rank-deficient basis?)")
    with _blas_one_thread():  # k x k is too small to share between threads
        lam, T = scipy.linalg.eigh(MG[1], MG[0], driver="gvd")
    order = np.argsort(lam)[::-1][:k]
    lam, T = np.maximum(lam[order], 0.0), T[:, order]
    s = np.sqrt(lam)
    Tb = T / np.where(s > 0, s, 1.0)[None, :]          # next basis = P Tb
    root = np.sqrt(s[:r])
    return np.concatenate([Tb, Tb[:, :r] * root[None, :], T[:, :r] * root[None, :]], axis=1)


def _factors(Y: torch.Tensor, P: torch.Tensor, coef: torch.Tensor, r: int, k: int):
    """U = Y T_r diag(sqrt s_r), V = diag(sqrt s_r) (P T_r / s_r)^T (float32, formed in float64) and
    the next basis P T / s, from the device copy of _ritz's coefficients."""
    PT = P.double() @ coef[:, :k + r]
    U = (Y.double() @ coef[:, k + r:]).float()
    V = PT[:, k:].T.float()
    return U, V, PT[:, :k].float().contiguous()


def _low_rank(Z: torch.Tensor, r: int, basis: Optional[torch.Tensor], power_iters: int, oversample: int,
              gen: torch.Generator, buf: _Buffers):
    """Approximate C_r(Z) for float32 Z [n_out, n_in]: (U, V) balanced float32 factors and the right
    basis [n_in, k] to warm-start the next call.

    Subspace iteration from the basis B (orthonormal); then, with Y = Z B and P = Z^T Y, M = Y^T Y =
    R^T R and the projected Gram R^-T (P^T P) R^-1 = W diag(s^2) W^T, the Ritz vectors of Z on
    span(Y) are Y T (left) and P T / s (right) with T = R^-1 W: U = Y T_r diag(sqrt s_r),
    V = diag(sqrt s_r) (P T_r / s_r)^T, next basis P T / s."""
    n_out, n_in = Z.shape
    k = min(r + oversample, n_out, n_in)
    if basis is None:
        B = torch.randn(n_in, k, generator=gen, device=Z.device, dtype=torch.float32)
        B = _orthonormalize(B, buf)
    else:
        B = basis
    Y, P, MG = _project(Z, B, power_iters, buf)
    coef = torch.from_numpy(_ritz(MG.cpu().numpy(), r, k)).to(device=Z.device)  # the one host round trip
    return _factors(Y, P, coef, r, k)


class _GraphStep:
    """One step of the loop as two HIP graphs around the host round trip: graph A = _device_part
    (projection, Z, subspace iteration, Gram matrices), then the Gram matrices to pinned host memory,
    _ritz on the host, its coefficients back, graph B = _factors plus the copies into the static U,
    V and basis that graph A reads on the next replay. Every kernel launch of a step comes from two
    graph launches; the results are those of the eager step (the same kernels on the same data)."""

    def __init__(self, W, W32, U, V, values, meta, basis, r, k, power_iters, buf):
        dev = W.device
        self.r, self.k = r, k
        self.U, self.V, self.basis = U.clone(), V.clone(), basis.clone()
        self.values, self.meta = values.clone(), meta.clone()
        self.coef = torch.empty((k, k + 2 * r), dtype=torch.float64, device=dev)
        self.coef_host = torch.empty((k, k + 2 * r), dtype=torch.float64, pin_memory=True)
        self.mg_host = torch.empty((2, k, k), dtype=torch.float64, pin_memory=True)
        self.ga, self.gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.ga):
            _, _, self.Z, self.Y, self.P, self.MG = _device_part(W, W32, self.U, self.V, self.values, self.meta,
                                                                 self.basis, r, k, power_iters, buf)
        with torch.cuda.graph(self.gb, pool=self.ga.pool()):
            self.U32, self.V32, nb = _factors(self.Y, self.P, self.coef, r, k)
            self.basis.copy_(nb)
            self.U.copy_(self.U32)
            self.V.copy_(self.V32)

    def run(self):
        stream = torch.cuda.current_stream()
        self.ga.replay()
        self.mg_host.copy_(self.MG, non_blocking=True)
        stream.synchronize()
        self.coef_host.copy_(torch.from_numpy(_ritz(self.mg_host.numpy(), self.r, self.k)))
        self.coef.copy_(self.coef_host, non_blocking=True)
        self.gb.replay()


def alternating_minimization(W: torch.Tensor, r: int, iters: int, *, power_iters: int = 2, start_iters: int = 6,
                             oversample: int = 16, seed: int = 0, X: Optional[torch.Tensor] = None,
                             track: bool = True, on_step: Optional[Callable[[Dict], None]] = None,
                             graphs: bool = True) -> Dict:
    """Run `iters` steps on W [n_out, n_in] (bfloat16 or float32, on the GPU).

    Returns dict(values, meta, U, V, objective, layer_rel_error, seconds, step_seconds): the packed
    S and factors after the last step; step_seconds[t] = host time from the end of step t-1 (or the
    start of the loop) to the end of step t (every step waits for the device once, for its Gram
    matrices, so in a steady state this is the step's time; the first step also takes the initial
    C_r(W) and the graph capture); objective[t] = ||W - S_t - U_t V_t||_F after step t (when `track`); with
    activations X [M, n_in], layer_rel_error[t] = ||X W^T - splr_linear(X)||_F / ||X W^T||_F.
    `on_step`, if given, is called after every step with dict(step, U_in, V_in: the stored factors
    the projection used; values, meta: the packed S it produced; U32, V32: the float32 factors of
    the low-rank step, before rounding to storage) -- device tensors, valid during the call.
    With `graphs` (and r > 0, no `on_step`), steps after the first replay two HIP graphs captured
    from the first (_GraphStep); the results equal those of the eager steps."""
    n_out, n_in = W.shape
    dtype = W.dtype
    gen = torch.Generator(device=W.device)
    gen.manual_seed(seed)
    W32 = W.float()
    basis = None
    buf = _Buffers()
    U = V = None
    k = min(r + oversample, n_out, n_in)
    t0 = time.perf_counter()
    if r > 0:
        U32, V32, basis = _low_rank(W32, r, None, start_iters, oversample, gen, buf)
        U, V = U32.to(dtype).contiguous(), V32.to(dtype).contiguous()
    objective: List[float] = []
    layer_err: List[float] = []
    ref = X.float() @ W32.T if X is not None else None
    values = meta = None
    runner: Optional[_GraphStep] = None
    marks = [time.perf_counter()]
    for step in range(iters):
        U_in, V_in = U, V
        if runner is not None:
            runner.run()
            values, meta, Z, U, V, basis = runner.values, runner.meta, runner.Z, runner.U, runner.V, runner.basis
        else:
            values, meta, Z, Y, P, MG = _device_part(W, W32, U, V, values, meta, basis, r, k, power_iters, buf)
            if r > 0:
                coef = torch.from_numpy(_ritz(MG.cpu().numpy(), r, k)).to(device=W.device)  # the host round trip
                U32, V32, basis = _factors(Y, P, coef, r, k)
                U, V = U32.to(dtype).contiguous(), V32.to(dtype).contiguous()
            if graphs and r > 0 and on_step is None and step + 1 < iters:
                runner = _GraphStep(W, W32, U, V, values, meta, basis, r, k, power_iters, buf)
        if on_step is not None:
            on_step(dict(step=step, U_in=U_in, V_in=V_in, values=values, meta=meta,
                         U32=U32 if r > 0 else None, V32=V32 if r > 0 else None))
        if track:
            L = U.float() @ V.float() if r > 0 else 0.0
            objective.append(float(torch.linalg.norm(Z - L)))
        if ref is not None:
            Yx = binding.linear(X, values, meta, U, V, n_out=n_out)
            layer_err.append(float(torch.linalg.norm(Yx - ref) / torch.linalg.norm(ref)))
        marks.append(time.perf_counter())
    torch.cuda.synchronize()
    return dict(values=values, meta=meta, U=U, V=V, objective=objective, layer_rel_error=layer_err,
                seconds=time.perf_counter() - t0, step_seconds=list(np.diff(marks)))
