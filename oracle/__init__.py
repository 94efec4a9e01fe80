"""CPU oracle for the 2:4 sparse + rank-r linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may import this
package. It wraps `splr_oracle.c` (plain C, float64 sums in index order, OpenMP over independent
outputs) through ctypes. It shares no code with the GPU library and never loads it.

Conventions: "bf16" arrays are numpy uint16 bit patterns, "fp32" arrays numpy float32.
Packed S is returned in its tiled layout (tiles of 16 rows x 64 input columns, see
splr_oracle.c): values shaped (TR, TK, 64, 8) and meta (TR, TKB, 64, 4) uint32 (blocks of 8
tile columns, 16 bytes per slot), with TR = ceil(n_out / 16), TK = ceil(n_in / 64),
TKB = ceil(TK / 8). `unpack` gives the logical per-group view.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "splr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DT = {"fp32": 0, "bf16": 1}
_NP = {"fp32": np.float32, "bf16": np.uint16}
_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fused multiply-add, so every sum is the written one)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.splr_ref_prune24_pack.argtypes = [P, I64, I64, ctypes.c_int, P, P]
        lib.splr_ref_prune24_pack_scaled.argtypes = [P, P, I64, I64, ctypes.c_int, P, P]
        lib.splr_ref_prune_nm.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        lib.splr_ref_residual.argtypes = [P, P, P, I64, I64, I64, ctypes.c_int, P]
        lib.splr_ref_prune24_pack_residual.argtypes = [P, P, P, I64, I64, I64, ctypes.c_int, P, P]
        lib.splr_ref_unpack.argtypes = [P, P, I64, I64, ctypes.c_int, P, P]
        lib.splr_ref_unpack.restype = ctypes.c_int
        lib.splr_ref_linear.argtypes = [P, I64, I64, P, P, I64, P, P, I64, ctypes.c_int, P, I64, P]
        lib.splr_ref_dense_reconstruct.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_int, P]
        for f in (lib.splr_ref_prune24_pack, lib.splr_ref_prune24_pack_scaled, lib.splr_ref_residual,
                  lib.splr_ref_prune24_pack_residual, lib.splr_ref_linear,
                  lib.splr_ref_dense_reconstruct):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a: np.ndarray, dtype: str, ndim: int, name: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != _NP[dtype] or a.ndim != ndim:
        raise TypeError(f"{name}: expected {ndim}-D {_NP[dtype].__name__} for {dtype}, got {a.dtype} {a.shape}")
    return a


def meta_shape(n_out: int, n_in: int) -> Tuple[int, int, int, int]:
    """Shape of the packed metadata: (TR, TKB, 64, 4) uint32, blocks of 8 tile columns."""
    TR, TK = tiles(n_out, n_in)
    return TR, (TK + 7) // 8, 64, 4


def tiles(n_out: int, n_in: int) -> Tuple[int, int]:
    """(TR, TK): tile rows and tile columns of the packed layout."""
    return (n_out + 15) // 16, (n_in + 63) // 64


def prune24_pack(R: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """2:4 projection of R [n_out x n_in] -> (values (TR, TK, 64, 8), meta uint32 (TR, TKB, 64, 4))."""
    R = _check(R, dtype, 2, "R")
    n_out, n_in = R.shape
    TR, TK = tiles(n_out, n_in)
    values = np.empty((TR, TK, 64, 8), dtype=_NP[dtype])
    meta = np.empty(meta_shape(n_out, n_in), dtype=np.uint32)
    rc = _load().splr_ref_prune24_pack(_ptr(R), n_out, n_in, _DT[dtype], _ptr(values), _ptr(meta))
    if rc:
        raise ValueError(f"splr_ref_prune24_pack failed ({rc}) for shape {R.shape}")
    return values, meta


def prune_nm(R: np.ndarray, n: int, m: int, dtype: str) -> np.ndarray:
    """N:M projection of R [n_out x n_in]: in every group of m consecutive columns keep the n
    entries of largest magnitude (ties to the lower column) as bit copies, the rest +0."""
    R = _check(R, dtype, 2, "R")
    n_out, n_in = R.shape
    Rp = np.empty_like(R)
    rc = _load().splr_ref_prune_nm(_ptr(R), n_out, n_in, n, m, _DT[dtype], _ptr(Rp))
    if rc:
        raise ValueError(f"splr_ref_prune_nm failed ({rc}) for shape {R.shape}, {n}:{m}")
    return Rp


def prune_nm_pack(R: np.ndarray, n: int, m: int, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """N:M projection, stored in the 2:4 packed layout: prune24_pack(prune_nm(R, n, m)). For n <= 2
    and 4 | m every aligned group of four holds at most two nonzeros of the projection, so the 2:4
    pack keeps all of them and the packed S is exactly the N:M matrix."""
    if not (n <= 2 and m % 4 == 0):
        raise ValueError(f"{n}:{m} is not storable in the 2:4 layout (needs n <= 2 and 4 | m)")
    return prune24_pack(prune_nm(R, n, m, dtype), dtype)


def prune24_pack_scaled(R: np.ndarray, d: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Activation-aware 2:4 projection of R [n_out x n_in] with per-column scales d (float32
    [n_in]): keeps the two entries of largest |R[n][k]| * |d[k]| per group (exact score, ties to the
    lower column, NaN scores above every number), storing R's own entries. Same layout as
    prune24_pack."""
    R = _check(R, dtype, 2, "R")
    d = np.ascontiguousarray(d, dtype=np.float32)
    n_out, n_in = R.shape
    if d.shape != (n_in,):
        raise ValueError(f"d: expected shape ({n_in},), got {d.shape}")
    TR, TK = tiles(n_out, n_in)
    values = np.empty((TR, TK, 64, 8), dtype=_NP[dtype])
    meta = np.empty(meta_shape(n_out, n_in), dtype=np.uint32)
    rc = _load().splr_ref_prune24_pack_scaled(_ptr(R), _ptr(d), n_out, n_in, _DT[dtype], _ptr(values), _ptr(meta))
    if rc:
        raise ValueError(f"splr_ref_prune24_pack_scaled failed ({rc}) for shape {R.shape}")
    return values, meta


def residual(W: np.ndarray, U: Optional[np.ndarray], V: Optional[np.ndarray], dtype: str) -> np.ndarray:
    """R = W - U V with the fused pack's pinned arithmetic: per entry acc = W, then
    acc = fmaf(-U[n][j], V[j][k], acc) for j = 0..r-1 in binary32, stored in the storage type
    (bfloat16: round to nearest even)."""
    W = _check(W, dtype, 2, "W")
    n_out, n_in = W.shape
    r = 0 if U is None else U.shape[1]
    if r:
        U, V = _check(U, dtype, 2, "U"), _check(V, dtype, 2, "V")
        if U.shape != (n_out, r) or V.shape != (r, n_in):
            raise ValueError(f"U {U.shape} / V {V.shape} do not match W {W.shape}")
    R = np.empty_like(W)
    rc = _load().splr_ref_residual(_ptr(W), _ptr(U if r else None), _ptr(V if r else None), n_out, n_in, r,
                                   _DT[dtype], _ptr(R))
    if rc:
        raise ValueError(f"splr_ref_residual failed ({rc})")
    return R


def prune24_pack_residual(W: np.ndarray, U: Optional[np.ndarray], V: Optional[np.ndarray],
                          dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Fused residual + 2:4 projection + pack: prune24_pack(residual(W, U, V))."""
    W = _check(W, dtype, 2, "W")
    n_out, n_in = W.shape
    r = 0 if U is None else U.shape[1]
    if r:
        U, V = _check(U, dtype, 2, "U"), _check(V, dtype, 2, "V")
    TR, TK = tiles(n_out, n_in)
    values = np.empty((TR, TK, 64, 8), dtype=_NP[dtype])
    meta = np.empty(meta_shape(n_out, n_in), dtype=np.uint32)
    rc = _load().splr_ref_prune24_pack_residual(_ptr(W), _ptr(U if r else None), _ptr(V if r else None), n_out, n_in,
                                                r, _DT[dtype], _ptr(values), _ptr(meta))
    if rc:
        raise ValueError(f"splr_ref_prune24_pack_residual failed ({rc})")
    return values, meta


def _check_packed(values, meta, n_out, n_in, dtype):
    TR, TK = tiles(n_out, n_in)
    values = _check(values, dtype, 4, "values")
    meta = np.ascontiguousarray(meta, dtype=np.uint32)
    if values.shape != (TR, TK, 64, 8) or meta.shape != meta_shape(n_out, n_in):
        raise ValueError(f"packed shapes {values.shape} {meta.shape} do not match {n_out} x {n_in}")
    return values, meta


def unpack(values: np.ndarray, meta: np.ndarray, n_out: int, n_in: int, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Logical view: kept [n_out x n_in/2] (the two kept entries of each group, in order) and the
    nibble (a | b << 2) of every group, uint8 [n_out x n_in/4]."""
    values, meta = _check_packed(values, meta, n_out, n_in, dtype)
    kept = np.empty((n_out, n_in // 2), dtype=_NP[dtype])
    nib = np.empty((n_out, n_in // 4), dtype=np.uint8)
    rc = _load().splr_ref_unpack(_ptr(values), _ptr(meta), n_out, n_in, _DT[dtype], _ptr(kept), _ptr(nib))
    if rc:
        raise ValueError(f"splr_ref_unpack failed ({rc})")
    return kept, nib


def linear(X: np.ndarray, values: np.ndarray, meta: np.ndarray, n_out: int, U: Optional[np.ndarray],
           V: Optional[np.ndarray], dtype: str, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """float64 Y = X S^T + (X V^T) U^T for all token rows, or only for `rows` (in that order)."""
    X = _check(X, dtype, 2, "X")
    M, n_in = X.shape
    values, meta = _check_packed(values, meta, n_out, n_in, dtype)
    r = 0 if U is None else U.shape[1]
    if r:
        U = _check(U, dtype, 2, "U")
        V = _check(V, dtype, 2, "V")
        if U.shape != (n_out, r) or V.shape != (r, n_in):
            raise ValueError("U/V shapes")
    else:
        U = V = None
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
    n_rows = M if rows is None else rows.shape[0]
    Y = np.empty((n_rows, n_out), dtype=np.float64)
    rc = _load().splr_ref_linear(_ptr(X), M, n_in, _ptr(values), _ptr(meta), n_out, _ptr(U), _ptr(V), r,
                                 _DT[dtype], _ptr(rows), n_rows, _ptr(Y))
    if rc:
        raise ValueError(f"splr_ref_linear failed ({rc})")
    return Y


def dense_reconstruct(values: np.ndarray, meta: np.ndarray, n_out: int, n_in: int, U: Optional[np.ndarray],
                      V: Optional[np.ndarray], dtype: str) -> np.ndarray:
    """float64 W_hat = S + U V, S scattered from (values, meta)."""
    values, meta = _check_packed(values, meta, n_out, n_in, dtype)
    r = 0 if U is None else U.shape[1]
    if r:
        U = _check(U, dtype, 2, "U")
        V = _check(V, dtype, 2, "V")
    else:
        U = V = None
    W = np.empty((n_out, n_in), dtype=np.float64)
    rc = _load().splr_ref_dense_reconstruct(_ptr(values), _ptr(meta), _ptr(U), _ptr(V), n_out, n_in, r,
                                            _DT[dtype], _ptr(W))
    if rc:
        raise ValueError(f"splr_ref_dense_reconstruct failed ({rc})")
    return W
