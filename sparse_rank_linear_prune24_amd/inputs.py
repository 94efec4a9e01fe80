"""Seeded synthetic inputs, shared by the HIP path's tests and the CPU oracle's tests.

This module draws and rounds numbers; it does none of the projection or the layer product.
Storage convention for every array it returns:
  * "fp32" -> numpy float32
  * "bf16" -> numpy uint16 holding the bfloat16 bit pattern

Generator: for each tensor, numpy's PCG64 seeded by SeedSequence([seed, config_id, layer_id,
tensor_id]) with tensor_id X=0, W=1, U=2, V=3, outlier columns=4. Values are drawn as float64
standard normals, scaled, rounded to nearest-even float32 and then (bf16 workloads) to
nearest-even bfloat16.

The projection's input is the dense residual R = W - U V of the rounded factors (the sparse step of
alternating minimization acts on W minus the current low-rank part: HASSLE-free §4, §4.1.1). It is
formed once per layer in float64 and rounded the same way, so both sides of a comparison receive
the very same bits.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from . import configs as _configs

TENSOR_X, TENSOR_W, TENSOR_U, TENSOR_V, TENSOR_OUTLIERS = 0, 1, 2, 3, 4


# ----------------------------------------------------------------------------- rounding helpers

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    NaN inputs map to a quiet NaN with the same sign; infinities stay infinities."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(a, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def from_f64(a, dtype: str) -> np.ndarray:
    """Round float64 values to storage: nearest-even float32, then nearest-even bfloat16."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "fp32":
        return a32
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(f"unknown dtype {dtype!r}")


def itemsize(dtype: str) -> int:
    return {"fp32": 4, "bf16": 2}[dtype]


# ----------------------------------------------------------------------------- generators

def rng_for(seed: int, config_id: int, layer_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, config_id, layer_id, tensor_id])))


def gaussian(shape, std: float, dtype: str, *, seed: int = 0, config_id: int = 0, layer_id: int = 0,
             tensor_id: int = 0) -> np.ndarray:
    g = rng_for(seed, config_id, layer_id, tensor_id)
    return from_f64(g.standard_normal(size=shape, dtype=np.float64) * std, dtype)


def activations(M: int, K: int, dtype: str, n_outliers: int, outlier_scale: float, *, seed: int,
                config_id: int, layer_id: int) -> np.ndarray:
    """X ~ N(0, 1) with `n_outliers` distinct whole input columns scaled by `outlier_scale`."""
    g = rng_for(seed, config_id, layer_id, TENSOR_X)
    x = g.standard_normal(size=(M, K), dtype=np.float64)
    if n_outliers:
        cols = rng_for(seed, config_id, layer_id, TENSOR_OUTLIERS).choice(K, size=n_outliers, replace=False)
        x[:, np.sort(cols)] *= outlier_scale
    return from_f64(x, dtype)


def residual(W, U, V, dtype: str) -> np.ndarray:
    """R = W - U V of the stored (rounded) factors, in float64, rounded back to storage."""
    w = to_f64(W, dtype)
    if U is None or U.shape[1] == 0:
        return from_f64(w, dtype)
    return from_f64(w - to_f64(U, dtype) @ to_f64(V, dtype), dtype)


def column_scales(X, dtype: str) -> np.ndarray:
    """Per-input-column scales for the activation-aware pack: the 2-norms of the calibration
    activations' columns, sqrt(sum_m X[m][k]^2), in float64 from the stored X, rounded to float32.
    (Set-up, like `residual`: the pack takes d as an input.)"""
    x = to_f64(X, dtype)
    return np.sqrt(np.einsum("mk,mk->k", x, x)).astype(np.float32)


@dataclass
class Layer:
    name: str
    dtype: str
    M: int
    n_in: int
    n_out: int
    r: int
    X: np.ndarray
    W: np.ndarray
    U: np.ndarray
    V: np.ndarray
    R: np.ndarray


def make_layer(cfg_name: str, layer_idx: int, *, seed: int = 0, M: Optional[int] = None,
               with_x: bool = True) -> Layer:
    """The seeded tensors of one layer of a named workload (optionally with fewer tokens)."""
    cfg = _configs.get(cfg_name)
    name, n_in, n_out = cfg.layers[layer_idx]
    wcfg = _configs.get(cfg.weights_from) if cfg.weights_from else cfg
    M = cfg.M if M is None else M
    W = gaussian((n_out, n_in), wcfg.w_std, cfg.dtype, seed=seed, config_id=wcfg.config_id,
                 layer_id=layer_idx, tensor_id=TENSOR_W)
    U = gaussian((n_out, cfg.r), wcfg.uv_std, cfg.dtype, seed=seed, config_id=wcfg.config_id,
                 layer_id=layer_idx, tensor_id=TENSOR_U)
    V = gaussian((cfg.r, n_in), wcfg.uv_std, cfg.dtype, seed=seed, config_id=wcfg.config_id,
                 layer_id=layer_idx, tensor_id=TENSOR_V)
    X = (activations(M, n_in, cfg.dtype, cfg.n_outliers, cfg.outlier_scale, seed=seed,
                     config_id=cfg.config_id, layer_id=layer_idx) if with_x else None)
    return Layer(name, cfg.dtype, M, n_in, n_out, cfg.r, X, W, U, V, residual(W, U, V, cfg.dtype))


def random_case(M: int, n_in: int, n_out: int, r: int, dtype: str, *, seed: int,
                x_std: float = 1.0, w_std: float = 0.02, uv_std: Optional[float] = None,
                n_outliers: int = 0) -> Layer:
    """A seeded layer of arbitrary shape (config_id 1000 keeps it apart from the named workloads)."""
    uv_std = (w_std / np.sqrt(r) if r else 0.0) if uv_std is None else uv_std
    W = gaussian((n_out, n_in), w_std, dtype, seed=seed, config_id=1000, tensor_id=TENSOR_W)
    U = gaussian((n_out, r), uv_std, dtype, seed=seed, config_id=1000, tensor_id=TENSOR_U)
    V = gaussian((r, n_in), uv_std, dtype, seed=seed, config_id=1000, tensor_id=TENSOR_V)
    X = activations(M, n_in, dtype, n_outliers, 20.0, seed=seed, config_id=1000, layer_id=0)
    if x_std != 1.0:
        X = from_f64(to_f64(X, dtype) * x_std, dtype)
    return Layer("random", dtype, M, n_in, n_out, r, X, W, U, V, residual(W, U, V, dtype))


def small_integers(shape, lo: int, hi: int, dtype: str, *, seed: int, tensor_id: int = 0) -> np.ndarray:
    """Uniform integers in [lo, hi], stored exactly (|v| <= 256 is exact in bfloat16)."""
    g = rng_for(seed, 2000, 0, tensor_id)
    return from_f64(g.integers(lo, hi + 1, size=shape).astype(np.float64), dtype)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def layer_hashes(layer: Layer) -> Dict[str, str]:
    return {k: sha256(getattr(layer, k)) for k in ("X", "W", "U", "V")}
