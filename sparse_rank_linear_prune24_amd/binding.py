"""Thin ctypes binding of libsplr.so (C ABI in include/splr.h).

Argument marshalling only: tensors are passed as device pointers together with torch's current
HIP stream; every step of the computation runs in the library's kernels. There is no fallback:
if the library is missing or a call fails, an exception is raised.

Conventions: bf16 tensors are torch.bfloat16, fp32 tensors torch.float32; metadata is int32
(the bits of the library's uint32 words). Packed S uses the library's tiled layout (16 rows x 64
input columns per tile, see include/splr.h): values are shaped (TR, TK, 64, 8) and metadata
(TR, TK, 2, 16), TR = ceil(n_out / 16), TK = ceil(n_in / 64). The layer's n_out is passed
explicitly where it cannot be read off U.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsplr.so")

SPLR_FP32, SPLR_BF16 = 0, 1
STATUS = {0: "SPLR_OK", 1: "SPLR_ERR_NULL", 2: "SPLR_ERR_SHAPE", 3: "SPLR_ERR_DTYPE", 4: "SPLR_ERR_ALIGN",
          5: "SPLR_ERR_HIP", 6: "SPLR_ERR_WORKSPACE"}
EXPORTS = ("splr_prune24_pack", "splr_prune_nm_pack", "splr_linear_ex", "splr_prune24_pack_scaled", "splr_prune24_pack_residual", "splr_packed_bytes", "splr_linear_workspace_bytes", "splr_linear",
           "splr_linear_stage1", "splr_linear_stage2", "splr_dense_reconstruct", "splr_status_string",
           "splr_version")

_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_lib = None


class SplrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


def lib() -> ctypes.CDLL:
    """The loaded library with argument types declared (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_rank_linear_prune24_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.splr_prune24_pack.argtypes = [_P, _I64, _I64, _I32, _P, _P, _P]
        L.splr_prune24_pack.restype = _I32
        L.splr_prune24_pack_scaled.argtypes = [_P, _P, _I64, _I64, _I32, _P, _P, _P]
        L.splr_prune_nm_pack.argtypes = [_P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P]
        L.splr_prune_nm_pack.restype = _I32
        L.splr_prune24_pack_scaled.restype = _I32
        L.splr_prune24_pack_residual.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P]
        L.splr_prune24_pack_residual.restype = _I32
        L.splr_packed_bytes.argtypes = [_I64, _I64, _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
        L.splr_packed_bytes.restype = _I32
        L.splr_linear_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I32]
        L.splr_linear_workspace_bytes.restype = _SZ
        L.splr_linear.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _I32, _P, _P, _SZ, _P]
        L.splr_linear_ex.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _I32, _I32, _P, _P, _SZ, _P]
        L.splr_linear_ex.restype = _I32
        L.splr_linear.restype = _I32
        L.splr_linear_stage1.argtypes = [_P, _I64, _I64, _P, _I64, _I32, _P, _SZ, _P]
        L.splr_linear_stage1.restype = _I32
        L.splr_linear_stage2.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _I64, _I32, _P, _P, _SZ, _P]
        L.splr_linear_stage2.restype = _I32
        L.splr_dense_reconstruct.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P]
        L.splr_dense_reconstruct.restype = _I32
        L.splr_status_string.argtypes = [_I32]
        L.splr_status_string.restype = ctypes.c_char_p
        L.splr_version.argtypes = []
        L.splr_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPLR_BF16
    if t.dtype == torch.float32:
        return SPLR_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (use torch.bfloat16 or torch.float32)")


def _dev(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise SplrError(fn, status)


def tiles(n_out: int, n_in: int) -> Tuple[int, int]:
    return (n_out + 15) // 16, (n_in + 63) // 64


def packed_bytes(n_out: int, n_in: int, dtype: torch.dtype) -> Tuple[int, int]:
    """(values bytes, metadata bytes) of the packed layout, as the library reports them."""
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    code = SPLR_BF16 if dtype == torch.bfloat16 else SPLR_FP32
    _check("splr_packed_bytes", lib().splr_packed_bytes(n_out, n_in, code, ctypes.byref(vb), ctypes.byref(mb)))
    return vb.value, mb.value


def prune24_pack(R: torch.Tensor, values: Optional[torch.Tensor] = None, meta: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """2:4 projection + pack of R [n_out, n_in] -> (values (TR, TK, 64, 8), meta int32 (TR, TK, 2, 16))."""
    n_out, n_in = R.shape
    TR, TK = tiles(n_out, n_in)
    if values is None:
        values = torch.empty((TR, TK, 64, 8), dtype=R.dtype, device=R.device)
    if meta is None:
        meta = torch.empty((TR, TK, 2, 16), dtype=torch.int32, device=R.device)
    _check("splr_prune24_pack", lib().splr_prune24_pack(_dev(R, "R"), n_out, n_in, _dtype_code(R),
                                                        _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def prune_nm_pack(R: torch.Tensor, n: int, m: int, values: Optional[torch.Tensor] = None,
                  meta: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """N:M projection (n in {1, 2}, m in {4, 8, 16}) of R [n_out, n_in], stored in the 2:4 packed
    layout -> (values, meta) as prune24_pack returns them."""
    n_out, n_in = R.shape
    TR, TK = tiles(n_out, n_in)
    if values is None:
        values = torch.empty((TR, TK, 64, 8), dtype=R.dtype, device=R.device)
    if meta is None:
        meta = torch.empty((TR, TK, 2, 16), dtype=torch.int32, device=R.device)
    _check("splr_prune_nm_pack", lib().splr_prune_nm_pack(_dev(R, "R"), n_out, n_in, n, m, _dtype_code(R),
                                                          _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def prune24_pack_residual(W: torch.Tensor, U: Optional[torch.Tensor], V: Optional[torch.Tensor],
                          values: Optional[torch.Tensor] = None, meta: Optional[torch.Tensor] = None,
                          stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """2:4 projection + pack of R = W - U V, formed in the kernel (pinned fused multiply-add order)."""
    n_out, n_in = W.shape
    r = 0 if U is None else U.shape[1]
    TR, TK = tiles(n_out, n_in)
    if values is None:
        values = torch.empty((TR, TK, 64, 8), dtype=W.dtype, device=W.device)
    if meta is None:
        meta = torch.empty((TR, TK, 2, 16), dtype=torch.int32, device=W.device)
    _check("splr_prune24_pack_residual",
           lib().splr_prune24_pack_residual(_dev(W, "W"), _dev(U, "U"), _dev(V, "V"), n_out, n_in, r, _dtype_code(W),
                                            _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def prune24_pack_scaled(R: torch.Tensor, d: torch.Tensor, values: Optional[torch.Tensor] = None,
                        meta: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Activation-aware 2:4 projection + pack of R [n_out, n_in] with per-column scales d (float32
    [n_in]): keeps the two entries of largest |R[n][k]| * |d[k]| per group. Same outputs as
    prune24_pack."""
    n_out, n_in = R.shape
    if d.dtype != torch.float32 or tuple(d.shape) != (n_in,):
        raise ValueError(f"d must be float32 of shape ({n_in},), got {d.dtype} {tuple(d.shape)}")
    TR, TK = tiles(n_out, n_in)
    if values is None:
        values = torch.empty((TR, TK, 64, 8), dtype=R.dtype, device=R.device)
    if meta is None:
        meta = torch.empty((TR, TK, 2, 16), dtype=torch.int32, device=R.device)
    _check("splr_prune24_pack_scaled",
           lib().splr_prune24_pack_scaled(_dev(R, "R"), _dev(d, "d"), n_out, n_in, _dtype_code(R),
                                          _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def workspace_bytes(M: int, n_out: int, n_in: int, r: int, dtype: torch.dtype) -> int:
    code = SPLR_BF16 if dtype == torch.bfloat16 else SPLR_FP32
    return int(lib().splr_linear_workspace_bytes(M, n_out, n_in, r, code))


def new_workspace(M: int, n_out: int, n_in: int, r: int, dtype: torch.dtype, device="cuda") -> Optional[torch.Tensor]:
    """A workspace for splr_linear with these sizes (None when none is needed). Any workspace of at
    least workspace_bytes() serves any call; this one is zero-filled so that nothing depends on
    leftover contents."""
    need = workspace_bytes(M, n_out, n_in, r, dtype)
    return torch.zeros(need, dtype=torch.uint8, device=device) if need else None


def _linear_args(X, values, U, n_out, out, workspace, with_workspace=True):
    M, n_in = X.shape
    if n_out is None:
        n_out = U.shape[0] if U is not None else values.shape[0] * 16
    r = 0 if U is None else U.shape[1]
    if out is None:
        out = torch.empty((M, n_out), dtype=torch.float32, device=X.device)
    if workspace is None and with_workspace:
        workspace = new_workspace(M, n_out, n_in, r, X.dtype, X.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return M, n_in, n_out, r, out, workspace, ws_bytes


def linear(X: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
           V: Optional[torch.Tensor], n_out: Optional[int] = None, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y [M, n_out] float32 = X S^T + (X V^T) U^T (n_out defaults to U's rows, else 16 * TR)."""
    M, n_in, n_out, r, out, workspace, ws_bytes = _linear_args(X, values, U, n_out, out, workspace)
    _check("splr_linear", lib().splr_linear(_dev(X, "X"), M, n_in, _dev(values, "values"), _dev(meta, "meta"), n_out,
                                            _dev(U, "U"), _dev(V, "V"), r, _dtype_code(X), _dev(out, "out"),
                                            _dev(workspace, "workspace"), ws_bytes, _stream(stream)))
    return out


def linear_ex(X: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
              V: Optional[torch.Tensor], y_dtype: torch.dtype = torch.float32, n_out: Optional[int] = None,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """splr_linear with the output type chosen: float32, or bfloat16 (each result rounded to nearest
    even)."""
    if y_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"y_dtype must be float32 or bfloat16, got {y_dtype}")
    M = X.shape[0]
    if n_out is None:
        n_out = U.shape[0] if U is not None else values.shape[0] * 16
    if out is None:
        out = torch.empty((M, n_out), dtype=y_dtype, device=X.device)
    if out.dtype != y_dtype:
        raise ValueError(f"out is {out.dtype}, expected {y_dtype}")
    M, n_in, n_out, r, _, workspace, ws_bytes = _linear_args(X, values, U, n_out, out, workspace)
    ycode = SPLR_BF16 if y_dtype == torch.bfloat16 else SPLR_FP32
    _check("splr_linear_ex", lib().splr_linear_ex(_dev(X, "X"), M, n_in, _dev(values, "values"), _dev(meta, "meta"),
                                                  n_out, _dev(U, "U"), _dev(V, "V"), r, _dtype_code(X), ycode,
                                                  _dev(out, "out"), _dev(workspace, "workspace"), ws_bytes,
                                                  _stream(stream)))
    return out


def linear_stage1(X: torch.Tensor, V: Optional[torch.Tensor], workspace: torch.Tensor, n_out: int = 0,
                  stream=None) -> torch.Tensor:
    """First low-rank stage T = X V^T into `workspace` (sized by workspace_bytes); returns it."""
    M, n_in = X.shape
    r = 0 if V is None else V.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("splr_linear_stage1", lib().splr_linear_stage1(_dev(X, "X"), M, n_in, _dev(V, "V"), r, _dtype_code(X),
                                                          _dev(workspace, "workspace"), ws_bytes, _stream(stream)))
    return workspace


def linear_stage2(X: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
                  workspace: Optional[torch.Tensor], n_out: Optional[int] = None, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Y = X S^T + T U^T with T left in `workspace` by linear_stage1 (same X and r)."""
    M, n_in, n_out, r, out, workspace, ws_bytes = _linear_args(X, values, U, n_out, out, workspace,
                                                               with_workspace=False)
    _check("splr_linear_stage2",
           lib().splr_linear_stage2(_dev(X, "X"), M, n_in, _dev(values, "values"), _dev(meta, "meta"), n_out,
                                    _dev(U, "U"), r, _dtype_code(X), _dev(out, "out"), _dev(workspace, "workspace"),
                                    ws_bytes, _stream(stream)))
    return out


def dense_reconstruct(values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
                      V: Optional[torch.Tensor], n_out: Optional[int] = None, n_in: Optional[int] = None,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """W_hat [n_out, n_in] float32 = S + U V (sizes default to U / V's, else to the tile grid)."""
    if n_out is None:
        n_out = U.shape[0] if U is not None else values.shape[0] * 16
    if n_in is None:
        n_in = V.shape[1] if V is not None else values.shape[1] * 64
    r = 0 if U is None else U.shape[1]
    if out is None:
        out = torch.empty((n_out, n_in), dtype=torch.float32, device=values.device)
    _check("splr_dense_reconstruct",
           lib().splr_dense_reconstruct(_dev(values, "values"), _dev(meta, "meta"), _dev(U, "U"), _dev(V, "V"),
                                        n_out, n_in, r, _dtype_code(values), _dev(out, "out"), _stream(stream)))
    return out


def version() -> str:
    return lib().splr_version().decode()
