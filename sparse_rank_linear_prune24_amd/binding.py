"""Thin ctypes binding of libsplr.so (C ABI in include/splr.h).

Argument marshalling only: tensors are passed as device pointers together with torch's current
HIP stream; every step of the computation runs in the library's kernels. There is no fallback:
if the library is missing or a call fails, an exception is raised.

Conventions: bf16 tensors are torch.bfloat16, fp32 tensors torch.float32; metadata is int32
(the bits of the library's uint32 words). Packed S uses the library's tiled layout (16 rows x 64
input columns per tile, see include/splr.h): values are shaped (TR, TK, 64, 8) and metadata
(TR, TKB, 64, 4) (blocks of 8 tile columns), TR = ceil(n_out / 16), TK = ceil(n_in / 64),
TKB = ceil(TK / 8). The layer's n_out is passed
explicitly where it cannot be read off U.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsplr.so")

SPLR_FP32, SPLR_BF16 = 0, 1
STATUS = {0: "SPLR_OK", 1: "SPLR_ERR_NULL", 2: "SPLR_ERR_SHAPE", 3: "SPLR_ERR_DTYPE", 4: "SPLR_ERR_ALIGN",
          5: "SPLR_ERR_HIP", 6: "SPLR_ERR_WORKSPACE", 7: "SPLR_ERR_SCRATCH"}
EXPORTS = ("splr_prune24_pack", "splr_prune_nm_pack", "splr_linear_ex", "splr_prune24_pack_scaled", "splr_prune24_pack_residual", "splr_packed_bytes", "splr_linear_workspace_bytes", "splr_linear",
           "splr_linear_stage1", "splr_linear_stage2", "splr_linear_stage2_dense", "splr_linear_group",
           "splr_linear_stage2_group", "splr_linear_noalloc", "splr_dense_reconstruct",
           "splr_gram_workspace_bytes", "splr_gram_f64", "splr_chol_rinv", "splr_status_string", "splr_version")

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
        L.splr_linear_stage2_dense.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _I64, _I32, _P, _P, _SZ, _P]
        L.splr_linear_stage2_dense.restype = _I32
        L.splr_linear_group.argtypes = [_I32, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _I32, _P, _P, _SZ, _P]
        L.splr_linear_group.restype = _I32
        L.splr_linear_stage2_group.argtypes = [_I32, _P, _I64, _I64, _P, _P, _I64, _P, _I64, _I32, _P, _P, _SZ, _P]
        L.splr_linear_stage2_group.restype = _I32
        L.splr_linear_noalloc.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _I32, _P, _P]
        L.splr_linear_noalloc.restype = _I32
        L.splr_dense_reconstruct.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P]
        L.splr_dense_reconstruct.restype = _I32
        L.splr_gram_workspace_bytes.argtypes = [_I64, _I64]
        L.splr_gram_workspace_bytes.restype = _SZ
        L.splr_gram_f64.argtypes = [_P, _I64, _I64, _P, _P, _SZ, _P]
        L.splr_gram_f64.restype = _I32
        L.splr_chol_rinv.argtypes = [_P, _I64, _P, _P]
        L.splr_chol_rinv.restype = _I32
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


def _is_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _dev(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    return _the_stream(stream).cuda_stream


def _the_stream(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _expect(t: Optional[torch.Tensor], name: str, dtype, numel: int, device, shape=None):
    """Raise ValueError unless `t` is a contiguous device tensor of `dtype` on `device` holding
    exactly `numel` elements (and of `shape`, when given). The C ABI sees only pointers, so a
    buffer of the wrong size would be read or written out of bounds: every tensor is checked here,
    before the call."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() != numel:
        raise ValueError(f"{name} holds {t.numel()} elements, expected {numel}")


def _matrix(t: torch.Tensor, name: str) -> Tuple[int, int]:
    if not isinstance(t, torch.Tensor) or not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape[0], t.shape[1]


def _packed_out(values, meta, n_out, n_in, dtype, device, stream):
    """Check caller-supplied packed buffers (or allocate them on the call's stream)."""
    TR, TK = tiles(n_out, n_in)
    if values is None or meta is None:
        with torch.cuda.stream(_the_stream(stream)):
            if values is None:
                values = torch.empty((TR, TK, 64, 8), dtype=dtype, device=device)
            if meta is None:
                meta = torch.empty(meta_shape(n_out, n_in), dtype=torch.int32, device=device)
    _expect(values, "values", dtype, TR * TK * 512, device)
    _expect(meta, "meta", torch.int32, _meta_words(n_out, n_in), device)
    return values, meta


def _meta_words(n_out: int, n_in: int) -> int:
    TR, TKB, lanes, words = meta_shape(n_out, n_in)
    return TR * TKB * lanes * words


def _check_packed_in(values, meta, n_out, n_in, dtype, device):
    TR, TK = tiles(n_out, n_in)
    _expect(values, "values", dtype, TR * TK * 512, device)
    _expect(meta, "meta", torch.int32, _meta_words(n_out, n_in), device)


def _check_factors(U, V, n_out, n_in, dtype, device):
    """U [n_out, r] and V [r, n_in] of the storage type (both or neither); returns r."""
    if (U is None) != (V is None):
        raise ValueError("U and V are given together (or neither, for no low-rank part)")
    if U is None:
        return 0
    r = U.shape[1] if U.dim() == 2 else -1
    _expect(U, "U", dtype, n_out * max(r, 0), device, (n_out, r))
    _expect(V, "V", dtype, r * n_in, device, (r, n_in))
    return r


def _check(fn: str, status: int):
    if status != 0:
        raise SplrError(fn, status)


def tiles(n_out: int, n_in: int) -> Tuple[int, int]:
    return (n_out + 15) // 16, (n_in + 63) // 64


def meta_shape(n_out: int, n_in: int) -> Tuple[int, int, int, int]:
    """Shape of the packed metadata (int32 words): (TR, TKB, 64, 4), blocks of 8 tile columns."""
    TR, TK = tiles(n_out, n_in)
    return TR, (TK + 7) // 8, 64, 4


def packed_bytes(n_out: int, n_in: int, dtype: torch.dtype) -> Tuple[int, int]:
    """(values bytes, metadata bytes) of the packed layout, as the library reports them."""
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    code = SPLR_BF16 if dtype == torch.bfloat16 else SPLR_FP32
    _check("splr_packed_bytes", lib().splr_packed_bytes(n_out, n_in, code, ctypes.byref(vb), ctypes.byref(mb)))
    return vb.value, mb.value


def prune24_pack(R: torch.Tensor, values: Optional[torch.Tensor] = None, meta: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """2:4 projection + pack of R [n_out, n_in] -> (values (TR, TK, 64, 8), meta int32 (TR, TKB, 64, 4))."""
    n_out, n_in = _matrix(R, "R")
    _dtype_code(R)
    values, meta = _packed_out(values, meta, n_out, n_in, R.dtype, R.device, stream)
    _check("splr_prune24_pack", lib().splr_prune24_pack(_dev(R, "R"), n_out, n_in, _dtype_code(R),
                                                        _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def prune_nm_pack(R: torch.Tensor, n: int, m: int, values: Optional[torch.Tensor] = None,
                  meta: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """N:M projection (n in {1, 2}, m in {4, 8, 16}) of R [n_out, n_in], stored in the 2:4 packed
    layout -> (values, meta) as prune24_pack returns them."""
    n_out, n_in = _matrix(R, "R")
    _dtype_code(R)
    values, meta = _packed_out(values, meta, n_out, n_in, R.dtype, R.device, stream)
    _check("splr_prune_nm_pack", lib().splr_prune_nm_pack(_dev(R, "R"), n_out, n_in, n, m, _dtype_code(R),
                                                          _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def prune24_pack_residual(W: torch.Tensor, U: Optional[torch.Tensor], V: Optional[torch.Tensor],
                          values: Optional[torch.Tensor] = None, meta: Optional[torch.Tensor] = None,
                          stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """2:4 projection + pack of R = W - U V, formed in the kernel (pinned fused multiply-add order)."""
    n_out, n_in = _matrix(W, "W")
    _dtype_code(W)
    r = _check_factors(U, V, n_out, n_in, W.dtype, W.device)
    values, meta = _packed_out(values, meta, n_out, n_in, W.dtype, W.device, stream)
    _check("splr_prune24_pack_residual",
           lib().splr_prune24_pack_residual(_dev(W, "W"), _dev(U, "U"), _dev(V, "V"), n_out, n_in, r, _dtype_code(W),
                                            _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def prune24_pack_scaled(R: torch.Tensor, d: torch.Tensor, values: Optional[torch.Tensor] = None,
                        meta: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Activation-aware 2:4 projection + pack of R [n_out, n_in] with per-column scales d (float32
    [n_in]): keeps the two entries of largest |R[n][k]| * |d[k]| per group. Same outputs as
    prune24_pack."""
    n_out, n_in = _matrix(R, "R")
    _dtype_code(R)
    _expect(d, "d", torch.float32, n_in, R.device, (n_in,))
    values, meta = _packed_out(values, meta, n_out, n_in, R.dtype, R.device, stream)
    _check("splr_prune24_pack_scaled",
           lib().splr_prune24_pack_scaled(_dev(R, "R"), _dev(d, "d"), n_out, n_in, _dtype_code(R),
                                          _dev(values, "values"), _dev(meta, "meta"), _stream(stream)))
    return values, meta


def workspace_bytes(M: int, n_out: int, n_in: int, r: int, dtype: torch.dtype) -> int:
    code = SPLR_BF16 if dtype == torch.bfloat16 else SPLR_FP32
    return int(lib().splr_linear_workspace_bytes(M, n_out, n_in, r, code))


def new_workspace(M: int, n_out: int, n_in: int, r: int, dtype: torch.dtype, device="cuda",
                  stream=None) -> Optional[torch.Tensor]:
    """A workspace for splr_linear with these sizes (None when none is needed), allocated on
    `stream` (default: the current stream). Any workspace of at least workspace_bytes() serves any
    call, and its contents need no initialisation: every byte the second stage reads is written by
    the first stage of the same call."""
    need = workspace_bytes(M, n_out, n_in, r, dtype)
    if not need:
        return None
    with torch.cuda.stream(_the_stream(stream)):
        return torch.empty(need, dtype=torch.uint8, device=device)


def _linear_args(X, values, meta, U, V, n_out, out, workspace, stream, y_dtype=torch.float32, with_workspace=True,
                 need_v=True):
    """Checks every tensor of a layer-product call against the sizes passed to the C ABI, and
    allocates what is missing on the call's stream."""
    M, n_in = _matrix(X, "X")
    _dtype_code(X)
    if n_out is None:
        n_out = U.shape[0] if U is not None else values.shape[0] * 16
    _check_packed_in(values, meta, n_out, n_in, X.dtype, X.device)
    if need_v:
        r = _check_factors(U, V, n_out, n_in, X.dtype, X.device)
    else:
        r = 0 if U is None else (U.shape[1] if U.dim() == 2 else -1)
        if U is not None:
            _expect(U, "U", X.dtype, n_out * max(r, 0), X.device, (n_out, r))
    if out is None:
        with torch.cuda.stream(_the_stream(stream)):
            out = torch.empty((M, n_out), dtype=y_dtype, device=X.device)
    if workspace is None and with_workspace:
        workspace = new_workspace(M, n_out, n_in, r, X.dtype, X.device, stream)
    _expect(out, "out", y_dtype, M * n_out, X.device, (M, n_out))
    if workspace is not None:
        if not _is_device(workspace) or workspace.device != X.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the device of X")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return M, n_in, n_out, r, out, workspace, ws_bytes


def linear(X: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
           V: Optional[torch.Tensor], n_out: Optional[int] = None, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y [M, n_out] float32 = X S^T + (X V^T) U^T (n_out defaults to U's rows, else 16 * TR)."""
    M, n_in, n_out, r, out, workspace, ws_bytes = _linear_args(X, values, meta, U, V, n_out, out, workspace, stream)
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
    M, n_in, n_out, r, out, workspace, ws_bytes = _linear_args(X, values, meta, U, V, n_out, out, workspace, stream,
                                                               y_dtype=y_dtype)
    ycode = SPLR_BF16 if y_dtype == torch.bfloat16 else SPLR_FP32
    _check("splr_linear_ex", lib().splr_linear_ex(_dev(X, "X"), M, n_in, _dev(values, "values"), _dev(meta, "meta"),
                                                  n_out, _dev(U, "U"), _dev(V, "V"), r, _dtype_code(X), ycode,
                                                  _dev(out, "out"), _dev(workspace, "workspace"), ws_bytes,
                                                  _stream(stream)))
    return out


def linear_stage1(X: torch.Tensor, V: Optional[torch.Tensor], workspace: torch.Tensor, n_out: int = 0,
                  stream=None) -> torch.Tensor:
    """First low-rank stage T = X V^T into `workspace` (sized by workspace_bytes); returns it."""
    M, n_in = _matrix(X, "X")
    _dtype_code(X)
    r = 0
    if V is not None:
        r = V.shape[0] if V.dim() == 2 else -1
        _expect(V, "V", X.dtype, max(r, 0) * n_in, X.device, (r, n_in))
    if workspace is not None and (not _is_device(workspace) or workspace.device != X.device
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the device of X")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("splr_linear_stage1", lib().splr_linear_stage1(_dev(X, "X"), M, n_in, _dev(V, "V"), r, _dtype_code(X),
                                                          _dev(workspace, "workspace"), ws_bytes, _stream(stream)))
    return workspace


def linear_stage2(X: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
                  workspace: Optional[torch.Tensor], n_out: Optional[int] = None, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Y = X S^T + T U^T with T left in `workspace` by linear_stage1 (same X and r)."""
    M, n_in, n_out, r, out, workspace, ws_bytes = _linear_args(X, values, meta, U, None, n_out, out, workspace, stream,
                                                               with_workspace=False, need_v=False)
    _check("splr_linear_stage2",
           lib().splr_linear_stage2(_dev(X, "X"), M, n_in, _dev(values, "values"), _dev(meta, "meta"), n_out,
                                    _dev(U, "U"), r, _dtype_code(X), _dev(out, "out"), _dev(workspace, "workspace"),
                                    ws_bytes, _stream(stream)))
    return out


GROUP_MAX = 4  # SPLR_GROUP_MAX


def _ptr_array(ts, name):
    """A host array of the tensors' device pointers (None for a missing list)."""
    if ts is None:
        return None
    return (ctypes.c_void_p * len(ts))(*[_dev(t, f"{name}[{i}]") for i, t in enumerate(ts)])


def _group_args(Xs, values, metas, Us, Vs, n_out, outs, workspaces, stream, with_stage1):
    """Checks every layer as the single-layer call would (allocating missing outputs and workspaces
    on the call's stream) and that the layers share their sizes and type."""
    count = len(Xs)
    if not 1 <= count <= GROUP_MAX:
        raise ValueError(f"a group holds 1..{GROUP_MAX} layers, got {count}")
    for name, lst in (("values", values), ("meta", metas), ("U", Us), ("V", Vs), ("outs", outs),
                      ("workspaces", workspaces)):
        if lst is not None and len(lst) != count:
            raise ValueError(f"{name} has {len(lst)} entries for {count} layers")
    per = []
    for i in range(count):
        U = None if Us is None else Us[i]
        V = None if Vs is None else Vs[i]
        out = None if outs is None else outs[i]
        ws = None if workspaces is None else workspaces[i]
        per.append(_linear_args(Xs[i], values[i], metas[i], U, V if with_stage1 else None, n_out, out, ws, stream,
                                with_workspace=with_stage1, need_v=with_stage1))
    shape = per[0][:4]
    if any(p[:4] != shape for p in per) or any(X.dtype != Xs[0].dtype for X in Xs):
        raise ValueError("the layers of a group share M, n_in, n_out, r and the storage type")
    M, n_in, n_out, r = shape
    outs = [p[4] for p in per]
    wss = [p[5] for p in per]
    ws_bytes = min(p[6] for p in per)
    return count, M, n_in, n_out, r, outs, wss, ws_bytes


def linear_group(Xs: Sequence[torch.Tensor], values: Sequence[torch.Tensor], metas: Sequence[torch.Tensor],
                 Us: Optional[Sequence[torch.Tensor]], Vs: Optional[Sequence[torch.Tensor]],
                 n_out: Optional[int] = None, outs: Optional[Sequence[torch.Tensor]] = None,
                 workspaces: Optional[Sequence[torch.Tensor]] = None, stream=None) -> List[torch.Tensor]:
    """splr_linear for up to GROUP_MAX layers of one shape, stage 2 of all of them in one launch
    (splr_linear_group); returns the layers' Y, each bit for bit its splr_linear result."""
    count, M, n_in, n_out, r, outs, wss, ws_bytes = _group_args(Xs, values, metas, Us, Vs, n_out, outs, workspaces,
                                                                stream, True)
    ws_arr = _ptr_array(wss, "workspace") if r > 0 else (ctypes.c_void_p * count)()
    _check("splr_linear_group",
           lib().splr_linear_group(count, _ptr_array(Xs, "X"), M, n_in, _ptr_array(values, "values"),
                                   _ptr_array(metas, "meta"), n_out, _ptr_array(Us, "U") if r > 0 else None,
                                   _ptr_array(Vs, "V") if r > 0 else None, r, _dtype_code(Xs[0]),
                                   _ptr_array(outs, "out"), ws_arr, ws_bytes, _stream(stream)))
    return outs


def linear_stage2_group(Xs: Sequence[torch.Tensor], values: Sequence[torch.Tensor], metas: Sequence[torch.Tensor],
                        Us: Optional[Sequence[torch.Tensor]], workspaces: Optional[Sequence[torch.Tensor]],
                        n_out: Optional[int] = None, outs: Optional[Sequence[torch.Tensor]] = None,
                        stream=None) -> List[torch.Tensor]:
    """linear_stage2 for up to GROUP_MAX layers of one shape in one launch (splr_linear_stage2_group),
    each layer's T left in its workspace by linear_stage1."""
    count, M, n_in, n_out, r, outs, wss, ws_bytes = _group_args(Xs, values, metas, Us, None, n_out, outs, workspaces,
                                                                stream, False)
    ws_arr = _ptr_array(wss, "workspace") if r > 0 else (ctypes.c_void_p * count)()
    _check("splr_linear_stage2_group",
           lib().splr_linear_stage2_group(count, _ptr_array(Xs, "X"), M, n_in, _ptr_array(values, "values"),
                                          _ptr_array(metas, "meta"), n_out, _ptr_array(Us, "U") if r > 0 else None,
                                          r, _dtype_code(Xs[0]), _ptr_array(outs, "out"), ws_arr, ws_bytes,
                                          _stream(stream)))
    return outs


def linear_stage2_dense(X: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
                        workspace: Optional[torch.Tensor], n_out: Optional[int] = None,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """linear_stage2 with S expanded to dense bfloat16 on chip and multiplied by dense MFMA
    (splr_linear_stage2_dense; bfloat16 only): the measured alternative to the structured-sparse
    instruction."""
    M, n_in, n_out, r, out, workspace, ws_bytes = _linear_args(X, values, meta, U, None, n_out, out, workspace, stream,
                                                               with_workspace=False, need_v=False)
    _check("splr_linear_stage2_dense",
           lib().splr_linear_stage2_dense(_dev(X, "X"), M, n_in, _dev(values, "values"), _dev(meta, "meta"), n_out,
                                          _dev(U, "U"), r, _dtype_code(X), _dev(out, "out"),
                                          _dev(workspace, "workspace"), ws_bytes, _stream(stream)))
    return out


def linear_noalloc(X: torch.Tensor, values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
                   V: Optional[torch.Tensor], n_out: Optional[int] = None, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """splr_linear with the library's built-in workspace (splr_linear_noalloc): nothing is allocated
    when `out` is given. Calls on one GPU share that workspace, so they must not overlap in time."""
    M, n_in, n_out, r, out, _, _ = _linear_args(X, values, meta, U, V, n_out, out, None, stream,
                                                with_workspace=False)
    _check("splr_linear_noalloc",
           lib().splr_linear_noalloc(_dev(X, "X"), M, n_in, _dev(values, "values"), _dev(meta, "meta"), n_out,
                                     _dev(U, "U"), _dev(V, "V"), r, _dtype_code(X), _dev(out, "out"),
                                     _stream(stream)))
    return out


def dense_reconstruct(values: torch.Tensor, meta: torch.Tensor, U: Optional[torch.Tensor],
                      V: Optional[torch.Tensor], n_out: Optional[int] = None, n_in: Optional[int] = None,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """W_hat [n_out, n_in] float32 = S + U V (sizes default to U / V's, else to the tile grid)."""
    if not _is_device(values):
        raise ValueError("values must be a device tensor")
    if n_out is None:
        n_out = U.shape[0] if U is not None else values.shape[0] * 16
    if n_in is None:
        n_in = V.shape[1] if V is not None else values.shape[1] * 64
    _dtype_code(values)
    _check_packed_in(values, meta, n_out, n_in, values.dtype, values.device)
    r = _check_factors(U, V, n_out, n_in, values.dtype, values.device)
    if out is None:
        with torch.cuda.stream(_the_stream(stream)):
            out = torch.empty((n_out, n_in), dtype=torch.float32, device=values.device)
    _expect(out, "out", torch.float32, n_out * n_in, values.device, (n_out, n_in))
    _check("splr_dense_reconstruct",
           lib().splr_dense_reconstruct(_dev(values, "values"), _dev(meta, "meta"), _dev(U, "U"), _dev(V, "V"),
                                        n_out, n_in, r, _dtype_code(values), _dev(out, "out"), _stream(stream)))
    return out


MAX_CHOL_K = 192


def gram_f64(Y: torch.Tensor, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """G = Y^T Y in float64 for float32 Y [n, k] (k <= 192), on the device (splr_gram_f64)."""
    n, k = _matrix(Y, "Y")
    if not 1 <= k <= MAX_CHOL_K:
        raise ValueError(f"Y has {k} columns; splr_gram_f64 takes 1 .. {MAX_CHOL_K}")
    _expect(Y, "Y", torch.float32, n * k, Y.device)
    need = int(lib().splr_gram_workspace_bytes(n, k))
    if need == 0:
        raise ValueError(f"Y of shape {(n, k)} is out of range for splr_gram_f64")
    with torch.cuda.stream(_the_stream(stream)):
        if out is None:
            out = torch.empty((k, k), dtype=torch.float64, device=Y.device)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=Y.device)
    _expect(out, "out", torch.float64, k * k, Y.device, (k, k))
    if not _is_device(workspace) or workspace.device != Y.device or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor on Y's device")
    _check("splr_gram_f64", lib().splr_gram_f64(_dev(Y, "Y"), n, k, _dev(out, "out"), _dev(workspace, "workspace"),
                                                workspace.numel(), _stream(stream)))
    return out


def chol_rinv(G: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """R^-1 (float32, upper triangular) for the Cholesky factor of float64 G = R^T R [k, k]
    (splr_chol_rinv); NaN entries when G is not numerically positive definite."""
    k, k2 = _matrix(G, "G")
    if k != k2 or not 1 <= k <= MAX_CHOL_K:
        raise ValueError(f"G must be square with 1 .. {MAX_CHOL_K} rows, got {(k, k2)}")
    _expect(G, "G", torch.float64, k * k, G.device)
    if out is None:
        with torch.cuda.stream(_the_stream(stream)):
            out = torch.empty((k, k), dtype=torch.float32, device=G.device)
    _expect(out, "out", torch.float32, k * k, G.device, (k, k))
    _check("splr_chol_rinv", lib().splr_chol_rinv(_dev(G, "G"), k, _dev(out, "out"), _stream(stream)))
    return out


def version() -> str:
    return lib().splr_version().decode()
