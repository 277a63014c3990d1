"""ctypes binding of ``libsketchmm.so`` (the C ABI in ``include/sketch_matmul.h``).

Argument marshalling only: every step of the sketched matmul runs in the HIP
library. PyTorch provides device memory (``tensor.data_ptr()``) and the
current HIP stream; nothing here computes on the host, and there is no
fallback: when the library is missing or its call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libsketchmm.so")
HEADER = os.path.join(ROOT, "include", "sketch_matmul.h")

SKM_F32, SKM_F16, SKM_BF16 = 0, 1, 2
STATUS = {
    0: "SKM_OK", -1: "SKM_EINVAL", -2: "SKM_EUNSUPPORTED", -3: "SKM_EALIGN",
    -4: "SKM_EWORKSPACE", -5: "SKM_EHIP", -6: "SKM_EALIAS",
}


class SketchError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_vp = ctypes.c_void_p
_c_size = ctypes.c_size_t
_c_f32 = ctypes.c_float

_SIGNATURES = {
    "sketch_matmul_fwd": (_c_int, [_c_vp, _c_int, _c_vp, _c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int,
                                   _c_vp, _c_vp, _c_size, _c_vp]),
    "sketch_matmul_fwd_workspace": (_c_size, [_c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int]),
    "sketch_matmul_fwd_multi": (_c_int, [_c_vp, _c_int, _c_vp, _c_vp, _c_int, _c_vp, _c_int, _c_i64, _c_i64, _c_i64,
                                         _c_int, _c_int, _c_vp, _c_vp]),
    "sketch_matmul_bwd": (_c_int, [_c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int,
                                   _c_vp, _c_vp, _c_int, _c_vp, _c_size, _c_vp]),
    "sketch_matmul_bwd_workspace": (_c_size, [_c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int]),
    "sketch_matmul_bwd_noalloc": (_c_int, [_c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int,
                                           _c_int, _c_vp, _c_vp, _c_int, _c_vp]),
    "sketch_dequant": (_c_int, [_c_vp, _c_vp, _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_vp, _c_vp]),
    "sketch_unpack_indices": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp]),
    "sketch_lut_adam_step": (_c_int, [_c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_f32, _c_f32,
                                      _c_f32, _c_f32, _c_f32, _c_f32, _c_vp]),
    "sketch_lut_sgd_step": (_c_int, [_c_vp, _c_vp, _c_int, _c_vp, _c_vp, _c_i64, _c_f32, _c_f32, _c_f32, _c_f32,
                                     _c_vp]),
    "sketch_column_weights": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp]),
    "sketch_lloyd": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_int, _c_vp]),
    "sketch_map_workspace": (_c_size, [_c_i64]),
    "sketch_map": (_c_int, [_c_vp, _c_vp, _c_vp, _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_vp, _c_vp, _c_size,
                            _c_vp]),
    "sketch_hessian_factor_workspace": (_c_size, [_c_i64]),
    "sketch_hessian_factor": (_c_int, [_c_vp, _c_i64, ctypes.c_double, _c_vp, _c_vp, _c_size, _c_vp]),
    "sketch_status_str": (ctypes.c_char_p, [_c_int]),
    "sketch_version": (_c_int, []),
}


def library_path() -> str:
    return os.environ.get("SKETCHMM_LIB", LIB_PATH)


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} not found: build it with `python -m lut_sketched_matmul_amd.build`")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list:
    """Names of the functions declared in include/sketch_matmul.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sketch_\w+)\s*\(", text)))


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SketchError(fn, status, lib().sketch_status_str(status).decode())


# --------------------------------------------------------------------------
# torch-facing wrappers
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: SKM_F32, torch.float16: SKM_F16, torch.bfloat16: SKM_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _require_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# The C ABI takes raw pointers and sizes, so it cannot see a tensor's extent:
# every tensor's shape (or element count) and dtype is checked against the
# sizes passed with it before the call, so that a wrong buffer is an exception
# here and never an out-of-bounds access on the device.

_FLOAT_DTYPES = ("float32", "float16", "bfloat16")


def _dtype_name(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _expect(t, name: str, shape=None, numel=None, dtypes=None):
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if dtypes is not None and _dtype_name(t) not in dtypes:
        raise TypeError(f"{name} has dtype {_dtype_name(t)}, expected one of {dtypes}")


def _check_bits(b: int, d: int):
    if b not in (2, 3, 4):
        raise ValueError(f"bit width b = {b}: supported are 2, 3 and 4")
    if d < 0 or (d * b) % 8:
        raise ValueError(f"d = {d} columns of {b} bits do not fill whole bytes")


def _check_sketch(idx_packed, lut, n: int, d: int, b: int, gpr: int, n_sets=None, lut_name="lut"):
    """idx_packed [n, d*b/8] uint8 and tables of n (x n_sets) rows of gpr groups of 2^b entries."""
    _check_bits(b, d)
    if gpr < 1:
        raise ValueError(f"gpr = {gpr} must be at least 1")
    _expect(idx_packed, "idx_packed", shape=(n, d * b // 8), dtypes=("uint8",))
    count = n * gpr * (1 << b) * (1 if n_sets is None else n_sets)
    _expect(lut, lut_name, numel=count, dtypes=_FLOAT_DTYPES)
    if n_sets is not None and (lut.dim() < 1 or lut.shape[0] != n_sets):
        raise ValueError(f"{lut_name} must have the table sets as its first dimension")


def _matrix(t, name: str):
    if t.dim() != 2:
        raise ValueError(f"{name} must be a matrix, got {t.dim()} dimensions")
    return t.shape


def sketch_matmul_fwd_workspace(m: int, n: int, d: int, b: int, gpr: int, x_dtype: int, lut_dtype: int) -> int:
    """Bytes of device workspace sketch_matmul_fwd needs for these sizes and dtypes."""
    return int(lib().sketch_matmul_fwd_workspace(m, n, d, b, gpr, x_dtype, lut_dtype))


def _workspace(ws, need: int, device):
    """The caller's workspace (checked), or a new one of `need` bytes, or None."""
    torch = _torch()
    if ws is not None:
        if ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes, {need} needed")
        return ws
    return torch.empty(need, dtype=torch.uint8, device=device) if need else None


def sketch_matmul_fwd(X, idx_packed, lut, b: int, gpr: int, out=None, workspace=None, stream=None):
    """Y = X W^T with W[i, j] = lut[i, j // (d/gpr), idx[i, j]].

    X [m, d] (f32/f16/bf16), idx_packed [n, d*b/8] uint8, lut [n, gpr, 2^b].
    Returns Y [m, n] in X's dtype. workspace: optional uint8 device buffer of
    at least sketch_matmul_fwd_workspace(...) bytes (allocated here when
    needed and omitted).
    """
    torch = _torch()
    m, d = _matrix(X, "X")
    n = idx_packed.shape[0]
    _expect(X, "X", dtypes=_FLOAT_DTYPES)
    _check_sketch(idx_packed, lut, n, d, b, gpr)
    _expect(out, "out", shape=(m, n), dtypes=(_dtype_name(X),))
    _expect(workspace, "workspace", dtypes=("uint8",))
    _require_device(X, idx_packed, lut, out, workspace)
    if out is None:
        out = torch.empty((m, n), dtype=X.dtype, device=X.device)
    ws = _workspace(workspace, sketch_matmul_fwd_workspace(m, n, d, b, gpr, dtype_code(X), dtype_code(lut)),
                    X.device)
    st = lib().sketch_matmul_fwd(X.data_ptr(), dtype_code(X), idx_packed.data_ptr(), lut.data_ptr(),
                                 dtype_code(lut), m, n, d, b, gpr, out.data_ptr() if out.numel() else None,
                                 ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                                 _stream_ptr(stream))
    _check("sketch_matmul_fwd", st)
    return out


def sketch_matmul_fwd_multi(X, idx_packed, luts, lut_set, b: int, gpr: int, out=None, stream=None):
    """Y[t] = X[t] W_{lut_set[t]}^T: one table set per token over shared indices.

    X [m, d] (f16/bf16, m <= 16), idx_packed [n, d*b/8] uint8, luts [n_sets, n,
    gpr, 2^b], lut_set [m] int32 (device). Returns Y [m, n] in X's dtype.
    """
    torch = _torch()
    m, d = _matrix(X, "X")
    n = idx_packed.shape[0]
    _expect(X, "X", dtypes=_FLOAT_DTYPES)
    if luts.dim() < 1:
        raise ValueError("luts must have the table sets as its first dimension")
    _check_sketch(idx_packed, luts, n, d, b, gpr, n_sets=luts.shape[0], lut_name="luts")
    if lut_set.dtype != torch.int32 or lut_set.numel() != m:
        raise ValueError("lut_set must be an int32 tensor with one entry per token")
    _expect(out, "out", shape=(m, n), dtypes=(_dtype_name(X),))
    _require_device(X, idx_packed, luts, lut_set, out)
    if out is None:
        out = torch.empty((m, n), dtype=X.dtype, device=X.device)
    st = lib().sketch_matmul_fwd_multi(X.data_ptr(), dtype_code(X), idx_packed.data_ptr(), luts.data_ptr(),
                                       dtype_code(luts), lut_set.data_ptr() if m else None, luts.shape[0], m, n, d,
                                       b, gpr, out.data_ptr() if out.numel() else None, _stream_ptr(stream))
    _check("sketch_matmul_fwd_multi", st)
    return out


def sketch_matmul_bwd_workspace(m: int, n: int, d: int, b: int, gpr: int, io_dtype: int, lut_dtype: int) -> int:
    """Bytes of device workspace sketch_matmul_bwd needs for these sizes and dtypes."""
    return int(lib().sketch_matmul_bwd_workspace(m, n, d, b, gpr, io_dtype, lut_dtype))


def sketch_matmul_bwd(dY, X, idx_packed, lut, b: int, gpr: int, d: Optional[int] = None,
                      need_dx: bool = True, need_dlut: bool = True, dlut_out=None, accumulate: bool = False,
                      workspace=None, stream=None) -> Tuple[object, object]:
    """(dX, dLUT) of the sketched matmul; both fp32. dLUT sums shared entries.

    dY [m, n], X [m, d] in the same dtype (X may be None when need_dlut is
    False; then d must be given), idx_packed [n, d*b/8] uint8, lut [n, gpr,
    2^b]. dlut_out: optional fp32 [n, gpr, 2^b] to write (accumulate=True adds
    to it). workspace: optional uint8 device buffer of at least
    sketch_matmul_bwd_workspace(...) bytes (allocated here when omitted).
    """
    torch = _torch()
    m, n = _matrix(dY, "dY")
    _expect(dY, "dY", dtypes=_FLOAT_DTYPES)
    if X is not None:
        mx, dx_cols = _matrix(X, "X")
        if d is not None and d != dx_cols:
            raise ValueError(f"d = {d} does not match X's {dx_cols} columns")
        d = dx_cols
        _expect(X, "X", shape=(m, d), dtypes=(_dtype_name(dY),))
    elif need_dlut:
        raise ValueError("the table gradient needs X")
    if d is None:
        raise ValueError("d must be given when X is None")
    K = 1 << b
    _check_sketch(idx_packed, lut, n, d, b, gpr)
    _expect(dlut_out, "dlut_out", shape=(n, gpr, K), dtypes=("float32",))
    _expect(workspace, "workspace", dtypes=("uint8",))
    _require_device(dY, X, idx_packed, lut, dlut_out, workspace)
    dX = torch.empty((m, d), dtype=torch.float32, device=dY.device) if need_dx else None
    dL = None
    if need_dlut:
        dL = dlut_out if dlut_out is not None else torch.empty((n, gpr, K), dtype=torch.float32, device=dY.device)
    workspace = _workspace(workspace, sketch_matmul_bwd_workspace(m, n, d, b, gpr, dtype_code(dY), dtype_code(lut)),
                           dY.device)
    st = lib().sketch_matmul_bwd(
        dY.data_ptr() if dY.numel() else None, X.data_ptr() if (X is not None and X.numel()) else None,
        dtype_code(dY), idx_packed.data_ptr(), lut.data_ptr(), dtype_code(lut), m, n, d, b, gpr,
        dX.data_ptr() if (dX is not None and dX.numel()) else None, dL.data_ptr() if dL is not None else None,
        1 if accumulate else 0, workspace.data_ptr() if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, _stream_ptr(stream))
    _check("sketch_matmul_bwd", st)
    return dX, dL


def sketch_matmul_bwd_noalloc(dY, X, idx_packed, lut, b: int, gpr: int, dx_out=None, dlut_out=None,
                              accumulate: bool = False, stream=None) -> None:
    """The backward pass into caller-given outputs with the library's own scratch (no allocation at all).

    dY [m, n], X [m, d] in the same dtype, idx_packed [n, d*b/8] uint8, lut [n, gpr, 2^b]; dx_out fp32
    [m, d] and dlut_out fp32 [n, gpr, 2^b] are written when given (at least one of them). Nothing is
    allocated here or in the library; calls that overlap in time on one GPU race on its scratch.
    """
    m, n = _matrix(dY, "dY")
    mx, d = _matrix(X, "X")
    _expect(dY, "dY", dtypes=_FLOAT_DTYPES)
    _expect(X, "X", shape=(m, d), dtypes=(_dtype_name(dY),))
    _check_sketch(idx_packed, lut, n, d, b, gpr)
    _expect(dx_out, "dx_out", shape=(m, d), dtypes=("float32",))
    _expect(dlut_out, "dlut_out", shape=(n, gpr, 1 << b), dtypes=("float32",))
    if dx_out is None and dlut_out is None:
        raise ValueError("give dx_out, dlut_out or both")
    _require_device(dY, X, idx_packed, lut, dx_out, dlut_out)
    st = lib().sketch_matmul_bwd_noalloc(
        dY.data_ptr() if dY.numel() else None, X.data_ptr() if X.numel() else None, dtype_code(dY),
        idx_packed.data_ptr(), lut.data_ptr(), dtype_code(lut), m, n, d, b, gpr,
        dx_out.data_ptr() if (dx_out is not None and dx_out.numel()) else None,
        dlut_out.data_ptr() if dlut_out is not None else None, 1 if accumulate else 0, _stream_ptr(stream))
    _check("sketch_matmul_bwd_noalloc", st)


def sketch_dequant(idx_packed, lut, d: int, b: int, gpr: int, stream=None):
    """Dense W [n, d] in the table dtype (a checking aid)."""
    torch = _torch()
    n = idx_packed.shape[0]
    _check_sketch(idx_packed, lut, n, d, b, gpr)
    _require_device(idx_packed, lut)
    W = torch.empty((n, d), dtype=lut.dtype, device=lut.device)
    st = lib().sketch_dequant(idx_packed.data_ptr(), lut.data_ptr(), dtype_code(lut), n, d, b, gpr, W.data_ptr(),
                              _stream_ptr(stream))
    _check("sketch_dequant", st)
    return W


def sketch_unpack_indices(idx_packed, d: int, b: int, stream=None):
    """One uint8 per weight: idx [n, d] (a checking aid)."""
    torch = _torch()
    n = idx_packed.shape[0]
    _check_bits(b, d)
    _expect(idx_packed, "idx_packed", shape=(n, d * b // 8), dtypes=("uint8",))
    _require_device(idx_packed)
    out = torch.empty((n, d), dtype=torch.uint8, device=idx_packed.device)
    st = lib().sketch_unpack_indices(idx_packed.data_ptr(), n, d, b, out.data_ptr(), _stream_ptr(stream))
    _check("sketch_unpack_indices", st)
    return out


def _copy_args(lut):
    """(pointer, dtype code) of an optional 16-bit compute copy."""
    if lut is None:
        return None, SKM_F16
    return lut.data_ptr(), dtype_code(lut)


def _check_f32(*ts):
    torch = _torch()
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise TypeError("master tables, gradients and optimizer state are fp32")


def sketch_lut_adam_step(master, grad, exp_avg, exp_avg_sq, step: int, lr: float, beta1: float = 0.9,
                         beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
                         grad_scale: float = 1.0, lut=None, stream=None) -> None:
    """One fused Adam(W) step on fp32 master tables; writes the 16-bit copy `lut` if given."""
    _require_device(master, grad, exp_avg, exp_avg_sq, lut)
    _check_f32(master, grad, exp_avg, exp_avg_sq)
    count = master.numel()
    for t in (grad, exp_avg, exp_avg_sq, lut):
        if t is not None and t.numel() != count:
            raise ValueError("all buffers must have the master's number of entries")
    lp, ldt = _copy_args(lut)
    st = lib().sketch_lut_adam_step(master.data_ptr(), lp, ldt, grad.data_ptr(), exp_avg.data_ptr(),
                                    exp_avg_sq.data_ptr(), count, step, lr, beta1, beta2, eps, weight_decay,
                                    grad_scale, _stream_ptr(stream))
    _check("sketch_lut_adam_step", st)


def sketch_lut_sgd_step(master, grad, lr: float, momentum: float = 0.0, weight_decay: float = 0.0,
                        grad_scale: float = 1.0, momentum_buf=None, lut=None, stream=None) -> None:
    """One fused SGD step on fp32 master tables; writes the 16-bit copy `lut` if given."""
    _require_device(master, grad, momentum_buf, lut)
    _check_f32(master, grad, momentum_buf)
    count = master.numel()
    for t in (grad, momentum_buf, lut):
        if t is not None and t.numel() != count:
            raise ValueError("all buffers must have the master's number of entries")
    lp, ldt = _copy_args(lut)
    st = lib().sketch_lut_sgd_step(master.data_ptr(), lp, ldt, grad.data_ptr(),
                                   momentum_buf.data_ptr() if momentum_buf is not None else None, count, lr,
                                   momentum, weight_decay, grad_scale, _stream_ptr(stream))
    _check("sketch_lut_sgd_step", st)


def sketch_column_weights(U, stream=None):
    """h[j] = 1 / [H^-1]_jj from the upper factor U (H^-1 = U^T U), fp32 [d]."""
    torch = _torch()
    d = U.shape[0]
    _expect(U, "U", shape=(d, d))
    _check_f32(U)
    _require_device(U)
    h = torch.empty(d, dtype=torch.float32, device=U.device)
    _check("sketch_column_weights", lib().sketch_column_weights(U.data_ptr(), d, h.data_ptr(), _stream_ptr(stream)))
    return h


def sketch_lloyd(W, h, b: int, gpr: int, iters: int, lut_dtype=None, out=None, stream=None):
    """Weighted Lloyd tables [n, gpr, 2^b] (fp32 unless lut_dtype / out say otherwise)."""
    torch = _torch()
    n, d = _matrix(W, "W")
    _check_f32(W, h)
    _check_bits(b, d)
    _expect(h, "h", numel=d)
    _expect(out, "out", numel=n * gpr * (1 << b), dtypes=_FLOAT_DTYPES)
    _require_device(W, h, out)
    if out is None:
        out = torch.empty((n, gpr, 1 << b), dtype=lut_dtype or torch.float32, device=W.device)
    st = lib().sketch_lloyd(W.data_ptr(), h.data_ptr(), n, d, b, gpr, iters, out.data_ptr(), dtype_code(out),
                            _stream_ptr(stream))
    _check("sketch_lloyd", st)
    return out


def sketch_map(W_work, U, lut, b: int, gpr: int, out=None, workspace=None, stream=None):
    """Error-compensated mapping -> idx_packed [n, d*b/8] uint8. W_work (fp32 [n, d]) is overwritten."""
    torch = _torch()
    n, d = _matrix(W_work, "W_work")
    _check_f32(W_work, U)
    _expect(U, "U", shape=(d, d))
    _check_sketch(out, lut, n, d, b, gpr)
    _require_device(W_work, U, lut, out, workspace)
    if out is None:
        out = torch.empty((n, d * b // 8), dtype=torch.uint8, device=W_work.device)
    ws = lib().sketch_map_workspace(n)
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=W_work.device)
    st = lib().sketch_map(W_work.data_ptr(), U.data_ptr(), lut.data_ptr(), dtype_code(lut), n, d, b, gpr,
                          out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream_ptr(stream))
    _check("sketch_map", st)
    return out


def sketch_hessian_factor(H, damp: float = 0.01, out=None, workspace=None, stream=None):
    """U [d, d] fp32, upper triangular, with U^T U = (H + damp * mean(diag H) * I)^-1, from the float64 Gram
    matrix H [d, d] of the sample inputs (only its entries with i <= j are read)."""
    torch = _torch()
    d, d2 = _matrix(H, "H")
    if d != d2:
        raise ValueError(f"H must be square, got {tuple(H.shape)}")
    _expect(H, "H", dtypes=("float64",))
    _expect(out, "out", shape=(d, d), dtypes=("float32",))
    _expect(workspace, "workspace", dtypes=("uint8",))
    _require_device(H, out, workspace)
    if out is None:
        out = torch.empty((d, d), dtype=torch.float32, device=H.device)
    ws = _workspace(workspace, lib().sketch_hessian_factor_workspace(d), H.device)
    st = lib().sketch_hessian_factor(H.data_ptr(), d, float(damp), out.data_ptr(),
                                     ws.data_ptr() if ws is not None else None,
                                     ws.numel() if ws is not None else 0, _stream_ptr(stream))
    _check("sketch_hessian_factor", st)
    return out
