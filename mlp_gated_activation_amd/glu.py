"""Thin Python binding of the C ABI in include/glu.h (libglu.so).

Argument marshalling only: shapes, row strides, dtype codes, device pointers
and the current HIP stream go to ``glu_fwd`` / ``glu_bwd``; every element of
the result is computed by the library's gfx950 kernels.  PyTorch supplies the
device memory and the stream.  Importing this module loads the library and
raises ImportError if it has not been built (there is no fallback).

Tensors: for ``glu_fwd`` / ``glu_bwd`` the activation dimension is the last
one and must be contiguous (column stride 1); leading dimensions are merged
into rows, which must be possible without a copy ("Write a Triton SiLU-Mul
(SwiGLU) Kernel", "Common failure modes": never silently read a transposed
view).  ``glu_fwd_strided`` / ``glu_bwd_strided`` take any views whose
leading dimensions merge into one (transposed, sliced, broadcast) and pass
both strides to the library.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libglu.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with "
                      "`python -m mlp_gated_activation_amd.build` (or __graft_entry__.build())")
_lib = ctypes.CDLL(_LIB_PATH)

_i = ctypes.c_int
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_lib.glu_fwd.argtypes = [_i, _i, _i, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i, _p]
_lib.glu_fwd.restype = _i
_lib.glu_bwd.argtypes = [_i, _i, _i, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i, _p]
_lib.glu_bwd.restype = _i
_lib.glu_add_rmsnorm_fwd.argtypes = [_i, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _p, _i64, _p,
                                     ctypes.c_float, _p]
_lib.glu_add_rmsnorm_fwd.restype = _i
_lib.glu_fwd_strided.argtypes = [_i, _i, _i64, _i64] + [_p, _i64, _i64] * 3 + [_p]
_lib.glu_fwd_strided.restype = _i
_lib.glu_bwd_strided.argtypes = [_i, _i, _i64, _i64] + [_p, _i64, _i64] * 5 + [_p]
_lib.glu_bwd_strided.restype = _i
_lib.glu_gemm_fwd.argtypes = [_i, _i, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.glu_gemm_fwd.restype = _i
_lib.glu_status_string.argtypes = [_i]
_lib.glu_status_string.restype = ctypes.c_char_p
_lib.glu_version.argtypes = []
_lib.glu_version.restype = _i

KINDS = {"silu": 0, "gelu_erf": 1, "gelu_tanh": 2, "relu": 3}
LAYOUTS = {"separate": 0, "gate_up": 1}
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
STATUS = {0: "GLU_OK", 1: "GLU_ERR_NULL", 2: "GLU_ERR_SHAPE", 3: "GLU_ERR_STRIDE", 4: "GLU_ERR_ENUM",
          5: "GLU_ERR_ALIAS", 6: "GLU_ERR_INPLACE", 7: "GLU_ERR_HIP", 8: "GLU_ERR_ARG"}


class GluError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.glu_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def library_path() -> str:
    return _LIB_PATH


def version() -> int:
    return int(_lib.glu_version())


def status_string(status: int) -> str:
    return _lib.glu_status_string(status).decode()


def _code(table, key, what):
    try:
        return table[key]
    except KeyError:
        raise ValueError(f"unknown {what} {key!r}; expected one of {list(table)}") from None


def _rows(t: torch.Tensor, name: str) -> torch.Tensor:
    """View t as (rows, last) without copying."""
    if t.dim() == 0:
        raise ValueError(f"{name} must have at least one dimension")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous (stride 1), got {t.stride()}; "
                         "glu_fwd_strided / glu_bwd_strided take other layouts")
    try:
        return t.view(-1, t.shape[-1]) if t.dim() != 2 else t
    except RuntimeError as e:
        raise ValueError(f"{name}: leading dimensions cannot be merged without a copy") from e


def _ld(t2: torch.Tensor) -> int:
    return int(t2.stride(0)) if t2.shape[0] > 1 else int(t2.shape[1])


def _check(tensors, dtype, device):
    for name, t in tensors:
        if t is None:
            continue
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


# The current stream's raw handle without building a Stream object (a few
# microseconds per call, which is most of a small launch's host cost).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device, stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


class _NoGuard:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


_NO_GUARD = _NoGuard()


def _on(device):
    """Make `device` current for the launch; a no-op when it already is."""
    if device.index is None or device.index == torch.cuda.current_device():
        return _NO_GUARD
    return torch.cuda.device(device)


def _ptr(t):
    return None if t is None else t.data_ptr()


# Fast path of glu_fwd / glu_bwd for the common call: 2-D tensors with a
# contiguous last dimension, one dtype, all on the current device, torch's
# current stream.  It makes the same checks as the general path with fewer
# Python operations (a call through the general path costs about 8 us of host
# time, of which the library call and the kernel launch are about 3.7); any
# call it does not cover, errors included, goes through the general path.
_get_device = getattr(torch._C, "_cuda_getDevice", None)
_fast = _raw_stream is not None and _get_device is not None


def _rowmajor2(t, shape, dtype, dev):
    return (t.dim() == 2 and t.dtype == dtype and t.get_device() == dev and t.shape == shape
            and (t.stride(1) == 1 or shape[1] <= 1))


def _ld2(t, rows, cols):
    return t.stride(0) if rows > 1 else cols


def glu_fwd(kind: str, layout: str, a: torch.Tensor, b: torch.Tensor | None = None,
            y: torch.Tensor | None = None, inplace: bool = False, stream=None) -> torch.Tensor:
    """y = act(a) * b.  layout "separate": a, b of shape (..., I).
    layout "gate_up": a is x of shape (..., 2I), b is None.
    inplace: the result overwrites b (separate) or x[..., I:] (gate_up) and
    that tensor (view) is returned; otherwise y (allocated if None) is."""
    if stream is None and layout == "separate" and b is not None and _fast:
        k, dt, dev, shape = KINDS.get(kind), DTYPES.get(a.dtype), a.get_device(), a.shape
        if (k is not None and dt is not None and dev >= 0 and dev == _get_device()
                and _rowmajor2(a, shape, a.dtype, dev) and _rowmajor2(b, shape, a.dtype, dev)):
            rows, cols = shape
            if inplace:
                if y is None:
                    st = _lib.glu_fwd(k, 0, dt, rows, cols, a.data_ptr(), _ld2(a, rows, cols), b.data_ptr(),
                                      _ld2(b, rows, cols), None, 0, 1, _raw_stream(dev))
                    if st != 0:
                        raise GluError(st, "glu_fwd")
                    return b
            else:
                if y is None:
                    y = a.new_empty(shape)     # a's dtype and device, contiguous
                if _rowmajor2(y, shape, a.dtype, dev):
                    st = _lib.glu_fwd(k, 0, dt, rows, cols, a.data_ptr(), _ld2(a, rows, cols), b.data_ptr(),
                                      _ld2(b, rows, cols), y.data_ptr(), _ld2(y, rows, cols), 0, _raw_stream(dev))
                    if st != 0:
                        raise GluError(st, "glu_fwd")
                    return y
    k = _code(KINDS, kind, "kind")
    lay = _code(LAYOUTS, layout, "layout")
    dt = _code(DTYPES, a.dtype, "dtype")
    if a.device.type != "cuda":
        raise ValueError("tensors must be on a ROCm (cuda) device")
    a2 = _rows(a, "a")
    if lay == 0:
        if b is None:
            raise ValueError("layout 'separate' needs b")
        if b.shape != a.shape:
            raise ValueError(f"a{tuple(a.shape)} and b{tuple(b.shape)} differ in shape")
        cols = a.shape[-1]
        out_shape = a.shape
        b2 = _rows(b, "b")
    else:
        if b is not None:
            raise ValueError("layout 'gate_up' takes x as a and no b")
        if a.shape[-1] % 2:
            raise ValueError(f"gate_up input width {a.shape[-1]} is odd")
        cols = a.shape[-1] // 2
        out_shape = a.shape[:-1] + (cols,)
        b2 = None
    if inplace:
        if y is not None:
            raise ValueError("inplace=True writes over b; do not pass y")
        out = b if lay == 0 else a[..., cols:]
        y2 = None
    else:
        if y is None:
            y = torch.empty(out_shape, dtype=a.dtype, device=a.device)
        if tuple(y.shape) != tuple(out_shape):
            raise ValueError(f"y has shape {tuple(y.shape)}, expected {tuple(out_shape)}")
        out = y
        y2 = _rows(y, "y")
    _check([("b", b), ("y", y)], a.dtype, a.device)
    rows = a2.shape[0]
    with _on(a.device):
        st = _lib.glu_fwd(k, lay, dt, rows, cols,
                          _ptr(a2), _ld(a2),
                          _ptr(b2), _ld(b2) if b2 is not None else 0,
                          _ptr(y2), _ld(y2) if y2 is not None else 0,
                          1 if inplace else 0, _stream(a.device, stream))
    if st != 0:
        raise GluError(st, "glu_fwd")
    return out


def glu_bwd(kind: str, layout: str, a: torch.Tensor, b: torch.Tensor | None, dy: torch.Tensor,
            da: torch.Tensor | None = None, db: torch.Tensor | None = None, inplace: bool = True,
            stream=None):
    """da = dy * act'(a) * b, db = dy * act(a).
    separate: returns (da, db); with inplace they are a and b themselves.
    gate_up: a is x (..., 2I), b is None; returns dx = [da | db] of x's shape
    (x itself when inplace; otherwise `da` is dx, allocated if None)."""
    if stream is None and inplace and layout == "separate" and b is not None and da is None and db is None and _fast:
        k, dt, dev, shape = KINDS.get(kind), DTYPES.get(a.dtype), a.get_device(), a.shape
        if (k is not None and dt is not None and dev >= 0 and dev == _get_device()
                and _rowmajor2(a, shape, a.dtype, dev) and _rowmajor2(b, shape, a.dtype, dev)
                and _rowmajor2(dy, shape, a.dtype, dev)):
            rows, cols = shape
            st = _lib.glu_bwd(k, 0, dt, rows, cols, a.data_ptr(), _ld2(a, rows, cols), b.data_ptr(),
                              _ld2(b, rows, cols), dy.data_ptr(), _ld2(dy, rows, cols), None, 0, None, 0, 1,
                              _raw_stream(dev))
            if st != 0:
                raise GluError(st, "glu_bwd")
            return a, b
    k = _code(KINDS, kind, "kind")
    lay = _code(LAYOUTS, layout, "layout")
    dt = _code(DTYPES, a.dtype, "dtype")
    if a.device.type != "cuda":
        raise ValueError("tensors must be on a ROCm (cuda) device")
    a2 = _rows(a, "a")
    if lay == 0:
        if b is None or b.shape != a.shape:
            raise ValueError("layout 'separate' needs b of a's shape")
        cols = a.shape[-1]
        b2 = _rows(b, "b")
        g_shape = a.shape
    else:
        if b is not None:
            raise ValueError("layout 'gate_up' takes x as a and no b")
        if a.shape[-1] % 2:
            raise ValueError(f"gate_up input width {a.shape[-1]} is odd")
        cols = a.shape[-1] // 2
        b2 = None
        g_shape = a.shape[:-1] + (cols,)
    if tuple(dy.shape) != tuple(g_shape):
        raise ValueError(f"dy has shape {tuple(dy.shape)}, expected {tuple(g_shape)}")
    dy2 = _rows(dy, "dy")
    if inplace:
        if da is not None or db is not None:
            raise ValueError("inplace=True writes over a and b; do not pass da/db")
        da2 = db2 = None
        result = (a, b) if lay == 0 else a
    else:
        if lay == 0:
            da = torch.empty_like(a) if da is None else da
            db = torch.empty_like(a) if db is None else db
            if da.shape != a.shape or db.shape != a.shape:
                raise ValueError("da and db must have a's shape")
            da2, db2 = _rows(da, "da"), _rows(db, "db")
            result = (da, db)
        else:
            if db is not None:
                raise ValueError("layout 'gate_up' writes dx through da; db must be None")
            da = torch.empty_like(a) if da is None else da
            if da.shape != a.shape:
                raise ValueError("dx must have x's shape")
            da2, db2 = _rows(da, "dx"), None
            result = da
    _check([("b", b), ("dy", dy), ("da", da), ("db", db)], a.dtype, a.device)
    rows = a2.shape[0]
    with _on(a.device):
        st = _lib.glu_bwd(k, lay, dt, rows, cols,
                          _ptr(a2), _ld(a2),
                          _ptr(b2), _ld(b2) if b2 is not None else 0,
                          _ptr(dy2), _ld(dy2),
                          _ptr(da2), _ld(da2) if da2 is not None else 0,
                          _ptr(db2), _ld(db2) if db2 is not None else 0,
                          1 if inplace else 0, _stream(a.device, stream))
    if st != 0:
        raise GluError(st, "glu_bwd")
    return result


def glu_add_rmsnorm_fwd(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                        h: torch.Tensor | None = None, y: torch.Tensor | None = None, rstd=False,
                        stream=None):
    """Fused residual add + RMSNorm forward over the last dimension.

    h = x + residual (allocated if None; pass h=x or h=residual to update the
    residual stream in place), y = h * rstd * gamma (allocated if None),
    rstd = 1/sqrt(mean(h^2) + eps) per row: with rstd=True a float32 tensor
    of the leading shape is allocated and returned, a float32 tensor may be
    passed instead, and rstd=False skips it.  Returns (h, y, rstd or None).
    ("Write a Triton Fused Add+RMSNorm Kernel", Required reasoning process.)
    """
    dt = _code(DTYPES, x.dtype, "dtype")
    if x.device.type != "cuda":
        raise ValueError("tensors must be on a ROCm (cuda) device")
    if residual.shape != x.shape:
        raise ValueError(f"residual{tuple(residual.shape)} differs from x{tuple(x.shape)}")
    hidden = x.shape[-1]
    if gamma.shape != (hidden,) or (hidden > 1 and gamma.stride(0) != 1):
        raise ValueError(f"gamma must be a contiguous ({hidden},) tensor")
    h = torch.empty_like(x) if h is None else h
    y = torch.empty_like(x) if y is None else y
    if h.shape != x.shape or y.shape != x.shape:
        raise ValueError("h and y must have x's shape")
    _check([("residual", residual), ("gamma", gamma), ("h", h), ("y", y)], x.dtype, x.device)
    lead = x.shape[:-1]
    if rstd is True:
        rstd = torch.empty(lead, dtype=torch.float32, device=x.device)
    elif rstd is False or rstd is None:
        rstd = None
    if rstd is not None and (rstd.dtype != torch.float32 or rstd.numel() != x.numel() // max(hidden, 1)
                             or not rstd.is_contiguous()):
        raise ValueError("rstd must be a contiguous float32 tensor with one value per row")
    x2, r2, h2, y2 = (_rows(t, n) for t, n in ((x, "x"), (residual, "residual"), (h, "h"), (y, "y")))
    rows = x2.shape[0] if x.dim() > 0 else 0
    with _on(x.device):
        st = _lib.glu_add_rmsnorm_fwd(dt, rows, hidden, _ptr(x2), _ld(x2), _ptr(r2), _ld(r2), _ptr(gamma),
                                      _ptr(h2), _ld(h2), _ptr(y2), _ld(y2), _ptr(rstd), float(eps),
                                      _stream(x.device, stream))
    if st != 0:
        raise GluError(st, "glu_add_rmsnorm_fwd")
    return h, y, rstd


def _view2(t: torch.Tensor, name: str):
    """(rows, cols, row stride, column stride) of t seen as a 2-D matrix over
    its last dimension, without copying."""
    if t.dim() == 0:
        raise ValueError(f"{name} must have at least one dimension")
    if t.dim() == 1:
        return 1, t.shape[0], t.shape[0], t.stride(0)
    try:
        v = t.view(-1, t.shape[-1])
    except RuntimeError as e:
        raise ValueError(f"{name}: leading dimensions cannot be merged without a copy") from e
    return v.shape[0], v.shape[1], v.stride(0), v.stride(1)


def _strided_operands(named, shape, dtype, device):
    out = []
    for name, t in named:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        _, _, rs, cs = _view2(t, name)
        out += [_ptr(t), rs, cs]
    return out


def glu_fwd_strided(kind: str, a: torch.Tensor, b: torch.Tensor, y: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """y = act(a) * b for views a, b, y of one shape and any strides.  y is
    allocated with a's layout when None; y may be a or b itself (in place)."""
    k = _code(KINDS, kind, "kind")
    dt = _code(DTYPES, a.dtype, "dtype")
    if a.device.type != "cuda":
        raise ValueError("tensors must be on a ROCm (cuda) device")
    if y is None:
        y = torch.empty_like(a)
    rows, cols, _, _ = _view2(a, "a")
    ops = _strided_operands([("a", a), ("b", b), ("y", y)], a.shape, a.dtype, a.device)
    with _on(a.device):
        st = _lib.glu_fwd_strided(k, dt, rows, cols, *ops, _stream(a.device, stream))
    if st != 0:
        raise GluError(st, "glu_fwd_strided")
    return y


def glu_bwd_strided(kind: str, a: torch.Tensor, b: torch.Tensor, dy: torch.Tensor,
                    da: torch.Tensor | None = None, db: torch.Tensor | None = None, stream=None):
    """da = dy * act'(a) * b, db = dy * act(a) for views of one shape and any
    strides.  da, db are allocated with a's layout when None; pass da=a,
    db=b to write the gradients over the inputs.  Returns (da, db)."""
    k = _code(KINDS, kind, "kind")
    dt = _code(DTYPES, a.dtype, "dtype")
    if a.device.type != "cuda":
        raise ValueError("tensors must be on a ROCm (cuda) device")
    da = torch.empty_like(a) if da is None else da
    db = torch.empty_like(a) if db is None else db
    rows, cols, _, _ = _view2(a, "a")
    ops = _strided_operands([("a", a), ("b", b), ("dy", dy), ("da", da), ("db", db)], a.shape, a.dtype,
                            a.device)
    with _on(a.device):
        st = _lib.glu_bwd_strided(k, dt, rows, cols, *ops, _stream(a.device, stream))
    if st != 0:
        raise GluError(st, "glu_bwd_strided")
    return da, db


def glu_gemm_fwd(kind: str, x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor | None = None,
                 h: torch.Tensor | None = None, gu=False, stream=None):
    """h = act(x @ w_gate^T) * (x @ w_up^T) on the matrix cores, with the
    activation in the GEMM epilogue ("Fused Kernels", section 4).

    x: (..., K); w_gate, w_up: (N, K), the weights of two linear layers; with
    w_up None, w_gate is one fused (2N, K) [gate | up] weight.  h (allocated
    if None) has shape (..., N).  gu=True also returns the pre-activations in
    the [gate | up] layout (..., 2N) (a tensor may be passed instead), which
    glu_bwd(kind, "gate_up", ...) takes.  Returns h, or (h, gu).
    bf16 / fp16 only; K and the row strides must be multiples of 8.
    """
    k = _code(KINDS, kind, "kind")
    dt = _code(DTYPES, x.dtype, "dtype")
    if x.device.type != "cuda":
        raise ValueError("tensors must be on a ROCm (cuda) device")
    if w_up is None:
        if w_gate.dim() != 2 or w_gate.shape[0] % 2:
            raise ValueError("a fused [gate | up] weight must be (2N, K)")
        n = w_gate.shape[0] // 2
        w_gate, w_up = w_gate[:n], w_gate[n:]
    if w_gate.dim() != 2 or w_up.shape != w_gate.shape or w_gate.shape[1] != x.shape[-1]:
        raise ValueError(f"weights must be (N, K) with K = x.shape[-1]; got {tuple(w_gate.shape)}, "
                         f"{tuple(w_up.shape)} for x {tuple(x.shape)}")
    N, K = w_gate.shape
    x2 = _rows(x, "x")
    wg2, wu2 = _rows(w_gate, "w_gate"), _rows(w_up, "w_up")
    out_shape = x.shape[:-1] + (N,)
    if h is None:
        h = torch.empty(out_shape, dtype=x.dtype, device=x.device)
    if tuple(h.shape) != tuple(out_shape):
        raise ValueError(f"h has shape {tuple(h.shape)}, expected {tuple(out_shape)}")
    h2 = _rows(h, "h")
    if gu is True:
        gu = torch.empty(x.shape[:-1] + (2 * N,), dtype=x.dtype, device=x.device)
    elif gu is False or gu is None:
        gu = None
    if gu is not None and tuple(gu.shape) != tuple(x.shape[:-1] + (2 * N,)):
        raise ValueError(f"gu has shape {tuple(gu.shape)}, expected {tuple(x.shape[:-1] + (2 * N,))}")
    gu2 = _rows(gu, "gu") if gu is not None else None
    _check([("w_gate", w_gate), ("w_up", w_up), ("h", h), ("gu", gu)], x.dtype, x.device)
    M = x2.shape[0]
    with _on(x.device):
        st = _lib.glu_gemm_fwd(k, dt, M, N, K, _ptr(x2), _ld(x2), _ptr(wg2), _ld(wg2), _ptr(wu2), _ld(wu2),
                               _ptr(h2), _ld(h2), _ptr(gu2), _ld(gu2) if gu2 is not None else 0,
                               _stream(x.device, stream))
    if st != 0:
        raise GluError(st, "glu_gemm_fwd")
    return (h, gu) if gu is not None else h
