"""Binding of the data-movement reference kernels (include/glu_ref.h,
libglu_ref.so): the access pattern and launch shape of the streaming
forward and backward with no arithmetic, timed beside them as the ceiling a
kernel of that traffic reaches.  Used by the benchmark; not part of the
method.  Raises ImportError if the library has not been built."""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libglu_ref.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m mlp_gated_activation_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)
_p, _u64 = ctypes.c_void_p, ctypes.c_uint64
_lib.glu_ref_fwd_mix.argtypes = [_p, _p, _p, _u64, _p]
_lib.glu_ref_bwd_mix.argtypes = [_p, _p, _p, _p, _p, _u64, _p]
_lib.glu_ref_rms_mix.argtypes = [_p, _p, _p, _p, _u64, _p]
_lib.glu_ref_copy.argtypes = [_p, _p, _u64, _p]
_i64 = ctypes.c_int64
_lib.glu_ref_tile_bwd_mix.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _p]
_lib.glu_ref_tile_fwd_mix.argtypes = [_p, _p, _p, _i64, _i64, _p]
for _f in (_lib.glu_ref_fwd_mix, _lib.glu_ref_bwd_mix, _lib.glu_ref_rms_mix, _lib.glu_ref_copy,
           _lib.glu_ref_tile_bwd_mix, _lib.glu_ref_tile_fwd_mix):
    _f.restype = ctypes.c_int


def library_path() -> str:
    return _LIB_PATH


def _nbytes(ts):
    n = ts[0].numel() * ts[0].element_size()
    for t in ts:
        if not t.is_contiguous() or t.numel() * t.element_size() != n:
            raise ValueError("reference kernels take contiguous tensors of equal byte size")
    return n


def _go(st, name):
    if st != 0:
        raise RuntimeError(f"{name} failed with status {st}")


def _raw(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def fwd_mix(a, b, y):
    """Read a and b, write y: the forward's bytes and access pattern."""
    _go(_lib.glu_ref_fwd_mix(a.data_ptr(), b.data_ptr(), y.data_ptr(), _nbytes([a, b, y]), _raw(a)),
        "glu_ref_fwd_mix")


def bwd_mix(a, b, dy, da, db):
    """Read a, b and dy, write da and db: the backward's bytes and pattern."""
    _go(_lib.glu_ref_bwd_mix(a.data_ptr(), b.data_ptr(), dy.data_ptr(), da.data_ptr(), db.data_ptr(),
                             _nbytes([a, b, dy, da, db]), _raw(a)), "glu_ref_bwd_mix")


def rms_mix(x, r, h, y):
    """Read x and residual, write h and y: the add + RMSNorm forward's bytes."""
    _go(_lib.glu_ref_rms_mix(x.data_ptr(), r.data_ptr(), h.data_ptr(), y.data_ptr(), _nbytes([x, r, h, y]), _raw(x)),
        "glu_ref_rms_mix")


def _tile_check(rowmajor, transposed):
    rows, cols = rowmajor[0].shape
    for t in rowmajor:
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.shape != (rows, cols):
            raise ValueError("tiled references take contiguous bf16 (rows, cols) row-major operands")
    if transposed.dtype != torch.bfloat16 or not transposed.is_contiguous() or transposed.shape != (cols, rows):
        raise ValueError("the transposed operand must be a contiguous bf16 (cols, rows) tensor")
    return rows, cols


def tile_bwd_mix(a, b, dyT, da, db):
    """The strided backward's bytes in the tiled kernel's pattern: a, b, da,
    db row-major (rows, cols), dyT stored as (cols, rows)."""
    rows, cols = _tile_check([a, b, da, db], dyT)
    _go(_lib.glu_ref_tile_bwd_mix(a.data_ptr(), b.data_ptr(), dyT.data_ptr(), da.data_ptr(), db.data_ptr(), rows, cols,
                                  _raw(a)), "glu_ref_tile_bwd_mix")


def tile_fwd_mix(a, b, yT):
    """The strided forward's bytes in the tiled kernel's pattern: a, b
    row-major (rows, cols), yT stored as (cols, rows)."""
    rows, cols = _tile_check([a, b], yT)
    _go(_lib.glu_ref_tile_fwd_mix(a.data_ptr(), b.data_ptr(), yT.data_ptr(), rows, cols, _raw(a)), "glu_ref_tile_fwd_mix")


def copy(src, dst):
    """dst := src, 16-byte vectors."""
    _go(_lib.glu_ref_copy(src.data_ptr(), dst.data_ptr(), _nbytes([src, dst]), _raw(src)), "glu_ref_copy")
