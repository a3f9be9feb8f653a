"""CPU oracle for the channels-last convolution forward and backward-data passes -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and the two share no code.

The arithmetic lives in ``conv_oracle.c`` (a direct loop nest over every
output, every tap and every input channel, accumulated in float64; see the
header of that file for the definition and the pages it follows).  This module
only marshals numpy arrays into it and decodes fp16/bf16/fp32 tensors to
float64, which is exact for all three formats.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


class _Shape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "n", "d", "h", "w", "c_in", "c_out",
        "k_d", "k_h", "k_w", "s_d", "s_h", "s_w", "p_d", "p_h", "p_w",
        "q_d", "q_h", "q_w", "e_d", "e_h", "e_w", "groups")]


def _load():
    global _lib
    if _lib is None:
        # ORACLE_CONV_LIB points the wrapper at another build of conv_oracle.c; the
        # mutation tests use it to load copies with planted mistakes.
        path = os.environ.get("ORACLE_CONV_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.oracle_conv_fwd.restype = ctypes.c_int64
        lib.oracle_conv_fwd.argtypes = [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_conv_bwd_data.restype = ctypes.c_int64
        lib.oracle_conv_bwd_data.argtypes = [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_out_extent.restype = ctypes.c_int64
        lib.oracle_out_extent.argtypes = [ctypes.c_int64] * 4
        lib.oracle_out_extent_ex.restype = ctypes.c_int64
        lib.oracle_out_extent_ex.argtypes = [ctypes.c_int64] * 6
        _lib = lib
    return _lib


def _triple(v, dims):
    if isinstance(v, int):
        return (v,) * dims
    v = tuple(int(e) for e in v)
    assert len(v) == dims
    return v


def out_extent(size: int, k: int, s: int, p: int) -> int:
    """floor((size + 2p - k) / s) + 1, or 0 if the padded input is shorter than k."""
    return int(_load().oracle_out_extent(size, k, s, p))


def out_extent_ex(size: int, k: int, s: int, p: int, q: int, e: int) -> int:
    """floor((size + p + q - e*(k-1) - 1) / s) + 1 (low / high pads p / q, taps e apart)."""
    return int(_load().oracle_out_extent_ex(size, k, s, p, q, e))


def _pads(padding, dims):
    """Per-dimension (low, high) pads from an int, a tuple of ints or a tuple of pairs."""
    if isinstance(padding, int):
        return ((padding, padding),) * dims
    padding = tuple(padding)
    assert len(padding) == dims
    return tuple((int(p), int(p)) if isinstance(p, (int, np.integer)) else (int(p[0]), int(p[1]))
                 for p in padding)


def conv_fwd(x: np.ndarray, w: np.ndarray, stride=1, padding=0, rows=None,
             return_macs: bool = False, dilation=1, groups: int = 1):
    """Direct convolution, float64.

    x: (N, H, W, C_in) or (N, D, H, W, C_in); w: (C_out, KH, KW, C_in/G) or
    (C_out, KD, KH, KW, C_in/G); stride and dilation: int or per-dimension
    tuple; padding: int, per-dimension int, or per-dimension (low, high) pair;
    groups: G, dividing C_in and C_out.  Returns y with shape
    (N, [D_out,] H_out, W_out, C_out), or, when ``rows`` (flat output-position
    indices) is given, an array (len(rows), C_out).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    dims = x.ndim - 2
    assert dims in (2, 3) and w.ndim == x.ndim and w.shape[-1] * groups == x.shape[-1]
    st = _triple(stride, dims)
    dl = _triple(dilation, dims)
    pp = _pads(padding, dims)
    if dims == 2:
        x5 = x.reshape(x.shape[0], 1, *x.shape[1:])
        w5 = w.reshape(w.shape[0], 1, *w.shape[1:])
        st, dl, pp = (1,) + st, (1,) + dl, ((0, 0),) + pp
    else:
        x5, w5 = x, w
    sh = _Shape(x5.shape[0], x5.shape[1], x5.shape[2], x5.shape[3], x5.shape[4], w5.shape[0],
                w5.shape[1], w5.shape[2], w5.shape[3], *st, *(p[0] for p in pp),
                *(p[1] for p in pp), *dl, groups)
    outs = [out_extent_ex(x5.shape[1 + i], w5.shape[1 + i], st[i], pp[i][0], pp[i][1], dl[i])
            for i in range(3)]
    if rows is None:
        y = np.zeros((x5.shape[0], *outs, w5.shape[0]), dtype=np.float64)
        rows_ptr, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        y = np.zeros((rows.shape[0], w5.shape[0]), dtype=np.float64)
        rows_ptr, nrows = rows.ctypes.data, rows.shape[0]
    macs = _load().oracle_conv_fwd(ctypes.byref(sh), x5.ctypes.data, w5.ctypes.data,
                                   rows_ptr, nrows, y.ctypes.data)
    if macs < 0:
        raise ValueError("oracle rejected the shape or a row index")
    if rows is None and dims == 2:
        y = y.reshape(y.shape[0], *y.shape[2:])
    return (y, int(macs)) if return_macs else y


def conv_bwd_data(dy: np.ndarray, w: np.ndarray, x_shape, stride=1, padding=0, dilation=1,
                  groups: int = 1, return_macs: bool = False, rows=None):
    """Backward-data of the forward convolution (x_shape, w, stride, padding, dilation, groups),
    float64: dx with shape x_shape from dy with the forward output's shape, or, when ``rows``
    (flat input-position indices) is given, an array (len(rows), C_in).  Arguments as for
    ``conv_fwd``; the definition is in conv_oracle.c (the adjoint of the forward map)."""
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    x_shape = tuple(int(e) for e in x_shape)
    dims = len(x_shape) - 2
    assert dims in (2, 3) and w.ndim == len(x_shape) and dy.ndim == len(x_shape)
    assert w.shape[-1] * groups == x_shape[-1] and dy.shape[-1] == w.shape[0]
    st = _triple(stride, dims)
    dl = _triple(dilation, dims)
    pp = _pads(padding, dims)
    if dims == 2:
        xs5 = (x_shape[0], 1, *x_shape[1:])
        w5 = w.reshape(w.shape[0], 1, *w.shape[1:])
        dy5 = dy.reshape(dy.shape[0], 1, *dy.shape[1:])
        st, dl, pp = (1,) + st, (1,) + dl, ((0, 0),) + pp
    else:
        xs5, w5, dy5 = x_shape, w, dy
    outs = [out_extent_ex(xs5[1 + i], w5.shape[1 + i], st[i], pp[i][0], pp[i][1], dl[i]) for i in range(3)]
    assert tuple(dy5.shape) == (xs5[0], *outs, w5.shape[0]), (dy5.shape, outs)
    sh = _Shape(*xs5, w5.shape[0], w5.shape[1], w5.shape[2], w5.shape[3], *st, *(p[0] for p in pp),
                *(p[1] for p in pp), *dl, groups)
    if rows is None:
        dx = np.zeros(xs5, dtype=np.float64)
        rows_ptr, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        dx = np.zeros((rows.shape[0], xs5[-1]), dtype=np.float64)
        rows_ptr, nrows = rows.ctypes.data, rows.shape[0]
    macs = _load().oracle_conv_bwd_data(ctypes.byref(sh), dy5.ctypes.data, w5.ctypes.data, rows_ptr,
                                        nrows, dx.ctypes.data)
    if macs < 0:
        raise ValueError("oracle rejected the shape or a row index")
    if rows is None:
        dx = dx.reshape(x_shape)
    return (dx, int(macs)) if return_macs else dx


def decode_fp16_bits(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) to float64, from the format's fields: sign bit 15,
    5-bit exponent (bias 15), 10-bit fraction; exponent 0 is the subnormal range
    (fraction * 2^-24), exponent 31 is infinity (fraction 0) or NaN.  Exact: every binary16
    value is a binary64 value."""
    b = bits.astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1024.0 + f, (e - 25).astype(np.int32))   # (1 + f/2^10) * 2^(e-15)
    sub = np.ldexp(f, -24)
    special = np.where(f == 0, np.inf, np.nan)
    return sign * np.where(e == 0, sub, np.where(e == 31, special, normal))


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64: a bfloat16 is the upper half of the binary32
    with the same sign, exponent and leading fraction bits, so the pattern shifted left by 16
    is that binary32, which widens to binary64 exactly."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_float64(t) -> np.ndarray:
    """Exact float64 copy of a CPU or GPU fp16 / bf16 / fp32 tensor (or ndarray).  torch only
    moves the tensor to the host and hands over its raw bits; fp16 and bf16 are decoded from
    those bits here."""
    if isinstance(t, np.ndarray):
        if t.dtype == np.float16:
            return decode_fp16_bits(t.view(np.uint16))
        return t.astype(np.float64)
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        bits = t.view(torch.int16).numpy().view(np.uint16)
        return decode_fp16_bits(bits) if t.dtype == torch.float16 else decode_bf16_bits(bits)
    return t.numpy().astype(np.float64)
