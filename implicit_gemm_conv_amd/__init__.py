"""Python binding of libconvfwd.so, the gfx950 channels-last implicit-GEMM convolution.

Argument marshalling only: every step of the convolution runs in the HIP
kernels behind the C ABI of include/convfwd.h.  PyTorch provides device
memory and the stream.  There is no CPU fallback: if the library is missing
or the tensors are not on a GPU, the call raises.

    import implicit_gemm_conv_amd as igc
    y = igc.conv_fwd(x, w, stride=1, padding=1)        # x (N,[D,]H,W,C), w (Co,[KD,]KH,KW,C)
    dx = igc.conv_bwd_data(dy, w, x.shape, stride=1, padding=1)   # gradient w.r.t. x
"""
import ctypes
import os

import torch

from .build import LIB as _LIB_PATH

PATHS = {"auto": 0, "main": 1, "flatk": 2, "rows": 3, "direct": 4, "brick": 5, "strip": 6, "runs": 7,
         "grouped": 8, "slab": 9, "phase": 10, "staged": 11}
PATH_NAMES = {v: k for k, v in PATHS.items()}
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class ConvError(RuntimeError):
    """A non-zero return code from the C ABI."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"convfwd error {code}: {msg}")
        self.code = code


class Desc(ctypes.Structure):
    """Mirror of convfwd_desc."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "n", "d", "h", "w", "c_in", "c_out", "k_d", "k_h", "k_w",
        "s_d", "s_h", "s_w", "p_d", "p_h", "p_w", "groups", "dtype")]


class DescEx(ctypes.Structure):
    """Mirror of convfwd_desc_ex (low / high padding, dilation, groups)."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "n", "d", "h", "w", "c_in", "c_out", "k_d", "k_h", "k_w",
        "s_d", "s_h", "s_w", "p_d", "p_h", "p_w", "q_d", "q_h", "q_w",
        "e_d", "e_h", "e_w", "groups", "dtype")]


# Every entry point the header declares: (name, restype, argtypes).
EXPORTS = [
    ("conv_out_shape", ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_int64)]),
    ("conv_select_path", ctypes.c_int, [ctypes.POINTER(Desc)]),
    ("conv_fwd", ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p]),
    ("conv_fwd_path", ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("conv_out_shape_ex", ctypes.c_int, [ctypes.POINTER(DescEx), ctypes.POINTER(ctypes.c_int64)]),
    ("conv_select_path_ex", ctypes.c_int, [ctypes.POINTER(DescEx)]),
    ("conv_fwd_ex", ctypes.c_int, [ctypes.POINTER(DescEx), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]),
    ("conv_fwd_path_ex", ctypes.c_int, [ctypes.POINTER(DescEx), ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("conv_bwd_data_filter", ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]),
    ("conv_bwd_data", ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]),
    ("conv_bwd_data_filter_ex", ctypes.c_int, [ctypes.POINTER(DescEx), ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p]),
    ("conv_bwd_data_ex", ctypes.c_int, [ctypes.POINTER(DescEx), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    ("conv_bwd_data_path_ex", ctypes.c_int, [ctypes.POINTER(DescEx), ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("conv_tune", ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]),
    ("conv_tune_ex", ctypes.c_int, [ctypes.POINTER(DescEx), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_float)]),
    ("conv_tuned_path_ex", ctypes.c_int, [ctypes.POINTER(DescEx)]),
    ("conv_tune_clear", ctypes.c_int, []),
    ("conv_strerror", ctypes.c_char_p, [ctypes.c_int]),
    ("conv_path_name", ctypes.c_char_p, [ctypes.c_int]),
]

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m implicit_gemm_conv_amd.build`")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, res, args in EXPORTS:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(code: int) -> int:
    if code < 0:
        raise ConvError(code, lib().conv_strerror(code).decode())
    return code


def _triple(v, dims, what):
    if isinstance(v, int):
        v = (v,) * dims
    v = tuple(int(e) for e in v)
    if len(v) != dims:
        raise ValueError(f"{what} needs {dims} entries, got {v}")
    return v


def _pairs(padding, dims):
    """Per-dimension (low, high) pads from an int, a tuple of ints or a tuple of pairs."""
    if isinstance(padding, int):
        return ((padding, padding),) * dims
    padding = tuple(padding)
    if len(padding) != dims:
        raise ValueError(f"padding needs {dims} entries, got {padding}")
    return tuple((int(q), int(q)) if isinstance(q, int) else (int(q[0]), int(q[1])) for q in padding)


def make_desc_ex(x_shape, w_shape, stride=1, padding=0, dilation=1, groups=1,
                 dtype=torch.float16) -> DescEx:
    """Extended descriptor for x (N,[D,]H,W,C_in) and w (C_out,[KD,]KH,KW,C_in/groups) shapes;
    padding is an int, one int per dimension, or one (low, high) pair per dimension."""
    dims = len(x_shape) - 2
    if dims not in (2, 3) or len(w_shape) != len(x_shape):
        raise ValueError(f"expected 4-D (2D) or 5-D (3D) x and w, got {x_shape}, {w_shape}")
    st = _triple(stride, dims, "stride")
    dl = _triple(dilation, dims, "dilation")
    pp = _pairs(padding, dims)
    if dims == 2:
        x_shape = (x_shape[0], 1, *x_shape[1:])
        w_shape = (w_shape[0], 1, *w_shape[1:])
        st, dl, pp = (1, *st), (1, *dl), ((0, 0), *pp)
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    return DescEx(x_shape[0], x_shape[1], x_shape[2], x_shape[3], x_shape[4], w_shape[0],
                  w_shape[1], w_shape[2], w_shape[3], *st, *(q[0] for q in pp),
                  *(q[1] for q in pp), *dl, groups, _DTYPES[dtype])


def make_desc(x_shape, w_shape, stride=1, padding=0, dtype=torch.float16, groups=1) -> Desc:
    """Descriptor for x (N,[D,]H,W,C_in) and w (C_out,[KD,]KH,KW,C_in) shapes."""
    dims = len(x_shape) - 2
    if dims not in (2, 3) or len(w_shape) != len(x_shape):
        raise ValueError(f"expected 4-D (2D) or 5-D (3D) x and w, got {x_shape}, {w_shape}")
    st = _triple(stride, dims, "stride")
    pd = _triple(padding, dims, "padding")
    if dims == 2:
        x_shape = (x_shape[0], 1, *x_shape[1:])
        w_shape = (w_shape[0], 1, *w_shape[1:])
        st, pd = (1, *st), (0, *pd)
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    return Desc(x_shape[0], x_shape[1], x_shape[2], x_shape[3], x_shape[4], w_shape[0],
                w_shape[1], w_shape[2], w_shape[3], *st, *pd, groups, _DTYPES[dtype])


def out_shape(x_shape, w_shape, stride=1, padding=0, dilation=1, groups=1):
    """Output shape (N,[D_out,]H_out,W_out,C_out) as the library computes it."""
    d = make_desc_ex(x_shape, w_shape, stride, padding, dilation, groups)
    out = (ctypes.c_int64 * 5)()
    _check(lib().conv_out_shape_ex(ctypes.byref(d), out))
    shape = tuple(int(v) for v in out)
    return shape if len(x_shape) == 5 else (shape[0], *shape[2:])


def select_path(x_shape, w_shape, stride=1, padding=0, dtype=torch.float16, dilation=1,
                groups=1) -> str:
    """Name of the path the library picks for this problem."""
    d = make_desc_ex(x_shape, w_shape, stride, padding, dilation, groups, dtype)
    return PATH_NAMES[_check(lib().conv_select_path_ex(ctypes.byref(d)))]


def _check_filter(x_shape, w_shape, groups):
    """w must have x's rank and C_in/groups input channels: the library sizes its reads of w
    from the descriptor, so a filter of another shape would be read out of bounds or with the
    wrong stride."""
    if len(w_shape) != len(x_shape):
        raise ValueError(f"x {tuple(x_shape)} and w {tuple(w_shape)} must have the same rank")
    if groups < 1 or w_shape[-1] * groups != x_shape[-1]:
        raise ValueError(f"w {tuple(w_shape)} must hold C_in/groups = {x_shape[-1]}/{groups} input "
                         f"channels in its last dimension")


def _check_out(out, shape, like, what="out"):
    if tuple(out.shape) != tuple(shape) or out.dtype != like.dtype or not out.is_contiguous() \
            or out.device != like.device:
        raise ValueError(f"{what} must be a contiguous {like.dtype} tensor of shape {tuple(shape)} "
                         f"on {like.device}")


def conv_fwd(x: torch.Tensor, w: torch.Tensor, stride=1, padding=0, out: torch.Tensor = None,
             path: str = "auto", dilation=1, groups: int = 1) -> torch.Tensor:
    """Channels-last convolution forward on the GPU.

    x: (N,H,W,C_in) or (N,D,H,W,C_in); w: (C_out,KH,KW,C_in/groups) or
    (C_out,KD,KH,KW,C_in/groups); same dtype (fp32, fp16 or bf16), same CUDA/HIP
    device.  stride, dilation: int or per dimension; padding: int, per
    dimension, or per dimension (low, high).  Non-contiguous inputs are made
    contiguous first.  Returns y (N,[D_out,]H_out,W_out,C_out) in x's dtype,
    launched on the current stream of x's device (not synchronised).
    """
    if not (x.is_cuda and w.is_cuda):
        raise ValueError("conv_fwd runs on the GPU only: x and w must be device tensors")
    if x.device != w.device or x.dtype != w.dtype:
        raise ValueError("x and w must share device and dtype")
    _check_filter(x.shape, w.shape, groups)
    x = x.contiguous()
    w = w.contiguous()
    d = make_desc_ex(tuple(x.shape), tuple(w.shape), stride, padding, dilation, groups, x.dtype)
    shape = out_shape(tuple(x.shape), tuple(w.shape), stride, padding, dilation, groups)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    else:
        _check_out(out, shape, x)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        _check(lib().conv_fwd_path_ex(ctypes.byref(d), PATHS[path], x.data_ptr(), w.data_ptr(),
                                      out.data_ptr(), stream))
    return out


def tune(x: torch.Tensor, w: torch.Tensor, stride=1, padding=0, dilation=1, groups: int = 1,
         reps: int = 10, out: torch.Tensor = None):
    """Time every path (and main tile configuration) that accepts the problem, record the fastest
    for this shape and its bucket (AUTO uses it from then on), and return (path name, mean
    microseconds per launch).  Synchronises the current stream."""
    if not (x.is_cuda and w.is_cuda) or x.device != w.device or x.dtype != w.dtype:
        raise ValueError("tune needs x and w on one GPU with one dtype")
    _check_filter(x.shape, w.shape, groups)
    x = x.contiguous()
    w = w.contiguous()
    d = make_desc_ex(tuple(x.shape), tuple(w.shape), stride, padding, dilation, groups, x.dtype)
    shape = out_shape(tuple(x.shape), tuple(w.shape), stride, padding, dilation, groups)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    else:
        _check_out(out, shape, x)
    us = ctypes.c_float(0.0)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        path = _check(lib().conv_tune_ex(ctypes.byref(d), x.data_ptr(), w.data_ptr(), out.data_ptr(), stream,
                                         int(reps), ctypes.byref(us)))
    return PATH_NAMES[path], float(us.value)


def tuned_path(x_shape, w_shape, stride=1, padding=0, dtype=torch.float16, dilation=1, groups=1):
    """The recorded path for this problem (exact shape, then its bucket), or None."""
    d = make_desc_ex(x_shape, w_shape, stride, padding, dilation, groups, dtype)
    path = _check(lib().conv_tuned_path_ex(ctypes.byref(d)))
    return PATH_NAMES[path] if path else None


def tune_clear():
    """Forget every recorded choice."""
    _check(lib().conv_tune_clear())


def bwd_data_filter(w: torch.Tensor, x_shape, stride=1, padding=0, dilation=1, groups: int = 1,
                    out: torch.Tensor = None) -> torch.Tensor:
    """The filter of the forward convolution (x_shape, w, ...) rearranged for backward-data
    (per stride phase, taps reversed, channels exchanged); same size and dtype as w.  It
    depends only on w and the problem, so it can be prepared once per filter."""
    if not w.is_cuda:
        raise ValueError("bwd_data_filter runs on the GPU only: w must be a device tensor")
    _check_filter(tuple(x_shape), w.shape, groups)
    w = w.contiguous()
    d = make_desc_ex(tuple(x_shape), tuple(w.shape), stride, padding, dilation, groups, w.dtype)
    if out is None:
        out = torch.empty_like(w)
    else:
        _check_out(out, w.shape, w)
    with torch.cuda.device(w.device):
        stream = torch.cuda.current_stream(w.device).cuda_stream
        _check(lib().conv_bwd_data_filter_ex(ctypes.byref(d), w.data_ptr(), out.data_ptr(), stream))
    return out


def conv_bwd_data(dy: torch.Tensor, w: torch.Tensor, x_shape, stride=1, padding=0, dilation=1,
                  groups: int = 1, out: torch.Tensor = None, path: str = "auto",
                  wt: torch.Tensor = None) -> torch.Tensor:
    """Backward-data of the forward convolution (x_shape, w, stride, padding, dilation, groups):
    dx with shape x_shape from dy with the forward output's shape (the transposed convolution
    of dy).  w is the forward filter (C_out,[KD,]KH,KW,C_in/groups); wt, if given, is its
    rearrangement from ``bwd_data_filter`` (else it is prepared here, a temporary the size of
    w).  path: "auto", "main", "runs" or "direct" for the per-phase kernels.  Launched on the
    current stream of dy's device, not synchronised."""
    if not (dy.is_cuda and w.is_cuda):
        raise ValueError("conv_bwd_data runs on the GPU only: dy and w must be device tensors")
    if dy.device != w.device or dy.dtype != w.dtype:
        raise ValueError("dy and w must share device and dtype")
    x_shape = tuple(int(e) for e in x_shape)
    _check_filter(x_shape, w.shape, groups)
    dy = dy.contiguous()
    y_shape = out_shape(x_shape, tuple(w.shape), stride, padding, dilation, groups)
    if tuple(dy.shape) != y_shape:
        raise ValueError(f"dy must have the forward output shape {y_shape}, got {tuple(dy.shape)}")
    if wt is None:
        wt = bwd_data_filter(w, x_shape, stride, padding, dilation, groups)
    else:
        _check_out(wt, w.shape, w, "wt (the rearranged filter)")
    d = make_desc_ex(x_shape, tuple(w.shape), stride, padding, dilation, groups, dy.dtype)
    if out is None:
        out = torch.empty(x_shape, dtype=dy.dtype, device=dy.device)
    else:
        _check_out(out, x_shape, dy)
    with torch.cuda.device(dy.device):
        stream = torch.cuda.current_stream(dy.device).cuda_stream
        _check(lib().conv_bwd_data_path_ex(ctypes.byref(d), PATHS[path], dy.data_ptr(), wt.data_ptr(),
                                           out.data_ptr(), stream))
    return out


def from_torch_weight(w_oc_first: torch.Tensor) -> torch.Tensor:
    """(C_out, C_in, [KD,] KH, KW) PyTorch-style filter -> (C_out, [KD,] KH, KW, C_in)."""
    perm = (0, *range(2, w_oc_first.dim()), 1)
    return w_oc_first.permute(perm).contiguous()
