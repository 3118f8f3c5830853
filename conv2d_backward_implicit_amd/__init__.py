"""MI355X (gfx950) convolution input-gradient as an implicit GEMM (and the
forward convolution on the same kernels).

Thin Python binding over the C ABI of ``libconv2d_bwd.so`` (declared in
``include/conv2d_bwd.h``).  Every step of the computation runs in the HIP
kernels of that library; this module only marshals arguments (device
pointers of torch tensors, the shape struct, torch's current HIP stream).
If the library has not been built, every call raises -- there is no CPU
fallback.

    import conv2d_backward_implicit_amd as c2b
    gi = c2b.grad_input(grad_out, weight, in_h=56, in_w=56, stride=1,
                        padding_h=1, padding_w=1)          # fp32 path
    gi = c2b.grad_input(..., f16=True)                     # f16-staged path
    y = c2b.forward(x, weight, stride=1, padding_h=1, padding_w=1)
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "Conv2dParams", "Conv2dError", "PlanInfo", "grad_input", "grad_input_into",
    "conv2d_grad_input", "conv2d_grad_input_f16", "check_params",
    "describe_plan", "check_indexing", "check_indexing_variant", "num_variants",
    "variant_is_f16", "variant_uses_column_taps", "variant_is_multi_class",
    "conv2d_grad_input_variant",
    "tune", "planned_variant", "select_variant", "describe_plan_variant",
    "forward", "forward_into", "conv2d_forward", "conv2d_forward_f16",
    "conv2d_forward_variant", "tune_forward", "planned_forward_variant",
    "select_forward_variant",
    "describe_forward_plan", "describe_forward_plan_variant",
    "check_indexing_forward", "check_indexing_forward_variant",
    "grad_weight", "grad_weight_into", "conv2d_grad_weight", "grad_weight_workspace_size",
    "check_indexing_grad_weight", "check_indexing_grad_weight_variant",
    "conv2d_grad_weight_variant", "describe_grad_weight_plan", "GRAD_WEIGHT_VARIANTS",
    "grad_weight_noalloc_into",
    "RmsMatmulParams", "make_rms_params", "rms_norm_matmul", "rms_norm_matmul_into",
    "conv2d_rms_norm_matmul_raw", "check_indexing_rms_norm_matmul",
    "MhaGradVParams", "make_mha_params", "mha_grad_v", "mha_grad_v_into", "mha_grad_v_raw",
    "check_indexing_mha_grad_v",
    "status_string", "library_path", "load_library",
    "make_params", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libconv2d_bwd.so")

# every extern "C" symbol include/conv2d_bwd.h declares
EXPORTED_SYMBOLS = (
    "conv2d_grad_input",
    "conv2d_grad_input_f16",
    "conv2d_check_params",
    "conv2d_status_string",
    "conv2d_describe_plan",
    "conv2d_check_indexing",
    "conv2d_num_variants",
    "conv2d_variant_is_f16",
    "conv2d_variant_uses_column_taps",
    "conv2d_variant_is_multi_class",
    "conv2d_grad_input_variant",
    "conv2d_check_indexing_variant",
    "conv2d_tune",
    "conv2d_planned_variant",
    "conv2d_select_variant",
    "conv2d_describe_plan_variant",
    "conv2d_forward",
    "conv2d_forward_f16",
    "conv2d_forward_variant",
    "conv2d_tune_forward",
    "conv2d_planned_forward_variant",
    "conv2d_select_forward_variant",
    "conv2d_describe_forward_plan",
    "conv2d_describe_forward_plan_variant",
    "conv2d_check_indexing_forward",
    "conv2d_check_indexing_forward_variant",
    "conv2d_grad_weight",
    "conv2d_grad_weight_workspace_size",
    "conv2d_check_indexing_grad_weight",
    "conv2d_grad_weight_variant",
    "conv2d_grad_weight_noalloc",
    "conv2d_grad_weight_variant_workspace_size",
    "conv2d_describe_grad_weight_plan",
    "conv2d_check_indexing_grad_weight_variant",
    # include/rms_norm_matmul.h
    "rms_norm_matmul",
    "rms_norm_matmul_check_indexing",
    # include/mha_grad_v.h
    "mha_grad_v",
    "mha_grad_v_check_indexing",
)

# weight-gradient column layouts: 0 flat tiles, 1..3 tap tiles of 1, 2, 4 taps
GRAD_WEIGHT_VARIANTS = 4

CONV2D_OK = 0
STATUS_NAMES = {
    0: "CONV2D_OK",
    -1: "CONV2D_ERR_NULL_PTR",
    -2: "CONV2D_ERR_BAD_SHAPE",
    -3: "CONV2D_ERR_ALIAS",
    -4: "CONV2D_ERR_OVERFLOW",
    -5: "CONV2D_ERR_UNSUPPORTED",
    -6: "CONV2D_ERR_HIP",
    -7: "CONV2D_ERR_WORKSPACE",
    -8: "CONV2D_ERR_SCRATCH",
}


class Conv2dParams(ctypes.Structure):
    """Mirror of ``conv2d_params`` (12 x uint32, header field order)."""
    _fields_ = [(name, ctypes.c_uint32) for name in (
        "batch", "in_channels", "in_h", "in_w", "out_channels", "kernel_h",
        "kernel_w", "stride", "padding_h", "padding_w", "out_h", "out_w")]

    def as_tuple(self):
        return tuple(getattr(self, f) for f, _ in self._fields_)

    def __repr__(self):
        return "Conv2dParams(%s)" % ", ".join(
            "%s=%d" % (f, getattr(self, f)) for f, _ in self._fields_)


class RmsMatmulParams(ctypes.Structure):
    """Mirror of ``rms_matmul_params`` (m, n, k as uint32, eps as float)."""
    _fields_ = [("m", ctypes.c_uint32), ("n", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("eps", ctypes.c_float)]


class MhaGradVParams(ctypes.Structure):
    """Mirror of ``mha_grad_v_params`` (7 x uint32)."""
    _fields_ = [(n, ctypes.c_uint32) for n in ("q_seq", "kv_seq", "heads", "kv_heads",
                                                "head_dim", "window", "causal")]


class PlanInfo(ctypes.Structure):
    """Mirror of ``conv2d_plan_info``."""
    _fields_ = [(name, ctypes.c_int64) for name in (
        "launches", "tiles", "phases", "zero_phases", "macs", "useful_macs")]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


class Conv2dError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = int(status)
        name = STATUS_NAMES.get(self.status, str(status))
        msg = "%s (%s)" % (name, status_string(self.status))
        super().__init__(msg + (": " + what if what else ""))


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libconv2d_bwd.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                "libconv2d_bwd.so is not built; run "
                "`python -m conv2d_backward_implicit_amd.build` (or "
                "__graft_entry__.build()) first")
        # torch carries its own HIP runtime: load it before this library so
        # that the library's kernels are registered with the runtime torch's
        # streams and allocations belong to (loaded the other way round, every
        # launch on a torch stream fails)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(Conv2dParams)
        for name in ("conv2d_grad_input", "conv2d_grad_input_f16", "conv2d_forward",
                     "conv2d_forward_f16"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, P,
                           ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.conv2d_check_params.argtypes = [P]
        lib.conv2d_check_params.restype = ctypes.c_int
        lib.conv2d_status_string.argtypes = [ctypes.c_int]
        lib.conv2d_status_string.restype = ctypes.c_char_p
        lib.conv2d_describe_plan.argtypes = [P, ctypes.c_int, ctypes.POINTER(PlanInfo)]
        lib.conv2d_describe_plan.restype = ctypes.c_int
        lib.conv2d_describe_plan_variant.argtypes = [P, ctypes.c_int, ctypes.POINTER(PlanInfo)]
        lib.conv2d_describe_plan_variant.restype = ctypes.c_int
        lib.conv2d_check_indexing.argtypes = [P, ctypes.c_int, ctypes.c_char_p,
                                              ctypes.c_size_t]
        lib.conv2d_check_indexing.restype = ctypes.c_int
        lib.conv2d_check_indexing_variant.argtypes = [P, ctypes.c_int, ctypes.c_char_p,
                                                      ctypes.c_size_t]
        lib.conv2d_check_indexing_variant.restype = ctypes.c_int
        lib.conv2d_num_variants.argtypes = []
        lib.conv2d_num_variants.restype = ctypes.c_int
        lib.conv2d_variant_is_f16.argtypes = [ctypes.c_int]
        lib.conv2d_variant_is_f16.restype = ctypes.c_int
        lib.conv2d_variant_uses_column_taps.argtypes = [ctypes.c_int]
        lib.conv2d_variant_uses_column_taps.restype = ctypes.c_int
        lib.conv2d_variant_is_multi_class.argtypes = [ctypes.c_int]
        lib.conv2d_variant_is_multi_class.restype = ctypes.c_int
        lib.conv2d_tune.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, P,
                                    ctypes.c_int, ctypes.c_void_p,
                                    ctypes.POINTER(ctypes.c_int)]
        lib.conv2d_tune.restype = ctypes.c_int
        lib.conv2d_planned_variant.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        lib.conv2d_planned_variant.restype = ctypes.c_int
        lib.conv2d_grad_input_variant.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, P, ctypes.c_int,
                                                  ctypes.c_void_p]
        lib.conv2d_grad_input_variant.restype = ctypes.c_int
        lib.conv2d_forward_variant.argtypes = lib.conv2d_grad_input_variant.argtypes
        lib.conv2d_forward_variant.restype = ctypes.c_int
        lib.conv2d_tune_forward.argtypes = lib.conv2d_tune.argtypes
        lib.conv2d_tune_forward.restype = ctypes.c_int
        lib.conv2d_planned_forward_variant.argtypes = lib.conv2d_planned_variant.argtypes
        lib.conv2d_planned_forward_variant.restype = ctypes.c_int
        for name in ("conv2d_select_variant", "conv2d_select_forward_variant"):
            fn = getattr(lib, name)
            fn.argtypes = [P, ctypes.c_int, ctypes.c_int]
            fn.restype = ctypes.c_int
        lib.conv2d_describe_forward_plan.argtypes = lib.conv2d_describe_plan.argtypes
        lib.conv2d_describe_forward_plan.restype = ctypes.c_int
        lib.conv2d_describe_forward_plan_variant.argtypes = \
            lib.conv2d_describe_plan_variant.argtypes
        lib.conv2d_describe_forward_plan_variant.restype = ctypes.c_int
        lib.conv2d_check_indexing_forward.argtypes = lib.conv2d_check_indexing.argtypes
        lib.conv2d_check_indexing_forward.restype = ctypes.c_int
        lib.conv2d_check_indexing_forward_variant.argtypes = \
            lib.conv2d_check_indexing_variant.argtypes
        lib.conv2d_check_indexing_forward_variant.restype = ctypes.c_int
        lib.conv2d_grad_weight.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           P, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]
        lib.conv2d_grad_weight.restype = ctypes.c_int
        lib.conv2d_grad_weight_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        lib.conv2d_grad_weight_workspace_size.restype = ctypes.c_int
        lib.conv2d_check_indexing_grad_weight.argtypes = [P, ctypes.c_char_p, ctypes.c_size_t]
        lib.conv2d_check_indexing_grad_weight.restype = ctypes.c_int
        lib.conv2d_grad_weight_variant.argtypes = lib.conv2d_grad_weight.argtypes + [ctypes.c_int]
        lib.conv2d_grad_weight_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p, P, ctypes.c_void_p]
        lib.conv2d_grad_weight_noalloc.restype = ctypes.c_int
        lib.conv2d_grad_weight_variant.restype = ctypes.c_int
        lib.conv2d_grad_weight_variant_workspace_size.argtypes = [
            P, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        lib.conv2d_grad_weight_variant_workspace_size.restype = ctypes.c_int
        lib.conv2d_describe_grad_weight_plan.argtypes = [P, ctypes.c_int,
                                                         ctypes.POINTER(ctypes.c_int32),
                                                         ctypes.c_int]
        lib.conv2d_describe_grad_weight_plan.restype = ctypes.c_int
        lib.conv2d_check_indexing_grad_weight_variant.argtypes = [P, ctypes.c_int,
                                                                  ctypes.c_char_p,
                                                                  ctypes.c_size_t]
        lib.conv2d_check_indexing_grad_weight_variant.restype = ctypes.c_int
        R = ctypes.POINTER(RmsMatmulParams)
        lib.rms_norm_matmul.argtypes = [ctypes.c_void_p] * 4 + [R, ctypes.c_void_p]
        lib.rms_norm_matmul.restype = ctypes.c_int
        lib.rms_norm_matmul_check_indexing.argtypes = [R, ctypes.c_char_p, ctypes.c_size_t]
        lib.rms_norm_matmul_check_indexing.restype = ctypes.c_int
        M = ctypes.POINTER(MhaGradVParams)
        lib.mha_grad_v.argtypes = [ctypes.c_void_p] * 5 + [M, ctypes.c_void_p]
        lib.mha_grad_v.restype = ctypes.c_int
        lib.mha_grad_v_check_indexing.argtypes = [M, ctypes.c_char_p, ctypes.c_size_t]
        lib.mha_grad_v_check_indexing.restype = ctypes.c_int
        _lib = lib
        return lib


def make_params(batch, in_channels, in_h, in_w, out_channels, kernel_h, kernel_w,
                stride=1, padding_h=0, padding_w=0, out_h=None, out_w=None):
    """Fill a Conv2dParams; out_h/out_w default to the forward extents
    floor((in + 2*pad - k) / stride) + 1."""
    if out_h is None:
        out_h = (in_h + 2 * padding_h - kernel_h) // stride + 1 if stride else 0
    if out_w is None:
        out_w = (in_w + 2 * padding_w - kernel_w) // stride + 1 if stride else 0
    vals = (batch, in_channels, in_h, in_w, out_channels, kernel_h, kernel_w, stride,
            padding_h, padding_w, out_h, out_w)
    for v in vals:
        if not 0 <= int(v) < 2 ** 32:
            raise Conv2dError(-4, "field out of uint32 range: %r" % (v,))
    return Conv2dParams(*(int(v) for v in vals))


def status_string(status: int) -> str:
    return load_library().conv2d_status_string(int(status)).decode()


def check_params(p: Conv2dParams) -> int:
    """Status of conv2d_check_params (pure host code, no device needed)."""
    return int(load_library().conv2d_check_params(ctypes.byref(p)))


def describe_plan(p: Conv2dParams, f16: bool = False) -> dict:
    """Launch plan of a shape (pure host code).  Raises on a bad shape."""
    info = PlanInfo()
    rc = load_library().conv2d_describe_plan(ctypes.byref(p), int(bool(f16)),
                                             ctypes.byref(info))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return info.as_dict()


def describe_plan_variant(p: Conv2dParams, variant: int) -> dict:
    """Launch plan with the kernel variant forced (pure host code)."""
    info = PlanInfo()
    rc = load_library().conv2d_describe_plan_variant(ctypes.byref(p), int(variant),
                                                     ctypes.byref(info))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return info.as_dict()


def check_indexing(p: Conv2dParams, f16: bool = False) -> tuple:
    """Host replay of the kernels' addressing for a shape (no device needed).
    Returns (status, message); status 0 means every check passed."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().conv2d_check_indexing(ctypes.byref(p), int(bool(f16)), buf,
                                              len(buf))
    return int(rc), buf.value.decode()


def check_indexing_variant(p: Conv2dParams, variant: int) -> tuple:
    """check_indexing with the kernel variant forced (host only)."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().conv2d_check_indexing_variant(ctypes.byref(p), int(variant), buf,
                                                      len(buf))
    return int(rc), buf.value.decode()


def num_variants() -> int:
    return int(load_library().conv2d_num_variants())


def variant_is_f16(variant: int) -> int:
    """1 (f16-staged), 0 (fp32) or a negative status for a bad index."""
    return int(load_library().conv2d_variant_is_f16(int(variant)))


def variant_uses_column_taps(variant: int) -> int:
    """1 (column taps in the matrix rows), 0, or a negative status."""
    return int(load_library().conv2d_variant_uses_column_taps(int(variant)))


def variant_is_multi_class(variant: int) -> int:
    """1 (all four classes of a stride-2 shape per tile), 0, or a negative
    status."""
    return int(load_library().conv2d_variant_is_multi_class(int(variant)))


def conv2d_grad_input(grad_out_ptr: int, weight_ptr: int, grad_input_ptr: int,
                      p: Conv2dParams, stream: int = 0) -> int:
    """Raw C-ABI call with integer device pointers; returns the status."""
    return int(load_library().conv2d_grad_input(
        ctypes.c_void_p(grad_out_ptr), ctypes.c_void_p(weight_ptr),
        ctypes.c_void_p(grad_input_ptr), ctypes.byref(p), ctypes.c_void_p(stream)))


def conv2d_grad_input_f16(grad_out_ptr: int, weight_ptr: int, grad_input_ptr: int,
                          p: Conv2dParams, stream: int = 0) -> int:
    """Raw C-ABI call of the f16-staged path; returns the status."""
    return int(load_library().conv2d_grad_input_f16(
        ctypes.c_void_p(grad_out_ptr), ctypes.c_void_p(weight_ptr),
        ctypes.c_void_p(grad_input_ptr), ctypes.byref(p), ctypes.c_void_p(stream)))


def conv2d_grad_input_variant(grad_out_ptr: int, weight_ptr: int, grad_input_ptr: int,
                              p: Conv2dParams, variant: int, stream: int = 0) -> int:
    """Raw C-ABI call with the kernel variant forced; returns the status."""
    return int(load_library().conv2d_grad_input_variant(
        ctypes.c_void_p(grad_out_ptr), ctypes.c_void_p(weight_ptr),
        ctypes.c_void_p(grad_input_ptr), ctypes.byref(p), ctypes.c_int(int(variant)),
        ctypes.c_void_p(stream)))


def _stream_id(stream) -> int:
    """HIP stream handle for a call: that of ``stream`` (a torch.cuda.Stream),
    or of torch's current stream on the current device, read as a raw handle
    without building a Stream object (a few microseconds less per call)."""
    import torch
    if stream is not None:
        return int(stream.cuda_stream)
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(torch.cuda.current_device()))
    return int(torch.cuda.current_stream().cuda_stream)


def _check_tensor(t, name, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))


def grad_input_into(grad_input, grad_out, weight, p: Conv2dParams, f16=False,
                    stream=None, variant=None):
    """Write the input gradient into ``grad_input`` on torch's current stream
    (or ``stream``, a torch.cuda.Stream).  ``variant`` forces a kernel
    variant (its path overrides ``f16``).  Raises Conv2dError on a bad
    status."""
    import torch
    _check_tensor(grad_out, "grad_out", (p.batch, p.out_channels, p.out_h, p.out_w))
    _check_tensor(weight, "weight", (p.out_channels, p.in_channels, p.kernel_h,
                                     p.kernel_w))
    _check_tensor(grad_input, "grad_input", (p.batch, p.in_channels, p.in_h, p.in_w))
    if not (grad_out.device == weight.device == grad_input.device):
        raise ValueError("all tensors must be on the same device")
    with torch.cuda.device(grad_input.device):
        sid = _stream_id(stream)
        if variant is not None:
            rc = conv2d_grad_input_variant(grad_out.data_ptr(), weight.data_ptr(),
                                           grad_input.data_ptr(), p, variant,
                                           sid)
        else:
            fn = conv2d_grad_input_f16 if f16 else conv2d_grad_input
            rc = fn(grad_out.data_ptr(), weight.data_ptr(), grad_input.data_ptr(), p,
                    sid)
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return grad_input


def tune(grad_input, grad_out, weight, p: Conv2dParams, f16=False, stream=None) -> int:
    """conv2d_tune on torch tensors (checked like grad_input_into): times the
    candidate variants of the path on these buffers and makes the fastest the
    shape's default plan; blocks until done; returns the chosen variant."""
    import torch
    _check_tensor(grad_out, "grad_out", (p.batch, p.out_channels, p.out_h, p.out_w))
    _check_tensor(weight, "weight", (p.out_channels, p.in_channels, p.kernel_h,
                                     p.kernel_w))
    _check_tensor(grad_input, "grad_input", (p.batch, p.in_channels, p.in_h, p.in_w))
    if not (grad_out.device == weight.device == grad_input.device):
        raise ValueError("all tensors must be on the same device")
    chosen = ctypes.c_int(-1)
    with torch.cuda.device(grad_input.device):
        sid = _stream_id(stream)
        rc = int(load_library().conv2d_tune(
            ctypes.c_void_p(grad_out.data_ptr()), ctypes.c_void_p(weight.data_ptr()),
            ctypes.c_void_p(grad_input.data_ptr()), ctypes.byref(p), int(bool(f16)),
            ctypes.c_void_p(sid), ctypes.byref(chosen)))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return int(chosen.value)


def planned_variant(p: Conv2dParams, f16: bool = False) -> int:
    """Variant the default entry point uses for this shape now (-1: nothing
    to launch); raises on an invalid shape."""
    v = ctypes.c_int(-1)
    rc = int(load_library().conv2d_planned_variant(ctypes.byref(p), int(bool(f16)),
                                                   ctypes.byref(v)))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return int(v.value)


def select_variant(p: Conv2dParams, f16: bool = False, variant: int = -1) -> None:
    """conv2d_select_variant: make ``variant`` (-1: the model's choice) the
    default entry point's variant for this shape; raises on a bad status."""
    rc = int(load_library().conv2d_select_variant(ctypes.byref(p), int(bool(f16)),
                                                  int(variant)))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)


def grad_input(grad_out, weight, in_h, in_w, stride=1, padding_h=0, padding_w=0,
               f16=False, out=None, stream=None):
    """Input gradient of conv2d for NCHW ``grad_out`` and [Co, Ci, kH, kW]
    ``weight`` (float32 GPU tensors).  Returns a new [N, Ci, in_h, in_w]
    tensor (or fills ``out``)."""
    import torch
    n, co, oh, ow = (int(v) for v in grad_out.shape)
    co2, ci, kh, kw = (int(v) for v in weight.shape)
    if co2 != co:
        raise ValueError("grad_out has %d channels, weight has %d" % (co, co2))
    p = make_params(n, ci, in_h, in_w, co, kh, kw, stride, padding_h, padding_w,
                    oh, ow)
    if out is None:
        out = torch.empty((n, ci, in_h, in_w), dtype=torch.float32,
                          device=grad_out.device)
    return grad_input_into(out, grad_out, weight, p, f16=f16, stream=stream)


# ---- forward convolution (the adjoint operator, on the same kernels) -------

def describe_forward_plan(p: Conv2dParams, f16: bool = False) -> dict:
    """Launch plan of the forward convolution of a shape (pure host code)."""
    info = PlanInfo()
    rc = load_library().conv2d_describe_forward_plan(ctypes.byref(p), int(bool(f16)),
                                                     ctypes.byref(info))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return info.as_dict()


def describe_forward_plan_variant(p: Conv2dParams, variant: int) -> dict:
    """Forward launch plan with the kernel variant forced (pure host code)."""
    info = PlanInfo()
    rc = load_library().conv2d_describe_forward_plan_variant(ctypes.byref(p), int(variant),
                                                             ctypes.byref(info))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return info.as_dict()


def check_indexing_forward(p: Conv2dParams, f16: bool = False) -> tuple:
    """Host replay of the forward launches' addressing (no device needed)."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().conv2d_check_indexing_forward(ctypes.byref(p), int(bool(f16)), buf,
                                                      len(buf))
    return int(rc), buf.value.decode()


def check_indexing_forward_variant(p: Conv2dParams, variant: int) -> tuple:
    """check_indexing_forward with the kernel variant forced (host only)."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().conv2d_check_indexing_forward_variant(ctypes.byref(p), int(variant),
                                                              buf, len(buf))
    return int(rc), buf.value.decode()


def conv2d_forward(x_ptr: int, weight_ptr: int, y_ptr: int, p: Conv2dParams,
                   stream: int = 0) -> int:
    """Raw C-ABI call of the forward convolution; returns the status."""
    return int(load_library().conv2d_forward(
        ctypes.c_void_p(x_ptr), ctypes.c_void_p(weight_ptr), ctypes.c_void_p(y_ptr),
        ctypes.byref(p), ctypes.c_void_p(stream)))


def conv2d_forward_f16(x_ptr: int, weight_ptr: int, y_ptr: int, p: Conv2dParams,
                       stream: int = 0) -> int:
    """Raw C-ABI call of the f16-staged forward convolution."""
    return int(load_library().conv2d_forward_f16(
        ctypes.c_void_p(x_ptr), ctypes.c_void_p(weight_ptr), ctypes.c_void_p(y_ptr),
        ctypes.byref(p), ctypes.c_void_p(stream)))


def conv2d_forward_variant(x_ptr: int, weight_ptr: int, y_ptr: int, p: Conv2dParams,
                           variant: int, stream: int = 0) -> int:
    """Raw C-ABI forward call with the kernel variant forced."""
    return int(load_library().conv2d_forward_variant(
        ctypes.c_void_p(x_ptr), ctypes.c_void_p(weight_ptr), ctypes.c_void_p(y_ptr),
        ctypes.byref(p), ctypes.c_int(int(variant)), ctypes.c_void_p(stream)))


def _check_forward_tensors(y, x, weight, p):
    _check_tensor(x, "x", (p.batch, p.in_channels, p.in_h, p.in_w))
    _check_tensor(weight, "weight", (p.out_channels, p.in_channels, p.kernel_h,
                                     p.kernel_w))
    _check_tensor(y, "y", (p.batch, p.out_channels, p.out_h, p.out_w))
    if not (x.device == weight.device == y.device):
        raise ValueError("all tensors must be on the same device")


def forward_into(y, x, weight, p: Conv2dParams, f16=False, stream=None, variant=None):
    """Write the forward convolution of ``x`` with ``weight`` into ``y`` on
    torch's current stream (or ``stream``); ``variant`` forces a kernel
    variant.  Raises Conv2dError on a bad status."""
    import torch
    _check_forward_tensors(y, x, weight, p)
    with torch.cuda.device(y.device):
        sid = _stream_id(stream)
        if variant is not None:
            rc = conv2d_forward_variant(x.data_ptr(), weight.data_ptr(), y.data_ptr(), p,
                                        variant, sid)
        else:
            fn = conv2d_forward_f16 if f16 else conv2d_forward
            rc = fn(x.data_ptr(), weight.data_ptr(), y.data_ptr(), p, sid)
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return y


def tune_forward(y, x, weight, p: Conv2dParams, f16=False, stream=None) -> int:
    """conv2d_tune_forward on torch tensors: the measured variant choice of
    the forward convolution for this shape; returns the chosen variant."""
    import torch
    _check_forward_tensors(y, x, weight, p)
    chosen = ctypes.c_int(-1)
    with torch.cuda.device(y.device):
        sid = _stream_id(stream)
        rc = int(load_library().conv2d_tune_forward(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(weight.data_ptr()),
            ctypes.c_void_p(y.data_ptr()), ctypes.byref(p), int(bool(f16)),
            ctypes.c_void_p(sid), ctypes.byref(chosen)))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return int(chosen.value)


def planned_forward_variant(p: Conv2dParams, f16: bool = False) -> int:
    """Variant the default forward entry point uses for this shape now."""
    v = ctypes.c_int(-1)
    rc = int(load_library().conv2d_planned_forward_variant(ctypes.byref(p), int(bool(f16)),
                                                           ctypes.byref(v)))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return int(v.value)


def select_forward_variant(p: Conv2dParams, f16: bool = False, variant: int = -1) -> None:
    """conv2d_select_forward_variant; raises on a bad status."""
    rc = int(load_library().conv2d_select_forward_variant(ctypes.byref(p), int(bool(f16)),
                                                          int(variant)))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)


def forward(x, weight, stride=1, padding_h=0, padding_w=0, f16=False, out=None, stream=None):
    """Forward conv2d of NCHW ``x`` with [Co, Ci, kH, kW] ``weight`` (float32
    GPU tensors, no bias).  Returns a new [N, Co, out_h, out_w] tensor (or
    fills ``out``)."""
    import torch
    n, ci, h, w_ = (int(v) for v in x.shape)
    co, ci2, kh, kw = (int(v) for v in weight.shape)
    if ci2 != ci:
        raise ValueError("x has %d channels, weight has %d" % (ci, ci2))
    p = make_params(n, ci, h, w_, co, kh, kw, stride, padding_h, padding_w)
    if out is None:
        out = torch.empty((n, co, p.out_h, p.out_w), dtype=torch.float32, device=x.device)
    return forward_into(out, x, weight, p, f16=f16, stream=stream)


# ---- weight gradient -----------------------------------------------------------

def grad_weight_workspace_size(p: Conv2dParams, variant: int = -1) -> int:
    """Workspace bytes conv2d_grad_weight (or, for variant >= 0,
    conv2d_grad_weight_variant) needs for this shape on the current device."""
    n = ctypes.c_size_t(0)
    lib = load_library()
    if variant < 0:
        rc = lib.conv2d_grad_weight_workspace_size(ctypes.byref(p), ctypes.byref(n))
    else:
        rc = lib.conv2d_grad_weight_variant_workspace_size(ctypes.byref(p), int(variant),
                                                           ctypes.byref(n))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return int(n.value)


def describe_grad_weight_plan(p: Conv2dParams, variant: int = -1) -> dict:
    """The weight-gradient plan (pure host code): column layout variant,
    channels and taps of a tap tile, tile counts and the pixel split."""
    info = (ctypes.c_int32 * 7)()
    rc = load_library().conv2d_describe_grad_weight_plan(ctypes.byref(p), int(variant), info, 7)
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    keys = ("variant", "tile_channels", "tile_taps", "co_tiles", "column_tiles", "chunks",
            "chunk_pixels")
    return dict(zip(keys, (int(v) for v in info)))


def check_indexing_grad_weight(p: Conv2dParams) -> tuple:
    """Host replay of the weight-gradient kernels (no device needed)."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().conv2d_check_indexing_grad_weight(ctypes.byref(p), buf, len(buf))
    return int(rc), buf.value.decode()


def check_indexing_grad_weight_variant(p: Conv2dParams, variant: int) -> tuple:
    """Host replay of the weight-gradient kernels for a forced variant."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().conv2d_check_indexing_grad_weight_variant(ctypes.byref(p), int(variant),
                                                                  buf, len(buf))
    return int(rc), buf.value.decode()


def conv2d_grad_weight(grad_out_ptr: int, x_ptr: int, grad_weight_ptr: int, p: Conv2dParams,
                       workspace_ptr: int, workspace_bytes: int, stream: int = 0) -> int:
    """Raw C-ABI call of the weight gradient; returns the status."""
    return int(load_library().conv2d_grad_weight(
        ctypes.c_void_p(grad_out_ptr), ctypes.c_void_p(x_ptr), ctypes.c_void_p(grad_weight_ptr),
        ctypes.byref(p), ctypes.c_void_p(workspace_ptr), ctypes.c_size_t(int(workspace_bytes)),
        ctypes.c_void_p(stream)))


def conv2d_grad_weight_variant(grad_out_ptr: int, x_ptr: int, grad_weight_ptr: int,
                               p: Conv2dParams, workspace_ptr: int, workspace_bytes: int,
                               stream: int, variant: int) -> int:
    """Raw C-ABI call of the weight gradient with a forced column layout."""
    return int(load_library().conv2d_grad_weight_variant(
        ctypes.c_void_p(grad_out_ptr), ctypes.c_void_p(x_ptr), ctypes.c_void_p(grad_weight_ptr),
        ctypes.byref(p), ctypes.c_void_p(workspace_ptr), ctypes.c_size_t(int(workspace_bytes)),
        ctypes.c_void_p(stream), int(variant)))


def grad_weight_into(grad_weight, grad_out, x, p: Conv2dParams, workspace=None, stream=None,
                     variant: int = -1):
    """Write the weight gradient into ``grad_weight`` on torch's current
    stream (or ``stream``).  ``workspace`` (a uint8 GPU tensor of at least
    grad_weight_workspace_size bytes) is allocated here by torch if not given.
    ``variant`` >= 0 forces a column layout (tests).  Raises Conv2dError on a
    bad status."""
    import torch
    _check_tensor(grad_out, "grad_out", (p.batch, p.out_channels, p.out_h, p.out_w))
    _check_tensor(x, "x", (p.batch, p.in_channels, p.in_h, p.in_w))
    _check_tensor(grad_weight, "grad_weight", (p.out_channels, p.in_channels, p.kernel_h,
                                               p.kernel_w))
    if not (grad_out.device == x.device == grad_weight.device):
        raise ValueError("all tensors must be on the same device")
    with torch.cuda.device(grad_weight.device):
        need = grad_weight_workspace_size(p, variant)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=grad_weight.device)
        sid = _stream_id(stream)
        args = (grad_out.data_ptr(), x.data_ptr(), grad_weight.data_ptr(), p,
                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                sid)
        rc = (conv2d_grad_weight(*args) if variant < 0 else
              conv2d_grad_weight_variant(*args, variant))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return grad_weight


def grad_weight_noalloc_into(grad_weight, grad_out, x, p: Conv2dParams, stream=None):
    """conv2d_grad_weight_noalloc: the weight gradient into ``grad_weight``
    with the library's own scratch instead of a workspace (nothing is
    allocated); raises Conv2dError on a bad status."""
    import torch
    _check_tensor(grad_out, "grad_out", (p.batch, p.out_channels, p.out_h, p.out_w))
    _check_tensor(x, "x", (p.batch, p.in_channels, p.in_h, p.in_w))
    _check_tensor(grad_weight, "grad_weight", (p.out_channels, p.in_channels, p.kernel_h,
                                               p.kernel_w))
    if not (grad_out.device == x.device == grad_weight.device):
        raise ValueError("all tensors must be on the same device")
    with torch.cuda.device(grad_weight.device):
        sid = _stream_id(stream)
        rc = int(load_library().conv2d_grad_weight_noalloc(
            ctypes.c_void_p(grad_out.data_ptr()), ctypes.c_void_p(x.data_ptr()),
            ctypes.c_void_p(grad_weight.data_ptr()), ctypes.byref(p),
            ctypes.c_void_p(sid)))
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return grad_weight


def grad_weight(grad_out, x, kernel_h, kernel_w, stride=1, padding_h=0, padding_w=0,
                out=None, stream=None):
    """Weight gradient [Co, Ci, kernel_h, kernel_w] of conv2d for NCHW
    ``grad_out`` and ``x`` (float32 GPU tensors)."""
    import torch
    n, co, oh, ow = (int(v) for v in grad_out.shape)
    n2, ci, h, w_ = (int(v) for v in x.shape)
    if n2 != n:
        raise ValueError("grad_out has batch %d, x has %d" % (n, n2))
    p = make_params(n, ci, h, w_, co, kernel_h, kernel_w, stride, padding_h, padding_w, oh, ow)
    if out is None:
        out = torch.empty((co, ci, kernel_h, kernel_w), dtype=torch.float32, device=x.device)
    return grad_weight_into(out, grad_out, x, p, stream=stream)


# ---- RMSNorm-fused matrix product ------------------------------------------------

def make_rms_params(m, n, k, eps=1e-6) -> RmsMatmulParams:
    return RmsMatmulParams(int(m), int(n), int(k), float(eps))


def check_indexing_rms_norm_matmul(p: RmsMatmulParams) -> tuple:
    """Host replay of the RMSNorm-fused product kernel (no device needed)."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().rms_norm_matmul_check_indexing(ctypes.byref(p), buf, len(buf))
    return int(rc), buf.value.decode()


def conv2d_rms_norm_matmul_raw(x_ptr: int, g_ptr: int, w_ptr: int, out_ptr: int,
                               p: RmsMatmulParams, stream: int = 0) -> int:
    """Raw C-ABI call of rms_norm_matmul; returns the status."""
    return int(load_library().rms_norm_matmul(
        ctypes.c_void_p(x_ptr), ctypes.c_void_p(g_ptr), ctypes.c_void_p(w_ptr),
        ctypes.c_void_p(out_ptr), ctypes.byref(p), ctypes.c_void_p(stream)))


def rms_norm_matmul_into(out, x, g, w, eps=1e-6, stream=None):
    """out [m, n] = RmsNorm(x [m, k], g [k], eps) @ w [k, n] on torch's current
    stream (or ``stream``); float32 GPU tensors.  Raises Conv2dError on a bad
    status."""
    import torch
    m, k = (int(v) for v in x.shape)
    n = int(w.shape[1])
    _check_tensor(x, "x", (m, k))
    _check_tensor(g, "norm_weight", (k,))
    _check_tensor(w, "proj", (k, n))
    _check_tensor(out, "out", (m, n))
    if not (x.device == g.device == w.device == out.device):
        raise ValueError("all tensors must be on the same device")
    p = make_rms_params(m, n, k, eps)
    with torch.cuda.device(out.device):
        sid = _stream_id(stream)
        rc = conv2d_rms_norm_matmul_raw(x.data_ptr(), g.data_ptr(), w.data_ptr(),
                                        out.data_ptr(), p, sid)
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return out


def rms_norm_matmul(x, g, w, eps=1e-6, stream=None):
    """RmsNorm(x, g, eps) @ w as a new float32 tensor [m, n]."""
    import torch
    out = torch.empty((int(x.shape[0]), int(w.shape[1])), dtype=torch.float32, device=x.device)
    return rms_norm_matmul_into(out, x, g, w, eps, stream)


# ---- attention dV ---------------------------------------------------------------

def make_mha_params(q_seq, kv_seq, heads, kv_heads, head_dim=64, window=0,
                    causal=True) -> MhaGradVParams:
    return MhaGradVParams(int(q_seq), int(kv_seq), int(heads), int(kv_heads), int(head_dim),
                          int(window), int(bool(causal)))


def check_indexing_mha_grad_v(p: MhaGradVParams) -> tuple:
    """Host replay of the attention-dV launch (no device needed)."""
    buf = ctypes.create_string_buffer(512)
    rc = load_library().mha_grad_v_check_indexing(ctypes.byref(p), buf, len(buf))
    return int(rc), buf.value.decode()


def mha_grad_v_raw(dout_ptr: int, q_ptr: int, k_ptr: int, lse_ptr: int, dv_ptr: int,
                   p: MhaGradVParams, stream: int = 0) -> int:
    """Raw C-ABI call of mha_grad_v; returns the status."""
    return int(load_library().mha_grad_v(
        ctypes.c_void_p(dout_ptr), ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr),
        ctypes.c_void_p(lse_ptr), ctypes.c_void_p(dv_ptr), ctypes.byref(p),
        ctypes.c_void_p(stream)))


def mha_grad_v_into(dv, dout, q, k, lse, window=0, causal=True, stream=None):
    """dV [kv_seq, kv_heads, 64] of attention into ``dv`` on torch's current
    stream (or ``stream``); float32 GPU tensors dout, q [q_seq, heads, 64],
    k [kv_seq, kv_heads, 64], lse [q_seq, heads, 2] (row max, log sum).
    Raises Conv2dError on a bad status."""
    import torch
    q_seq, heads, d = (int(v) for v in q.shape)
    kv_seq, kv_heads = int(k.shape[0]), int(k.shape[1])
    _check_tensor(dout, "dout", (q_seq, heads, d))
    _check_tensor(q, "q", (q_seq, heads, d))
    _check_tensor(k, "k", (kv_seq, kv_heads, d))
    _check_tensor(lse, "lse", (q_seq, heads, 2))
    _check_tensor(dv, "dv", (kv_seq, kv_heads, d))
    p = make_mha_params(q_seq, kv_seq, heads, kv_heads, d, window, causal)
    with torch.cuda.device(dv.device):
        sid = _stream_id(stream)
        rc = mha_grad_v_raw(dout.data_ptr(), q.data_ptr(), k.data_ptr(), lse.data_ptr(),
                            dv.data_ptr(), p, sid)
    if rc != CONV2D_OK:
        raise Conv2dError(rc)
    return dv


def mha_grad_v(dout, q, k, lse, window=0, causal=True, stream=None):
    """dV as a new float32 tensor [kv_seq, kv_heads, 64]."""
    import torch
    dv = torch.empty(tuple(k.shape), dtype=torch.float32, device=k.device)
    return mha_grad_v_into(dv, dout, q, k, lse, window, causal, stream)
