"""Python binding of libaarms.so: fused residual-add + RMSNorm, SwiGLU and
their FP8 (E4M3) epilogues on MI355X (gfx950).

Argument marshalling only.  Every step of every op runs in the HIP kernels of
libaarms.so (see include/aarms.h for the arithmetic, layouts and errors);
PyTorch supplies device memory and the current stream.  There is no CPU or
PyTorch fallback: if the library cannot be loaded or built, every call raises.

bf16 tensors are ``torch.bfloat16``; FP8 tensors are ``torch.float8_e4m3fn``
(OCP E4M3FN) or ``torch.uint8`` holding the same codes.
"""

from __future__ import annotations

import ctypes as C
import os
import threading

import torch

__all__ = [
    "AarmsError", "load", "lib_path",
    "fused_add_rmsnorm", "fused_add_rmsnorm_quant_fp8", "fused_add_rmsnorm_quant_fp8_static",
    "rmsnorm", "rmsnorm_quant_fp8", "rmsnorm_quant_fp8_static",
    "fused_add_rmsnorm_quant_mxfp4", "rmsnorm_quant_mxfp4",
    "fused_add_rmsnorm_quant_nvfp4", "rmsnorm_quant_nvfp4", "swiglu_quant_nvfp4",
    "swiglu", "swiglu_quant_fp8", "swiglu_quant_fp8_dynamic", "swiglu_quant_mxfp4",
    "variant_count", "variant_name", "variant_fits", "pick_variant",
    "OP_NORM", "OP_SWIGLU", "OP_SWIGLU_DYNAMIC", "OP_RMSNORM",
]

# Variants installed by tuning.tune() / tuning.load(), keyed by (form, width,
# token bucket); consulted by the entry points below when variant == -1.
_TUNED: dict = {}


def _variant(form: str, tokens: int, width: int, variant: int) -> int:
    if variant != -1 or not _TUNED:
        return variant
    t = max(1, int(tokens))
    return _TUNED.get((form, int(width), 1 << (t - 1).bit_length()), -1)


_HERE = os.path.dirname(os.path.abspath(__file__))
# AARMS_LIB names another build of the same library (the host-sanitizer test
# loads one whose C entry points are built with AddressSanitizer and UBSan).
_LIB_PATH = os.environ.get("AARMS_LIB") or os.path.join(_HERE, "libaarms.so")
_LOCK = threading.Lock()
_LIB = None

OP_NORM = 0
OP_SWIGLU = 1
OP_SWIGLU_DYNAMIC = 2
OP_RMSNORM = 3
FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


class AarmsError(RuntimeError):
    """A libaarms entry point returned an error code."""

    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, _status_string(status), status))
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libaarms.so, building it with hipcc first if it is not there."""
    global _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        if not os.path.exists(_LIB_PATH):
            from . import _build
            _build.build()
        lib = C.CDLL(_LIB_PATH)
        vp, i64, f32, i32 = C.c_void_p, C.c_int64, C.c_float, C.c_int
        sigs = {
            "fused_add_rmsnorm": [vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "fused_add_rmsnorm_ex": [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "fused_add_rmsnorm_quant_fp8": [vp, vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "fused_add_rmsnorm_quant_fp8_ex": [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "swiglu": [vp, vp, i64, i64, vp],
            "swiglu_ex": [vp, vp, i64, i64, i32, vp],
            "swiglu_quant_fp8": [vp, vp, vp, i64, i64, vp],
            "swiglu_quant_fp8_ex": [vp, vp, vp, i64, i64, i32, vp],
            "fused_add_rmsnorm_quant_fp8_static": [vp, vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "fused_add_rmsnorm_quant_fp8_static_ex": [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm": [vp, vp, vp, i64, i64, f32, vp],
            "rmsnorm_quant_fp8": [vp, vp, vp, vp, i64, i64, f32, vp],
            "rmsnorm_quant_fp8_static": [vp, vp, vp, vp, i64, i64, f32, vp],
            "swiglu_quant_fp8_dynamic": [vp, vp, vp, i64, i64, vp],
            "swiglu_quant_nvfp4": [vp, vp, vp, vp, i64, i64, vp],
            "swiglu_quant_nvfp4_ex": [vp, vp, vp, vp, i64, i64, i32, vp],
            "fused_add_rmsnorm_quant_nvfp4": [vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "fused_add_rmsnorm_quant_nvfp4_ex": [vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm_quant_nvfp4": [vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "rmsnorm_quant_nvfp4_ex": [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "swiglu_quant_mxfp4": [vp, vp, vp, i64, i64, vp],
            "swiglu_quant_mxfp4_ex": [vp, vp, vp, i64, i64, i32, vp],
            "fused_add_rmsnorm_quant_mxfp4": [vp, vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "fused_add_rmsnorm_quant_mxfp4_ex": [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm_quant_mxfp4": [vp, vp, vp, vp, i64, i64, f32, vp],
            "rmsnorm_quant_mxfp4_ex": [vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm_ex": [vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm_quant_fp8_ex": [vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm_quant_fp8_static_ex": [vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "swiglu_quant_fp8_dynamic_ex": [vp, vp, vp, i64, i64, i32, vp],
            "fused_add_rmsnorm_quant_fp8_group": [vp, vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "fused_add_rmsnorm_quant_fp8_group_ex": [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm_quant_fp8_group": [vp, vp, vp, vp, i64, i64, f32, vp],
            "rmsnorm_quant_fp8_group_ex": [vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "swiglu_quant_fp8_group": [vp, vp, vp, i64, i64, vp],
            "swiglu_quant_fp8_group_ex": [vp, vp, vp, i64, i64, i32, vp],
            "aarms_variant_count": [i32],
            "aarms_pick_variant": [i32, i64, i64, i32],
            "aarms_variant_fits": [i32, i32, i64],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = C.c_int
        lib.aarms_status_string.argtypes = [C.c_int]
        lib.aarms_status_string.restype = C.c_char_p
        lib.aarms_variant_name.argtypes = [C.c_int, C.c_int]
        lib.aarms_variant_name.restype = C.c_char_p
        _LIB = lib
        return lib


def _status_string(status: int) -> str:
    s = load().aarms_status_string(int(status))
    return s.decode() if s else "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise AarmsError(status, what)


def _require(t: torch.Tensor, name: str, dtypes, shape) -> None:
    # the common case in one expression (a few attribute reads); the checks
    # below name what is wrong
    if isinstance(t, torch.Tensor) and t.is_cuda and t.dtype in dtypes and t.shape == shape and t.is_contiguous():
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU (got %s); there is no CPU path" % (name, t.device))
    if t.dtype not in dtypes:
        raise TypeError("%s must have dtype %s, got %s" % (name, " or ".join(map(str, dtypes)), t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# The current stream's raw handle without building a torch.cuda.Stream per
# call (the same handle torch.cuda.current_stream(i).cuda_stream gives).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: int) -> int:
    """hipStream_t of the current stream on GPU `device` (an index)."""
    if _raw_stream is not None:
        return _raw_stream(device)
    return torch.cuda.current_stream(device).cuda_stream


def _same_device(*ts: torch.Tensor) -> None:
    d = ts[0].get_device()
    for t in ts[1:]:
        if t.get_device() != d:
            raise ValueError("all tensors must be on the same device")


def fused_add_rmsnorm(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor, eps: float,
                      out: torch.Tensor | None = None, residual_out: torch.Tensor | None = None,
                      variant: int = -1):
    """Residual add + RMSNorm in one kernel.  Returns (out, residual_out).

    x, residual: bf16 [T, H]; weight: bf16 [H].  out=x and/or
    residual_out=residual run in place."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(residual, "residual", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    if out is None:
        out = torch.empty_like(x)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _require(out, "out", (torch.bfloat16,), (T, H))
    _require(residual_out, "residual_out", (torch.bfloat16,), (T, H))
    _same_device(x, residual, weight, out, residual_out)
    lib = load()
    variant = _variant("fused_add_rmsnorm", T, H, variant)
    _check(lib.fused_add_rmsnorm_ex(out.data_ptr(), residual_out.data_ptr(), x.data_ptr(),
                                    residual.data_ptr(), weight.data_ptr(), T, H, float(eps),
                                    int(variant), _stream(x.get_device())), "fused_add_rmsnorm")
    return out, residual_out


def fused_add_rmsnorm_quant_fp8(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor,
                                eps: float, out: torch.Tensor | None = None,
                                scale_out: torch.Tensor | None = None,
                                residual_out: torch.Tensor | None = None, variant: int = -1):
    """fused_add_rmsnorm with a dynamic per-token E4M3 epilogue.
    Returns (q [T, H] fp8, scale [T] fp32, residual_out [T, H] bf16)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(residual, "residual", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=x.device)
    if scale_out is None:
        scale_out = torch.empty((T,), dtype=torch.float32, device=x.device)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _require(out, "out", FP8_DTYPES, (T, H))
    _require(scale_out, "scale_out", (torch.float32,), (T,))
    _require(residual_out, "residual_out", (torch.bfloat16,), (T, H))
    _same_device(x, residual, weight, out, scale_out, residual_out)
    lib = load()
    variant = _variant("fused_add_rmsnorm_quant_fp8", T, H, variant)
    _check(lib.fused_add_rmsnorm_quant_fp8_ex(out.data_ptr(), scale_out.data_ptr(),
                                              residual_out.data_ptr(), x.data_ptr(),
                                              residual.data_ptr(), weight.data_ptr(), T, H,
                                              float(eps), int(variant), _stream(x.get_device())),
           "fused_add_rmsnorm_quant_fp8")
    return out, scale_out, residual_out


def fused_add_rmsnorm_quant_fp8_static(x: torch.Tensor, residual: torch.Tensor,
                                       weight: torch.Tensor, scale: torch.Tensor, eps: float,
                                       out: torch.Tensor | None = None,
                                       residual_out: torch.Tensor | None = None, variant: int = -1):
    """fused_add_rmsnorm with a static per-tensor E4M3 epilogue; scale is a
    1-element fp32 GPU tensor read by the kernel.
    Returns (q [T, H] fp8, residual_out [T, H] bf16)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(residual, "residual", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    _require(scale, "scale", (torch.float32,), (1,))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=x.device)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _require(out, "out", FP8_DTYPES, (T, H))
    _require(residual_out, "residual_out", (torch.bfloat16,), (T, H))
    _same_device(x, residual, weight, scale, out, residual_out)
    lib = load()
    variant = _variant("fused_add_rmsnorm_quant_fp8_static", T, H, variant)
    _check(lib.fused_add_rmsnorm_quant_fp8_static_ex(out.data_ptr(), residual_out.data_ptr(),
                                                     x.data_ptr(), residual.data_ptr(),
                                                     weight.data_ptr(), scale.data_ptr(), T, H,
                                                     float(eps), int(variant), _stream(x.get_device())),
           "fused_add_rmsnorm_quant_fp8_static")
    return out, residual_out


def rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float, out: torch.Tensor | None = None,
            variant: int = -1):
    """RMSNorm without the residual add.  x: bf16 [T, H]; out=x runs in place."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    if out is None:
        out = torch.empty_like(x)
    _require(out, "out", (torch.bfloat16,), (T, H))
    _same_device(x, weight, out)
    lib = load()
    variant = _variant("rmsnorm", T, H, variant)
    _check(lib.rmsnorm_ex(out.data_ptr(), x.data_ptr(), weight.data_ptr(), T, H, float(eps),
                          int(variant), _stream(x.get_device())), "rmsnorm")
    return out


def rmsnorm_quant_fp8(x: torch.Tensor, weight: torch.Tensor, eps: float,
                      out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                      variant: int = -1):
    """rmsnorm with a dynamic per-token E4M3 epilogue.
    Returns (q [T, H] fp8, scale [T] fp32)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=x.device)
    if scale_out is None:
        scale_out = torch.empty((T,), dtype=torch.float32, device=x.device)
    _require(out, "out", FP8_DTYPES, (T, H))
    _require(scale_out, "scale_out", (torch.float32,), (T,))
    _same_device(x, weight, out, scale_out)
    lib = load()
    variant = _variant("rmsnorm_quant_fp8", T, H, variant)
    _check(lib.rmsnorm_quant_fp8_ex(out.data_ptr(), scale_out.data_ptr(), x.data_ptr(),
                                    weight.data_ptr(), T, H, float(eps), int(variant),
                                    _stream(x.get_device())), "rmsnorm_quant_fp8")
    return out, scale_out


def rmsnorm_quant_fp8_static(x: torch.Tensor, weight: torch.Tensor, scale: torch.Tensor, eps: float,
                             out: torch.Tensor | None = None, variant: int = -1):
    """rmsnorm with a static per-tensor E4M3 epilogue.  Returns q [T, H] fp8."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    _require(scale, "scale", (torch.float32,), (1,))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=x.device)
    _require(out, "out", FP8_DTYPES, (T, H))
    _same_device(x, weight, scale, out)
    lib = load()
    variant = _variant("rmsnorm_quant_fp8_static", T, H, variant)
    _check(lib.rmsnorm_quant_fp8_static_ex(out.data_ptr(), x.data_ptr(), weight.data_ptr(),
                                           scale.data_ptr(), T, H, float(eps), int(variant),
                                           _stream(x.get_device())), "rmsnorm_quant_fp8_static")
    return out


def _mx_outputs(T, H, device, out, scale_out):
    if H % 32:
        raise ValueError("the row width must be a multiple of 32 for MXFP4")
    if out is None:
        out = torch.empty((T, H // 2), dtype=torch.uint8, device=device)
    if scale_out is None:
        scale_out = torch.empty((T, H // 32), dtype=torch.uint8, device=device)
    _require(out, "out", (torch.uint8,), (T, H // 2))
    _require(scale_out, "scale_out", (torch.uint8,), (T, H // 32))
    return out, scale_out


def fused_add_rmsnorm_quant_mxfp4(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor,
                                  eps: float, out: torch.Tensor | None = None,
                                  scale_out: torch.Tensor | None = None,
                                  residual_out: torch.Tensor | None = None, variant: int = -1):
    """fused_add_rmsnorm with an MXFP4 epilogue.  Returns (q [T, H/2] uint8,
    two E2M1 codes per byte; scale [T, H/32] uint8 E8M0; residual_out)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(residual, "residual", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    out, scale_out = _mx_outputs(T, H, x.device, out, scale_out)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _require(residual_out, "residual_out", (torch.bfloat16,), (T, H))
    _same_device(x, residual, weight, out, scale_out, residual_out)
    lib = load()
    variant = _variant("fused_add_rmsnorm_quant_mxfp4", T, H, variant)
    _check(lib.fused_add_rmsnorm_quant_mxfp4_ex(out.data_ptr(), scale_out.data_ptr(),
                                                residual_out.data_ptr(), x.data_ptr(),
                                                residual.data_ptr(), weight.data_ptr(), T, H,
                                                float(eps), int(variant), _stream(x.get_device())),
           "fused_add_rmsnorm_quant_mxfp4")
    return out, scale_out, residual_out


def rmsnorm_quant_mxfp4(x: torch.Tensor, weight: torch.Tensor, eps: float,
                        out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                        variant: int = -1):
    """rmsnorm with an MXFP4 epilogue.  Returns (q [T, H/2], scale [T, H/32])."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    out, scale_out = _mx_outputs(T, H, x.device, out, scale_out)
    _same_device(x, weight, out, scale_out)
    lib = load()
    variant = _variant("rmsnorm_quant_mxfp4", T, H, variant)
    _check(lib.rmsnorm_quant_mxfp4_ex(out.data_ptr(), scale_out.data_ptr(), x.data_ptr(),
                                      weight.data_ptr(), T, H, float(eps), int(variant),
                                      _stream(x.get_device())), "rmsnorm_quant_mxfp4")
    return out, scale_out


def _nv_outputs(T, H, device, out, scale_out):
    if H % 16:
        raise ValueError("the row width must be a multiple of 16 for NVFP4")
    if out is None:
        out = torch.empty((T, H // 2), dtype=torch.uint8, device=device)
    if scale_out is None:
        scale_out = torch.empty((T, H // 16), dtype=torch.uint8, device=device)
    _require(out, "out", (torch.uint8,), (T, H // 2))
    _require(scale_out, "scale_out", (torch.uint8, torch.float8_e4m3fn), (T, H // 16))
    return out, scale_out


def fused_add_rmsnorm_quant_nvfp4(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor,
                                  tensor_scale: torch.Tensor, eps: float, out: torch.Tensor | None = None,
                                  scale_out: torch.Tensor | None = None,
                                  residual_out: torch.Tensor | None = None, variant: int = -1):
    """fused_add_rmsnorm with an NVFP4 epilogue under the 1-element fp32 GPU
    tensor scale.  Returns (q [T, H/2] uint8, scale [T, H/16] E4M3 bytes,
    residual_out)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(residual, "residual", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    _require(tensor_scale, "tensor_scale", (torch.float32,), (1,))
    out, scale_out = _nv_outputs(T, H, x.device, out, scale_out)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _require(residual_out, "residual_out", (torch.bfloat16,), (T, H))
    _same_device(x, residual, weight, tensor_scale, out, scale_out, residual_out)
    lib = load()
    variant = _variant("fused_add_rmsnorm_quant_nvfp4", T, H, variant)
    _check(lib.fused_add_rmsnorm_quant_nvfp4_ex(out.data_ptr(), scale_out.data_ptr(),
                                                residual_out.data_ptr(), x.data_ptr(),
                                                residual.data_ptr(), weight.data_ptr(),
                                                tensor_scale.data_ptr(), T, H, float(eps),
                                                int(variant), _stream(x.get_device())),
           "fused_add_rmsnorm_quant_nvfp4")
    return out, scale_out, residual_out


def rmsnorm_quant_nvfp4(x: torch.Tensor, weight: torch.Tensor, tensor_scale: torch.Tensor, eps: float,
                        out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                        variant: int = -1):
    """rmsnorm with an NVFP4 epilogue.  Returns (q [T, H/2], scale [T, H/16])."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    _require(tensor_scale, "tensor_scale", (torch.float32,), (1,))
    out, scale_out = _nv_outputs(T, H, x.device, out, scale_out)
    _same_device(x, weight, tensor_scale, out, scale_out)
    lib = load()
    variant = _variant("rmsnorm_quant_nvfp4", T, H, variant)
    _check(lib.rmsnorm_quant_nvfp4_ex(out.data_ptr(), scale_out.data_ptr(), x.data_ptr(),
                                      weight.data_ptr(), tensor_scale.data_ptr(), T, H, float(eps),
                                      int(variant), _stream(x.get_device())), "rmsnorm_quant_nvfp4")
    return out, scale_out


def swiglu(gate_up: torch.Tensor, out: torch.Tensor | None = None, variant: int = -1):
    """silu(gate) * up with gate_up = [gate | up] of shape [T, 2N]; returns bf16 [T, N]."""
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [tokens, 2 * inter]")
    T, N = gate_up.shape[0], gate_up.shape[1] // 2
    _require(gate_up, "gate_up", (torch.bfloat16,), (T, 2 * N))
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=gate_up.device)
    _require(out, "out", (torch.bfloat16,), (T, N))
    _same_device(gate_up, out)
    lib = load()
    variant = _variant("swiglu", T, N, variant)
    _check(lib.swiglu_ex(out.data_ptr(), gate_up.data_ptr(), T, N, int(variant),
                         _stream(gate_up.get_device())), "swiglu")
    return out


def swiglu_quant_fp8(gate_up: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None,
                     variant: int = -1):
    """swiglu with a static per-tensor E4M3 epilogue; scale is a 1-element
    fp32 GPU tensor read by the kernel.  Returns fp8 [T, N]."""
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [tokens, 2 * inter]")
    T, N = gate_up.shape[0], gate_up.shape[1] // 2
    _require(gate_up, "gate_up", (torch.bfloat16,), (T, 2 * N))
    _require(scale, "scale", (torch.float32,), (1,))
    if out is None:
        out = torch.empty((T, N), dtype=torch.float8_e4m3fn, device=gate_up.device)
    _require(out, "out", FP8_DTYPES, (T, N))
    _same_device(gate_up, scale, out)
    lib = load()
    variant = _variant("swiglu_quant_fp8", T, N, variant)
    _check(lib.swiglu_quant_fp8_ex(out.data_ptr(), gate_up.data_ptr(), scale.data_ptr(), T, N,
                                   int(variant), _stream(gate_up.get_device())), "swiglu_quant_fp8")
    return out


FP8_GROUP = 128   # values per scale of the per-group (block) E4M3 forms


def _group_outputs(T, W, device, out, scale_out):
    if W % FP8_GROUP:
        raise ValueError("the row width must be a multiple of %d for per-group E4M3" % FP8_GROUP)
    if out is None:
        out = torch.empty((T, W), dtype=torch.float8_e4m3fn, device=device)
    if scale_out is None:
        scale_out = torch.empty((T, W // FP8_GROUP), dtype=torch.float32, device=device)
    _require(out, "out", FP8_DTYPES, (T, W))
    _require(scale_out, "scale_out", (torch.float32,), (T, W // FP8_GROUP))
    return out, scale_out


def fused_add_rmsnorm_quant_fp8_group(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor,
                                      eps: float, out: torch.Tensor | None = None,
                                      scale_out: torch.Tensor | None = None,
                                      residual_out: torch.Tensor | None = None, variant: int = -1):
    """fused_add_rmsnorm with E4M3 codes under an fp32 scale per 128 values.
    Returns (q [T, H] fp8, scale [T, H/128] fp32, residual_out [T, H] bf16)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(residual, "residual", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    out, scale_out = _group_outputs(T, H, x.device, out, scale_out)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _require(residual_out, "residual_out", (torch.bfloat16,), (T, H))
    _same_device(x, residual, weight, out, scale_out, residual_out)
    lib = load()
    variant = _variant("fused_add_rmsnorm_quant_fp8_group", T, H, variant)
    _check(lib.fused_add_rmsnorm_quant_fp8_group_ex(out.data_ptr(), scale_out.data_ptr(),
                                                    residual_out.data_ptr(), x.data_ptr(),
                                                    residual.data_ptr(), weight.data_ptr(), T, H,
                                                    float(eps), int(variant), _stream(x.get_device())),
           "fused_add_rmsnorm_quant_fp8_group")
    return out, scale_out, residual_out


def rmsnorm_quant_fp8_group(x: torch.Tensor, weight: torch.Tensor, eps: float,
                            out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                            variant: int = -1):
    """rmsnorm with E4M3 codes under an fp32 scale per 128 values.
    Returns (q [T, H] fp8, scale [T, H/128] fp32)."""
    if x.dim() != 2:
        raise ValueError("x must be [tokens, hidden]")
    T, H = x.shape
    _require(x, "x", (torch.bfloat16,), (T, H))
    _require(weight, "weight", (torch.bfloat16,), (H,))
    out, scale_out = _group_outputs(T, H, x.device, out, scale_out)
    _same_device(x, weight, out, scale_out)
    lib = load()
    variant = _variant("rmsnorm_quant_fp8_group", T, H, variant)
    _check(lib.rmsnorm_quant_fp8_group_ex(out.data_ptr(), scale_out.data_ptr(), x.data_ptr(),
                                          weight.data_ptr(), T, H, float(eps), int(variant),
                                          _stream(x.get_device())), "rmsnorm_quant_fp8_group")
    return out, scale_out


def swiglu_quant_fp8_group(gate_up: torch.Tensor, out: torch.Tensor | None = None,
                           scale_out: torch.Tensor | None = None, variant: int = -1):
    """swiglu with E4M3 codes under an fp32 scale per 128 outputs.
    Returns (q [T, N] fp8, scale [T, N/128] fp32)."""
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [tokens, 2 * inter]")
    T, N = gate_up.shape[0], gate_up.shape[1] // 2
    _require(gate_up, "gate_up", (torch.bfloat16,), (T, 2 * N))
    out, scale_out = _group_outputs(T, N, gate_up.device, out, scale_out)
    _same_device(gate_up, out, scale_out)
    lib = load()
    variant = _variant("swiglu_quant_fp8_group", T, N, variant)
    _check(lib.swiglu_quant_fp8_group_ex(out.data_ptr(), scale_out.data_ptr(), gate_up.data_ptr(),
                                         T, N, int(variant), _stream(gate_up.get_device())),
           "swiglu_quant_fp8_group")
    return out, scale_out


def swiglu_quant_fp8_dynamic(gate_up: torch.Tensor, out: torch.Tensor | None = None,
                             scale_out: torch.Tensor | None = None, variant: int = -1):
    """swiglu with a dynamic per-token E4M3 epilogue.
    Returns (q [T, N] fp8, scale [T] fp32)."""
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [tokens, 2 * inter]")
    T, N = gate_up.shape[0], gate_up.shape[1] // 2
    _require(gate_up, "gate_up", (torch.bfloat16,), (T, 2 * N))
    if out is None:
        out = torch.empty((T, N), dtype=torch.float8_e4m3fn, device=gate_up.device)
    if scale_out is None:
        scale_out = torch.empty((T,), dtype=torch.float32, device=gate_up.device)
    _require(out, "out", FP8_DTYPES, (T, N))
    _require(scale_out, "scale_out", (torch.float32,), (T,))
    _same_device(gate_up, out, scale_out)
    lib = load()
    variant = _variant("swiglu_quant_fp8_dynamic", T, N, variant)
    _check(lib.swiglu_quant_fp8_dynamic_ex(out.data_ptr(), scale_out.data_ptr(), gate_up.data_ptr(),
                                           T, N, int(variant), _stream(gate_up.get_device())),
           "swiglu_quant_fp8_dynamic")
    return out, scale_out


def swiglu_quant_mxfp4(gate_up: torch.Tensor, out: torch.Tensor | None = None,
                       scale_out: torch.Tensor | None = None, variant: int = -1):
    """swiglu with an MXFP4 epilogue.  Returns (q [T, N/2] uint8, two E2M1
    codes per byte; scale [T, N/32] uint8 E8M0)."""
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [tokens, 2 * inter]")
    T, N = gate_up.shape[0], gate_up.shape[1] // 2
    _require(gate_up, "gate_up", (torch.bfloat16,), (T, 2 * N))
    out, scale_out = _mx_outputs(T, N, gate_up.device, out, scale_out)
    _same_device(gate_up, out, scale_out)
    lib = load()
    variant = _variant("swiglu_quant_mxfp4", T, N, variant)
    _check(lib.swiglu_quant_mxfp4_ex(out.data_ptr(), scale_out.data_ptr(), gate_up.data_ptr(), T, N,
                                     int(variant), _stream(gate_up.get_device())), "swiglu_quant_mxfp4")
    return out, scale_out


def swiglu_quant_nvfp4(gate_up: torch.Tensor, tensor_scale: torch.Tensor, out: torch.Tensor | None = None,
                       scale_out: torch.Tensor | None = None, variant: int = -1):
    """swiglu with an NVFP4 epilogue.  Returns (q [T, N/2] uint8, scale [T, N/16])."""
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [tokens, 2 * inter]")
    T, N = gate_up.shape[0], gate_up.shape[1] // 2
    _require(gate_up, "gate_up", (torch.bfloat16,), (T, 2 * N))
    _require(tensor_scale, "tensor_scale", (torch.float32,), (1,))
    out, scale_out = _nv_outputs(T, N, gate_up.device, out, scale_out)
    _same_device(gate_up, tensor_scale, out, scale_out)
    lib = load()
    variant = _variant("swiglu_quant_nvfp4", T, N, variant)
    _check(lib.swiglu_quant_nvfp4_ex(out.data_ptr(), scale_out.data_ptr(), gate_up.data_ptr(),
                                     tensor_scale.data_ptr(), T, N, int(variant), _stream(gate_up.get_device())),
           "swiglu_quant_nvfp4")
    return out, scale_out


def variant_count(op: int) -> int:
    return int(load().aarms_variant_count(int(op)))


def variant_name(op: int, variant: int) -> str | None:
    s = load().aarms_variant_name(int(op), int(variant))
    return s.decode() if s else None


def variant_fits(op: int, variant: int, width: int) -> bool:
    """Whether the variant runs rows of `width` values (the library's own
    check: capacity, and a multiple of 512 for the resident-row norms)."""
    return bool(load().aarms_variant_fits(int(op), int(variant), int(width)))


def pick_variant(op: int, tokens: int, width: int, quant: int | bool = False) -> int:
    """The heuristic's variant.  quant, the output format: for the norms
    (OP_NORM, OP_RMSNORM) 0 bf16, 1 E4M3 per token, 2 E4M3 per tensor,
    3 MXFP4, 4 NVFP4, 5 E4M3 per 128-value group; for OP_SWIGLU 0 bf16,
    1 E4M3, 2 MXFP4, 3 NVFP4, 4 E4M3 per 128-value group."""
    return int(load().aarms_pick_variant(int(op), int(tokens), int(width), int(quant)))
