"""CPU oracle for fused residual-add + RMSNorm, SwiGLU and their FP8 and
block-scaled FP4 (MXFP4, NVFP4) epilogues.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it; the product path never does.  It
shares no code with the HIP library.  The arithmetic lives in
``aarms_oracle.c`` (plain C, see its header for the definitions followed and
the pages they come from); this module only builds that file and marshals
numpy arrays.

bf16 tensors are numpy ``uint16`` bit patterns, E4M3 tensors ``uint8`` codes.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "aarms_oracle.c")
# AARMS_ORACLE_LIB names another build of aarms_oracle.c (the host-sanitizer
# test loads one built with AddressSanitizer and UBSan).
_LIB_PATH = os.environ.get("AARMS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_LOCK = threading.Lock()
_LIB = None

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile aarms_oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = C.CDLL(_LIB_PATH)
            u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
            u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
            f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
            f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
            i64, f32, f64 = C.c_int64, C.c_float, C.c_double
            sig = {
                "aarms_oracle_bf16_to_f32": (f32, [C.c_uint16]),
                "aarms_oracle_bf16_from_f64": (C.c_uint16, [f64]),
                "aarms_oracle_e4m3_from_f64": (C.c_uint8, [f64]),
                "aarms_oracle_e4m3_to_f64": (f64, [C.c_uint8]),
                "aarms_oracle_residual_add": (None, [u16p, u16p, i64, u16p]),
                "aarms_oracle_rms_scale": (None, [u16p, i64, i64, f32, f32p, C.c_void_p]),
                "aarms_oracle_rmsnorm_apply": (None, [u16p, u16p, f32p, i64, i64, u16p]),
                "aarms_oracle_rms_window": (None, [f64p, i64, f64, f32p, f32p]),
                "aarms_oracle_fused_add_rmsnorm": (None, [u16p, u16p, u16p, i64, i64, f32, u16p, u16p, f32p]),
                "aarms_oracle_rmsnorm": (None, [u16p, u16p, i64, i64, f32, u16p, f32p]),
                "aarms_oracle_quant_fp8_static": (None, [u16p, i64, f32, u8p]),
                "aarms_oracle_quant_fp8_per_row": (None, [u16p, i64, i64, u8p, f32p]),
                "aarms_oracle_quant_fp8_per_group": (None, [u16p, i64, i64, i64, u8p, f32p]),
                "aarms_oracle_fused_add_rmsnorm_quant_fp8": (
                    None, [u16p, u16p, u16p, i64, i64, f32, u16p, u8p, f32p, u16p, f32p]),
                "aarms_oracle_silu_bf16": (C.c_uint16, [C.c_uint16]),
                "aarms_oracle_swiglu": (None, [u16p, i64, i64, u16p]),
                "aarms_oracle_swiglu_quant_fp8": (None, [u16p, i64, i64, f32, u8p]),
                "aarms_oracle_swiglu_quant_fp8_per_row": (None, [u16p, i64, i64, u16p, u8p, f32p]),
                "aarms_oracle_e2m1_from_f64": (C.c_uint8, [f64]),
                "aarms_oracle_e2m1_to_f64": (f64, [C.c_uint8]),
                "aarms_oracle_e8m0_to_f64": (f64, [C.c_uint8]),
                "aarms_oracle_quant_mxfp4": (None, [u16p, i64, i64, u8p, u8p]),
                "aarms_oracle_quant_nvfp4": (None, [u16p, i64, i64, f32, u8p, u8p]),
                "aarms_oracle_num_threads": (C.c_int, []),
                "aarms_oracle_set_threads": (None, [C.c_int]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _LIB = lib
    return _LIB


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 tensors are passed as uint16 bit patterns, got %s" % a.dtype)
    return a


def _rows(a: np.ndarray):
    if a.ndim != 2:
        raise ValueError("expected a 2-D [tokens, width] array")
    return a.shape


# ---------------------------------------------------------------- formats

def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_from_f64(v: float) -> int:
    return int(_lib().aarms_oracle_bf16_from_f64(float(v)))


def e4m3_from_f64(v: float) -> int:
    return int(_lib().aarms_oracle_e4m3_from_f64(float(v)))


def e4m3_to_f64(q: int) -> float:
    return float(_lib().aarms_oracle_e4m3_to_f64(int(q)))


def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (NaN for the two NaN codes)."""
    return np.array([e4m3_to_f64(q) for q in range(256)], dtype=np.float64)


# ---------------------------------------------------------------- norm

def residual_add(x, residual) -> np.ndarray:
    x, residual = _u16(x), _u16(residual)
    if x.shape != residual.shape:
        raise ValueError("shape mismatch")
    out = np.empty_like(x)
    _lib().aarms_oracle_residual_add(x.reshape(-1), residual.reshape(-1), x.size, out.reshape(-1))
    return out


def rms_scale(r, eps: float):
    """Per-row float32 multiplier 1/sqrt(mean(h^2) + eps) and its binary64 centre."""
    r = _u16(r)
    T, H = _rows(r)
    rs = np.empty(T, np.float32)
    rs_exact = np.empty(T, np.float64)
    _lib().aarms_oracle_rms_scale(r, T, H, float(eps), rs, rs_exact.ctypes.data_as(C.c_void_p))
    return rs, rs_exact


def rmsnorm_apply(r, weight, rho) -> np.ndarray:
    r, weight = _u16(r), _u16(weight)
    T, H = _rows(r)
    rho = np.ascontiguousarray(rho, dtype=np.float32)
    if weight.shape != (H,) or rho.shape != (T,):
        raise ValueError("shape mismatch")
    y = np.empty_like(r)
    _lib().aarms_oracle_rmsnorm_apply(r, weight, rho, T, H, y)
    return y


def rms_window(rs_exact, delta: float):
    rs_exact = np.ascontiguousarray(rs_exact, dtype=np.float64)
    lo = np.empty(rs_exact.shape, np.float32)
    hi = np.empty(rs_exact.shape, np.float32)
    _lib().aarms_oracle_rms_window(rs_exact, rs_exact.size, float(delta), lo, hi)
    return lo, hi


def fused_add_rmsnorm(x, residual, weight, eps: float):
    """Returns (out, residual_out, rs)."""
    x, residual, weight = _u16(x), _u16(residual), _u16(weight)
    T, H = _rows(x)
    if residual.shape != (T, H) or weight.shape != (H,):
        raise ValueError("shape mismatch")
    out = np.empty_like(x)
    res_out = np.empty_like(x)
    rs = np.empty(T, np.float32)
    _lib().aarms_oracle_fused_add_rmsnorm(x, residual, weight, T, H, float(eps), out, res_out, rs)
    return out, res_out, rs


def rmsnorm(x, weight, eps: float):
    """RMSNorm without the residual add.  Returns (out, rs)."""
    x, weight = _u16(x), _u16(weight)
    T, H = _rows(x)
    if weight.shape != (H,):
        raise ValueError("shape mismatch")
    out = np.empty_like(x)
    rs = np.empty(T, np.float32)
    _lib().aarms_oracle_rmsnorm(x, weight, T, H, float(eps), out, rs)
    return out, rs


# ---------------------------------------------------------------- fp8

def quant_fp8_static(y, scale: float) -> np.ndarray:
    y = _u16(y)
    q = np.empty(y.shape, np.uint8)
    _lib().aarms_oracle_quant_fp8_static(y.reshape(-1), y.size, float(np.float32(scale)), q.reshape(-1))
    return q


def quant_fp8_per_row(y):
    """Returns (q, s): per-row scale s = max|y| / 448 and the E4M3 codes."""
    y = _u16(y)
    T, H = _rows(y)
    q = np.empty((T, H), np.uint8)
    s = np.empty(T, np.float32)
    _lib().aarms_oracle_quant_fp8_per_row(y, T, H, q, s)
    return q, s


FP8_GROUP = 128   # values per scale group of the per-group (block) E4M3 forms


def quant_fp8_per_group(y, group: int = FP8_GROUP):
    """Returns (q, s): for each row, groups of `group` consecutive values,
    s[row, g] = max|y| over the group / 448 (binary32), and the E4M3 codes of
    y divided by its group's scale."""
    y = _u16(y)
    T, H = _rows(y)
    if group <= 0 or H % group:
        raise ValueError("the row width must be a multiple of the group size")
    q = np.empty((T, H), np.uint8)
    s = np.empty((T, H // group), np.float32)
    _lib().aarms_oracle_quant_fp8_per_group(y, T, H, group, q, s)
    return q, s


def fused_add_rmsnorm_quant_fp8_group(x, residual, weight, eps: float, group: int = FP8_GROUP):
    """fused_add_rmsnorm, its bf16 output quantised per group.  Returns (q,
    s [T, H/group], residual_out, y, rs)."""
    out, res_out, rs = fused_add_rmsnorm(x, residual, weight, eps)
    q, s = quant_fp8_per_group(out, group)
    return q, s, res_out, out, rs


def rmsnorm_quant_fp8_group(x, weight, eps: float, group: int = FP8_GROUP):
    """rmsnorm (no residual add), quantised per group.  Returns (q, s, y, rs)."""
    out, rs = rmsnorm(x, weight, eps)
    q, s = quant_fp8_per_group(out, group)
    return q, s, out, rs


def swiglu_quant_fp8_group(gate_up, group: int = FP8_GROUP):
    """swiglu, quantised per group.  Returns (q, s [T, N/group], y)."""
    y = swiglu(gate_up)
    q, s = quant_fp8_per_group(y, group)
    return q, s, y


def fused_add_rmsnorm_quant_fp8(x, residual, weight, eps: float):
    """Returns (q, s, residual_out, y, rs); y is the bf16 norm output before
    quantisation."""
    x, residual, weight = _u16(x), _u16(residual), _u16(weight)
    T, H = _rows(x)
    if residual.shape != (T, H) or weight.shape != (H,):
        raise ValueError("shape mismatch")
    y = np.empty_like(x)
    q = np.empty((T, H), np.uint8)
    s = np.empty(T, np.float32)
    res_out = np.empty_like(x)
    rs = np.empty(T, np.float32)
    _lib().aarms_oracle_fused_add_rmsnorm_quant_fp8(x, residual, weight, T, H, float(eps),
                                                   y, q, s, res_out, rs)
    return q, s, res_out, y, rs


def fused_add_rmsnorm_quant_fp8_static(x, residual, weight, eps: float, scale: float):
    """The norm with its bf16 output quantised with a given per-tensor scale.
    Returns (q, residual_out, y, rs)."""
    out, res_out, rs = fused_add_rmsnorm(x, residual, weight, eps)
    return quant_fp8_static(out, scale), res_out, out, rs


def rmsnorm_quant_fp8(x, weight, eps: float):
    """RMSNorm (no residual add), quantised per token.  Returns (q, s, y, rs)."""
    out, rs = rmsnorm(x, weight, eps)
    q, s = quant_fp8_per_row(out)
    return q, s, out, rs


def rmsnorm_quant_fp8_static(x, weight, eps: float, scale: float):
    """RMSNorm (no residual add), quantised with a per-tensor scale.
    Returns (q, y, rs)."""
    out, rs = rmsnorm(x, weight, eps)
    return quant_fp8_static(out, scale), out, rs


# ---------------------------------------------------------------- mxfp4

def e2m1_from_f64(v: float) -> int:
    return int(_lib().aarms_oracle_e2m1_from_f64(float(v)))


def e2m1_to_f64(q: int) -> float:
    return float(_lib().aarms_oracle_e2m1_to_f64(int(q)))


def e2m1_table() -> np.ndarray:
    """Values of the 16 E2M1 codes."""
    return np.array([e2m1_to_f64(q) for q in range(16)], dtype=np.float64)


def e8m0_to_f64(b: int) -> float:
    return float(_lib().aarms_oracle_e8m0_to_f64(int(b)))


def quant_mxfp4(y):
    """MXFP4 of each row (width a multiple of 32).  Returns (q [T, H/2]
    uint8, two codes per byte with the first in the low nibble;
    s [T, H/32] uint8 E8M0 block scales)."""
    y = _u16(y)
    T, H = _rows(y)
    if H % 32:
        raise ValueError("width must be a multiple of 32")
    q = np.empty((T, H // 2), np.uint8)
    s = np.empty((T, H // 32), np.uint8)
    _lib().aarms_oracle_quant_mxfp4(y, T, H, q, s)
    return q, s


def mxfp4_decode(q, s) -> np.ndarray:
    """float64 values of MXFP4 codes q [T, H/2] with block scales s [T, H/32]."""
    q, s = np.asarray(q, np.uint8), np.asarray(s, np.uint8)
    tab = e2m1_table()
    el = np.stack([tab[q & 0xF], tab[q >> 4]], axis=-1).reshape(q.shape[0], -1)
    sc = np.array([e8m0_to_f64(b) for b in range(256)])[s]
    return el * np.repeat(sc, 32, axis=1)


def quant_nvfp4(y, tensor_scale: float):
    """NVFP4 of each row (width a multiple of 16) under the fp32 tensor scale.
    Returns (q [T, H/2] uint8, two codes per byte with the first in the low
    nibble; s [T, H/16] uint8 E4M3 block scales)."""
    y = _u16(y)
    T, H = _rows(y)
    if H % 16:
        raise ValueError("width must be a multiple of 16")
    q = np.empty((T, H // 2), np.uint8)
    s = np.empty((T, H // 16), np.uint8)
    _lib().aarms_oracle_quant_nvfp4(y, T, H, float(np.float32(tensor_scale)), q, s)
    return q, s


def nvfp4_decode(q, s, tensor_scale: float) -> np.ndarray:
    """float64 values of NVFP4 codes q [T, H/2], block scales s [T, H/16]."""
    q, s = np.asarray(q, np.uint8), np.asarray(s, np.uint8)
    tab = e2m1_table()
    el = np.stack([tab[q & 0xF], tab[q >> 4]], axis=-1).reshape(q.shape[0], -1)
    g = float(np.float32(tensor_scale)) or 1.0
    sc = e4m3_table()[s] * g
    return el * np.repeat(sc, 16, axis=1)


def fused_add_rmsnorm_quant_nvfp4(x, residual, weight, eps: float, tensor_scale: float):
    """The norm, its bf16 output in NVFP4.  Returns (q, s, residual_out, y, rs)."""
    out, res_out, rs = fused_add_rmsnorm(x, residual, weight, eps)
    q, s = quant_nvfp4(out, tensor_scale)
    return q, s, res_out, out, rs


def rmsnorm_quant_nvfp4(x, weight, eps: float, tensor_scale: float):
    """RMSNorm (no residual add), its bf16 output in NVFP4.  Returns (q, s, y, rs)."""
    out, rs = rmsnorm(x, weight, eps)
    q, s = quant_nvfp4(out, tensor_scale)
    return q, s, out, rs


def fused_add_rmsnorm_quant_mxfp4(x, residual, weight, eps: float):
    """The norm, its bf16 output in MXFP4.  Returns (q, s, residual_out, y, rs)."""
    out, res_out, rs = fused_add_rmsnorm(x, residual, weight, eps)
    q, s = quant_mxfp4(out)
    return q, s, res_out, out, rs


def rmsnorm_quant_mxfp4(x, weight, eps: float):
    """RMSNorm (no residual add), its bf16 output in MXFP4.  Returns (q, s, y, rs)."""
    out, rs = rmsnorm(x, weight, eps)
    q, s = quant_mxfp4(out)
    return q, s, out, rs


# ---------------------------------------------------------------- swiglu

def silu_bf16(g_bits) -> np.ndarray:
    """bf16(silu(g)) for each bf16 bit pattern g."""
    g = np.asarray(g_bits, dtype=np.uint16)
    f = _lib().aarms_oracle_silu_bf16
    return np.array([f(int(v)) for v in g.reshape(-1)], dtype=np.uint16).reshape(g.shape)


def silu_table() -> np.ndarray:
    """bf16(silu(g)) for all 65,536 bf16 patterns g, indexed by the pattern."""
    return silu_bf16(np.arange(65536, dtype=np.uint16))


def swiglu(gate_up) -> np.ndarray:
    gu = _u16(gate_up)
    T, W = _rows(gu)
    if W % 2:
        raise ValueError("gate_up width must be even")
    y = np.empty((T, W // 2), np.uint16)
    _lib().aarms_oracle_swiglu(gu, T, W // 2, y)
    return y


def swiglu_quant_fp8(gate_up, scale: float) -> np.ndarray:
    gu = _u16(gate_up)
    T, W = _rows(gu)
    if W % 2:
        raise ValueError("gate_up width must be even")
    q = np.empty((T, W // 2), np.uint8)
    _lib().aarms_oracle_swiglu_quant_fp8(gu, T, W // 2, float(np.float32(scale)), q)
    return q


def swiglu_quant_fp8_dynamic(gate_up):
    """SwiGLU quantised per token.  Returns (q, s, y); y is the bf16 SwiGLU
    output before quantisation."""
    gu = _u16(gate_up)
    T, W = _rows(gu)
    if W % 2:
        raise ValueError("gate_up width must be even")
    y = np.empty((T, W // 2), np.uint16)
    q = np.empty((T, W // 2), np.uint8)
    s = np.empty(T, np.float32)
    _lib().aarms_oracle_swiglu_quant_fp8_per_row(gu, T, W // 2, y, q, s)
    return q, s, y


def set_threads(n: int) -> None:
    """Threads for the oracle's OpenMP loops in this process."""
    _lib().aarms_oracle_set_threads(int(n))


def swiglu_quant_mxfp4(gate_up):
    """SwiGLU, its bf16 output in MXFP4.  Returns (q, s, y)."""
    y = swiglu(gate_up)
    q, s = quant_mxfp4(y)
    return q, s, y


def swiglu_quant_nvfp4(gate_up, tensor_scale: float):
    """SwiGLU, its bf16 output in NVFP4.  Returns (q, s, y)."""
    y = swiglu(gate_up)
    q, s = quant_nvfp4(y, tensor_scale)
    return q, s, y


def num_threads() -> int:
    return int(_lib().aarms_oracle_num_threads())
