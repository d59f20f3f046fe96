"""GPU parity, breadth: every gate pattern through every quantised SwiGLU
kernel, the four boundary entry points called directly through ctypes, and
the persistent norm kernels walking several rows in every output format.

Same bar as tests/test_parity_gpu.py: SwiGLU forms bit-exact against the
oracle (their SiLU is correctly rounded, so y has no knife-edges); norm
outputs equal to an admissible oracle value (tests/parity.py).
"""

from __future__ import annotations

import ctypes as C

import numpy as np
import pytest
import torch

import activation_add_rmsnorm_amd as A
import oracle
from tests import parity as P
from workloads import configs as W
from workloads import gen

pytestmark = pytest.mark.gpu

DEV = "cuda"


def announce(*what):
    print("[gpu]", *what, flush=True)


def bf16(bits):
    return P.to_gpu_bf16(bits, DEV)


def bits(t):
    return P.from_gpu_bits(t)


def f32(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


# ------------------------------------------------------------------ every gate, every quantised SwiGLU

GATES_PER_ROW = 512


def _every_gate_rows():
    """All 65,536 bf16 gate patterns in 128 rows of 512 (so that a row's
    scales come from its own gates: the non-finite patterns fill rows of
    their own), once with up = 1 (y = bf16(silu(g))) and once with up = 1.5
    (y = bf16(1.5 bf16(silu(g))), another rounding position for every gate)."""
    g = np.arange(65536, dtype=np.uint16).reshape(-1, GATES_PER_ROW)
    rows = []
    for u in (1.0, 1.5):
        up = np.full_like(g, oracle.bf16_from_f64(u))
        rows.append(np.concatenate([g, up], axis=1))
    return np.concatenate(rows, axis=0)


def _swiglu_variants():
    return range(A.variant_count(A.OP_SWIGLU))


def _rowq_variants(N):
    out = []
    for v in range(A.variant_count(A.OP_SWIGLU_DYNAMIC)):
        name = A.variant_name(A.OP_SWIGLU_DYNAMIC, v)
        w = 1 if name.startswith("wave/row") else int(name.split()[0])
        jobs = int(name.split("x")[-1].split()[0])
        if w * 64 * jobs * 8 >= N:
            out.append(v)
    return out


def test_every_gate_static_fp8_every_variant():
    gu = _every_gate_rows()
    gt = bf16(gu)
    for scale in (0.05, 1.0, 2.0 ** -10, 3.0e-3):
        for v in _swiglu_variants():
            announce("swiglu_quant_fp8 every gate", gu.shape, "scale", scale, "variant", v)
            q = bits(A.swiglu_quant_fp8(gt, f32(scale), variant=v))
            P.check_swiglu_fp8(gu, scale, q)


def test_every_gate_per_token_fp8_every_variant():
    gu = _every_gate_rows()
    gt = bf16(gu)
    for v in _rowq_variants(GATES_PER_ROW):
        announce("swiglu_quant_fp8_dynamic every gate", gu.shape, "variant", v,
                 A.variant_name(A.OP_SWIGLU_DYNAMIC, v))
        q, s = A.swiglu_quant_fp8_dynamic(gt, variant=v)
        P.check_swiglu_fp8_dynamic(gu, bits(q), bits(s))


def test_every_gate_block_scaled_every_variant():
    gu = _every_gate_rows()
    gt = bf16(gu)
    for v in _swiglu_variants():
        announce("swiglu block-scaled forms every gate", gu.shape, "variant", v)
        q, s = A.swiglu_quant_mxfp4(gt, variant=v)
        P.check_swiglu_mxfp4(gu, bits(q), bits(s))
        for g in (0.05, 1.0):
            q, s = A.swiglu_quant_nvfp4(gt, f32(g), variant=v)
            P.check_swiglu_nvfp4(gu, g, bits(q), bits(s))
        q, s = A.swiglu_quant_fp8_group(gt, variant=v)
        P.check_swiglu_fp8_group(gu, bits(q), bits(s))


def _flat_variant():
    return [v for v in _swiglu_variants() if A.variant_name(A.OP_SWIGLU, v) == "1 job/lane, flat rows"][0]


def _every_gate_in_rows_of(N, up):
    """All 65,536 gate patterns (then the first ones again to fill the last
    row) in rows of N gates, up constant."""
    T = -(-65536 // N)
    g = np.resize(np.arange(65536, dtype=np.uint16), T * N).reshape(T, N)
    return np.concatenate([g, np.full_like(g, oracle.bf16_from_f64(up))], axis=1)


def test_flat_grid_every_form_straddling_rows():
    """The flat grid's blocks of 256 jobs over rows of 257 jobs (N = 2,056:
    every block spans two rows, the last block is partial) and of 272 jobs
    (N = 2,176, the smallest width above 256 jobs that every block-scaled
    form takes), every gate pattern, in every output form, bit-exact."""
    v = _flat_variant()
    gu = _every_gate_in_rows_of(2056, 1.5)
    gt = bf16(gu)
    announce("flat grid bf16 and static E4M3", gu.shape)
    P.check_swiglu(gu, bits(A.swiglu(gt, variant=v)))
    for scale in (0.05, 2.0 ** -10):
        P.check_swiglu_fp8(gu, scale, bits(A.swiglu_quant_fp8(gt, f32(scale), variant=v)))
    gu = _every_gate_in_rows_of(2176, 1.5)
    gt = bf16(gu)
    announce("flat grid block-scaled forms", gu.shape)
    q, s = A.swiglu_quant_mxfp4(gt, variant=v)
    P.check_swiglu_mxfp4(gu, bits(q), bits(s))
    q, s = A.swiglu_quant_nvfp4(gt, f32(0.05), variant=v)
    P.check_swiglu_nvfp4(gu, 0.05, bits(q), bits(s))
    q, s = A.swiglu_quant_fp8_group(gt, variant=v)
    P.check_swiglu_fp8_group(gu, bits(q), bits(s))
    # the rows past the last one a block reaches are not written
    out = torch.full((gu.shape[0] + 1, gu.shape[1] // 2), -1, dtype=torch.int16, device=DEV)
    A.swiglu(gt, out=out[:-1].view(torch.bfloat16), variant=v)
    assert bool((out[-1] == -1).all())


def test_swiglu_fp8_dynamic_scales_every_significand():
    """The per-token and per-group scales are binary32(a / 448) for a bf16 a,
    and every such quotient goes through the corrected-quotient path: sweep
    every y (gate = 8, so silu rounds to 8, up = every bf16) against the
    scale of every one of the 128 bf16 significands, in two binades."""
    u = np.arange(65536, dtype=np.uint16)
    g = np.full(65536, oracle.bf16_from_f64(8.0), np.uint16)
    gu = np.concatenate([g, u])[None, :]
    gt = bf16(gu)
    for exp_bits in (0x4000, 0x3C00):            # a in [2, 4) and in [2^-7, 2^-6)
        for m in range(128):
            a = oracle.bf16_to_f32(np.array([exp_bits | m], np.uint16))[0]
            s = float(np.float32(a) / np.float32(448))
            q = bits(A.swiglu_quant_fp8(gt, f32(s)))
            P.check_swiglu_fp8(gu, s, q)


# ------------------------------------------------------------------ the boundary symbols themselves

def _lib():
    lib = A.load()
    vp, i64, f = C.c_void_p, C.c_int64, C.c_float
    lib.fused_add_rmsnorm.argtypes = [vp, vp, vp, vp, vp, i64, i64, f, vp]
    lib.fused_add_rmsnorm.restype = C.c_int
    lib.swiglu.argtypes = [vp, vp, i64, i64, vp]
    lib.swiglu.restype = C.c_int
    lib.swiglu_quant_fp8.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.swiglu_quant_fp8.restype = C.c_int
    lib.fused_add_rmsnorm_quant_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f, vp]
    lib.fused_add_rmsnorm_quant_fp8.restype = C.c_int
    return lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_boundary_fused_add_rmsnorm_direct():
    """fused_add_rmsnorm itself (not the _ex form the binding calls), on the
    16-token workload and on the 4,096-token prefill norm."""
    lib = _lib()
    for wl in (W.NORM_DECODE16, W.NORM_PREFILL4096):
        d = W.norm_inputs(wl)
        x, r, w = bf16(d["x"]), bf16(d["residual"]), bf16(d["weight"])
        out, ro = torch.empty_like(x), torch.empty_like(r)
        announce("fused_add_rmsnorm (C symbol)", (wl.tokens, wl.hidden))
        st = lib.fused_add_rmsnorm(out.data_ptr(), ro.data_ptr(), x.data_ptr(), r.data_ptr(), w.data_ptr(),
                                   wl.tokens, wl.hidden, wl.eps, _stream())
        assert st == 0, A._status_string(st)
        torch.cuda.synchronize()
        P.check_norm(d["x"], d["residual"], d["weight"], wl.eps, bits(out), bits(ro))


def test_boundary_swiglu_direct():
    lib = _lib()
    for T in (16, 4096):
        gu = gen.normal_bf16((T, 2 * 8960), T, 4)
        gt = bf16(gu)
        y = torch.empty((T, 8960), dtype=torch.bfloat16, device=DEV)
        announce("swiglu (C symbol)", gu.shape)
        st = lib.swiglu(y.data_ptr(), gt.data_ptr(), T, 8960, _stream())
        assert st == 0, A._status_string(st)
        torch.cuda.synchronize()
        P.check_swiglu(gu, bits(y))


def test_boundary_swiglu_quant_fp8_direct():
    """The Llama-70B activation's distribution and scale on 64 of its rows."""
    lib = _lib()
    wl = W.SWIGLU_FP8_LLAMA70B
    T, N = 64, wl.inter
    gu = gen.normal_bf16((T, 2 * N), 0, 4, std=wl.gate_up_std)
    gt = bf16(gu)
    q = torch.empty((T, N), dtype=torch.uint8, device=DEV)
    s = f32(wl.scale)
    announce("swiglu_quant_fp8 (C symbol)", gu.shape, "scale", wl.scale)
    st = lib.swiglu_quant_fp8(q.data_ptr(), gt.data_ptr(), s.data_ptr(), T, N, _stream())
    assert st == 0, A._status_string(st)
    torch.cuda.synchronize()
    P.check_swiglu_fp8(gu, wl.scale, bits(q))


def test_boundary_fused_add_rmsnorm_quant_fp8_direct():
    """The Llama-405B norm's distribution (0.1% outliers x50), eps and width
    on 64 rows."""
    lib = _lib()
    wl = W.NORM_FP8_LLAMA405B
    d = W.norm_inputs(wl, tokens=64)
    x, r, w = bf16(d["x"]), bf16(d["residual"]), bf16(d["weight"])
    T, H = x.shape
    q = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    sc = torch.empty((T,), dtype=torch.float32, device=DEV)
    ro = torch.empty_like(r)
    announce("fused_add_rmsnorm_quant_fp8 (C symbol)", (T, H))
    st = lib.fused_add_rmsnorm_quant_fp8(q.data_ptr(), sc.data_ptr(), ro.data_ptr(), x.data_ptr(), r.data_ptr(),
                                         w.data_ptr(), T, H, wl.eps, _stream())
    assert st == 0, A._status_string(st)
    torch.cuda.synchronize()
    P.check_norm_fp8(d["x"], d["residual"], d["weight"], wl.eps, bits(q), bits(sc), bits(ro))


# ------------------------------------------------------------------ persistent norms, every epilogue

def _pipelined_variants():
    out = []
    for v in range(A.variant_count(A.OP_NORM)):
        name = A.variant_name(A.OP_NORM, v)
        if "pipelined" not in name:
            continue
        w = 1 if name.startswith("wave/row") else int(name.split()[0])
        vec = int(name.split("x")[-1].split()[0])
        bpc = int(name.split("pipelined")[1].split()[0])
        out.append((v, name, w, vec, bpc))
    return out


def _all_norm_forms(x, r, w, eps, g, v):
    """Every norm output format, with the residual add and without, at
    variant v, each checked against the oracle."""
    xt, rt, wt = bf16(x), bf16(r), bf16(w)
    gt = f32(g)
    o, ro = A.fused_add_rmsnorm(xt, rt, wt, eps, variant=v)
    P.check_norm(x, r, w, eps, bits(o), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8(xt, rt, wt, eps, variant=v)
    P.check_norm_fp8(x, r, w, eps, bits(q), bits(s), bits(ro))
    q, ro = A.fused_add_rmsnorm_quant_fp8_static(xt, rt, wt, gt, eps, variant=v)
    P.check_norm_fp8_static(x, r, w, eps, g, bits(q), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8_group(xt, rt, wt, eps, variant=v)
    P.check_norm_fp8_group(x, r, w, eps, bits(q), bits(s), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_mxfp4(xt, rt, wt, eps, variant=v)
    P.check_norm_mxfp4(x, r, w, eps, bits(q), bits(s), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_nvfp4(xt, rt, wt, gt, eps, variant=v)
    P.check_norm_nvfp4(x, r, w, eps, g, bits(q), bits(s), bits(ro))
    o = A.rmsnorm(xt, wt, eps, variant=v)
    P.check_rmsnorm(x, w, eps, bits(o))
    q, s = A.rmsnorm_quant_fp8(xt, wt, eps, variant=v)
    P.check_rmsnorm_fp8(x, w, eps, bits(q), bits(s))
    q = A.rmsnorm_quant_fp8_static(xt, wt, gt, eps, variant=v)
    P.check_rmsnorm_fp8_static(x, w, eps, g, bits(q))
    q, s = A.rmsnorm_quant_fp8_group(xt, wt, eps, variant=v)
    P.check_rmsnorm_fp8_group(x, w, eps, bits(q), bits(s))
    q, s = A.rmsnorm_quant_mxfp4(xt, wt, eps, variant=v)
    P.check_rmsnorm_mxfp4(x, w, eps, bits(q), bits(s))
    q, s = A.rmsnorm_quant_nvfp4(xt, wt, gt, eps, variant=v)
    P.check_rmsnorm_nvfp4(x, w, eps, g, bits(q), bits(s))
    torch.cuda.synchronize()


@pytest.mark.parametrize("v,name,w,vec,bpc", _pipelined_variants() if torch.cuda.is_available() else [])
def test_pipelined_variant_walks_rows_every_epilogue(v, name, w, vec, bpc):
    """More rows than the persistent grid holds (two rows per block, some a
    third), so every block carries the next row's registers, its partial-sum
    slot and the NVFP4 reciprocal table across rows, in every output format,
    with and without the residual add."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows_per_block = 4 if w == 1 else 1
    H = min(w * 64 * vec * 8, 16384) if w > 1 else 1536
    T = 2 * cus * bpc * rows_per_block + 37
    x = gen.normal_bf16((T, H), v, 1, outlier_frac=0.001)
    r = gen.normal_bf16((T, H), v, 2)
    wt = gen.normal_bf16((H,), v, 3, mean=1.0, std=0.1)
    announce("norm forms", name, (T, H))
    _all_norm_forms(x, r, wt, 1e-5, 0.02, v)


@pytest.mark.parametrize("v,name,w,vec,bpc", _pipelined_variants() if torch.cuda.is_available() else [])
def test_pipelined_variant_special_rows_between_normal_ones(v, name, w, vec, bpc):
    """The special rows (zero, NaN, Inf, subnormal, extreme scales,
    cancelling, overflowing) as the first and the last rows of a batch the
    persistent grid walks, so that blocks carry their registers, partial-sum
    slot and reciprocal table from a special row into normal ones and from
    normal rows into special ones: nothing may leak across rows."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows_per_block = 4 if w == 1 else 1
    H = min(w * 64 * vec * 8, 16384) if w > 1 else 1536
    T = 2 * cus * bpc * rows_per_block + 37
    x = gen.normal_bf16((T, H), v + 100, 1, outlier_frac=0.001)
    r = gen.normal_bf16((T, H), v + 100, 2)
    sx, sr = _special_rows(12, H, v + 100)
    x[:10], r[:10] = sx[:10], sr[:10]
    x[-10:], r[-10:] = sx[:10], sr[:10]
    wt = gen.normal_bf16((H,), v + 100, 3, mean=1.0, std=0.1)
    announce("norm forms, special rows", name, (T, H))
    _all_norm_forms(x, r, wt, 1e-5, 0.02, v)


def _resident_variants():
    return [(v, A.variant_name(A.OP_NORM, v)) for v in range(A.variant_count(A.OP_NORM))
            if "resident" in A.variant_name(A.OP_NORM, v)]


@pytest.mark.parametrize("T,H", [(37, 512), (5, 16384), (130, 12800), (300, 16384)])
def test_resident_variants_every_epilogue(T, H):
    """The resident-row kernels (one wave holds a whole row; four rows per
    block) in every output format, with and without the residual add: rows
    narrower than the 32 slices a lane can hold (whole slices past the row
    end, 512 and 12,800 wide), waves past the last row (T not a multiple of
    4), and more blocks than one per CU."""
    x = gen.normal_bf16((T, H), T, 1, outlier_frac=0.001)
    r = gen.normal_bf16((T, H), T, 2)
    wt = gen.normal_bf16((H,), T, 3, mean=1.0, std=0.1)
    for v, name in _resident_variants():
        announce("norm forms", name, (T, H))
        _all_norm_forms(x, r, wt, 1e-5, 0.02, v)


@pytest.mark.parametrize("T", [1024, 2040])
def test_resident_default_pick_per_token(T):
    """Per-token E4M3 with the residual add where the library picks the
    resident rows (about one and about two four-row blocks per CU), against
    the oracle, with the Llama-405B norm's input recipe."""
    H = 16384
    name = A.variant_name(A.OP_NORM, A.pick_variant(A.OP_NORM, T, H, 1))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:
        assert "resident" in name, name
    x = gen.normal_bf16((T, H), T, 1, outlier_frac=0.001, outlier_mult=50.0)
    r = gen.normal_bf16((T, H), T, 2)
    wt = gen.normal_bf16((H,), T, 3, mean=1.0, std=0.1)
    announce("fused_add_rmsnorm_quant_fp8 default", name, (T, H))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8(bf16(x), bf16(r), bf16(wt), 1e-5)
    torch.cuda.synchronize()
    P.check_norm_fp8(x, r, wt, 1e-5, bits(q), bits(s), bits(ro))


@pytest.mark.parametrize("T,H,f", [(1792, 8192, 0), (2048, 6144, 0), (832, 10240, 1), (1024, 12288, 2),
                                   (2048, 10240, 2), (1920, 12288, 1)])
def test_resident_default_pick_mid_widths(T, H, f):
    """The forms with the residual add where the library picks the resident
    rows on rows of 6,144-12,288 (bf16 in the second band from 6,144, every
    E4M3 form in both bands from 10,240), against the oracle."""
    name = A.variant_name(A.OP_NORM, A.pick_variant(A.OP_NORM, T, H, f))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert "resident" in name, name
    x = gen.normal_bf16((T, H), T + H, 1, outlier_frac=0.001, outlier_mult=50.0)
    r = gen.normal_bf16((T, H), T + H, 2)
    wt = gen.normal_bf16((H,), T + H, 3, mean=1.0, std=0.1)
    announce("norm form", f, "default", name, (T, H))
    if f == 0:
        o, ro = A.fused_add_rmsnorm(bf16(x), bf16(r), bf16(wt), 1e-6)
        torch.cuda.synchronize()
        P.check_norm(x, r, wt, 1e-6, bits(o), bits(ro))
    elif f == 1:
        q, s, ro = A.fused_add_rmsnorm_quant_fp8(bf16(x), bf16(r), bf16(wt), 1e-5)
        torch.cuda.synchronize()
        P.check_norm_fp8(x, r, wt, 1e-5, bits(q), bits(s), bits(ro))
    else:
        q, ro = A.fused_add_rmsnorm_quant_fp8_static(bf16(x), bf16(r), bf16(wt), f32(0.02), 1e-5)
        torch.cuda.synchronize()
        P.check_norm_fp8_static(x, r, wt, 1e-5, 0.02, bits(q), bits(ro))


def _special_rows(T, H, seed):
    """Rows the resident kernels have to get right besides random ones (bf16
    bit patterns): zero, constant, a NaN, an infinity, bf16 subnormals,
    rows scaled by 1e30 and 1e-30, a lone outlier, x = -residual (a zero
    sum), and a sum that overflows bf16; the rest random."""
    x = gen.normal_bf16((T, H), seed, 1, outlier_frac=0.001)
    r = gen.normal_bf16((T, H), seed, 2)
    one = lambda v: np.uint16(oracle.bf16_from_f64(v))
    x[0, :] = 0
    r[0, :] = 0
    x[1, :] = one(1.0)
    r[1, :] = 0
    x[2, 100] = 0x7FC0                                  # NaN
    r[3, 7] = 0x7F80                                    # +inf
    x[4, :] = (np.arange(H) % 127 + 1).astype(np.uint16)  # bf16 subnormals
    r[4, :] = 0
    x[5, :] = one(1e30)
    x[5, ::3] = one(-1e30)
    r[5, :] = 0
    x[6, :] = one(1e-30)
    r[6, ::5] = one(-2e-30)
    x[7, :] = 0
    r[7, :] = 0
    x[7, H // 2 + 3] = one(3e4)
    r[8, :] = x[8, :] ^ np.uint16(0x8000)               # x + residual = 0 exactly
    x[9, :] = one(3e38)
    r[9, :] = one(3e38)                                 # the sum rounds to +inf in bf16
    return x, r


@pytest.mark.parametrize("H", [1024, 16384])
def test_resident_variants_special_rows(H):
    """Zero, constant, non-finite, subnormal, extreme-scale and cancelling
    rows through the resident-row kernels in every output format, with and
    without the residual add (the library's default variant at this shape,
    rows split over waves, runs the same rows as a control)."""
    T = 12
    x, r = _special_rows(T, H, 7)
    wt = gen.normal_bf16((H,), 7, 3, mean=1.0, std=0.1)
    for v, name in _resident_variants() + [(-1, "default")]:
        announce("special rows", name, (T, H))
        _all_norm_forms(x, r, wt, 1e-5, 0.02, v)
