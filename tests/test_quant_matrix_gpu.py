"""GPU parity for the rest of the quantisation matrix: RMSNorm without the
residual add (bf16, per-token E4M3, per-tensor E4M3), the residual-add norm
with a per-tensor E4M3 scale, and SwiGLU with a per-token E4M3 scale -- the
HIP kernels through the C ABI against the CPU oracle, to the same bar as the
other ops (tests/parity.py)."""

from __future__ import annotations

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
SCALES = [0.05, 0.0125, 1.0, 2.0 ** -126, 2.0 ** 120, 0.0]


def announce(*what):
    print("[gpu]", *what, flush=True)


def bf16(b):
    return P.to_gpu_bf16(b, DEV)


def bits(t):
    return P.from_gpu_bits(t)


def scale_t(s):
    return torch.tensor([s], dtype=torch.float32, device=DEV)


def norm_case(T, H, seed=0, outliers=0.0, std=1.0):
    x = gen.normal_bf16((T, H), seed, 1, std=std, outlier_frac=outliers)
    r = gen.normal_bf16((T, H), seed, 2, outlier_frac=outliers)
    w = gen.normal_bf16((H,), seed, 3, mean=1.0, std=0.1)
    return x, r, w


def variants_for(op, width):
    return [v for v in range(A.variant_count(op)) if A.variant_fits(op, v, width)]


def run_rms(x, w, eps, variant=-1):
    announce("rmsnorm", x.shape, "eps", eps, "variant", variant)
    out = A.rmsnorm(bf16(x), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(out)


def run_rms_fp8(x, w, eps, variant=-1):
    announce("rmsnorm_quant_fp8", x.shape, "eps", eps, "variant", variant)
    q, s = A.rmsnorm_quant_fp8(bf16(x), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


def run_rms_static(x, w, eps, scale, variant=-1):
    announce("rmsnorm_quant_fp8_static", x.shape, "eps", eps, "scale", scale, "variant", variant)
    q = A.rmsnorm_quant_fp8_static(bf16(x), bf16(w), scale_t(scale), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q)


def run_fused_static(x, r, w, eps, scale, variant=-1):
    announce("fused_add_rmsnorm_quant_fp8_static", x.shape, "eps", eps, "scale", scale, "variant", variant)
    q, ro = A.fused_add_rmsnorm_quant_fp8_static(bf16(x), bf16(r), bf16(w), scale_t(scale), eps,
                                                 variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(ro)


def run_swiglu_dyn(gu, variant=-1):
    announce("swiglu_quant_fp8_dynamic", gu.shape, "variant", variant)
    q, s = A.swiglu_quant_fp8_dynamic(bf16(gu), variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


# ------------------------------------------------------------------ rmsnorm

@pytest.mark.parametrize("T,H", [(1, 8), (3, 24), (16, 1536), (257, 1536), (4, 16384), (3, 16392),
                                 (1, 65536), (1023, 1536), (1024, 1536)])
def test_rmsnorm_shapes_default_variant(T, H):
    x, _, w = norm_case(T, H, seed=T * 7 + H)
    announce(P.check_rmsnorm(x, w, 1e-6, run_rms(x, w, 1e-6)))


@pytest.mark.parametrize("H", [1536, 16384])
def test_rmsnorm_forms_every_variant(H):
    T = 37
    x, _, w = norm_case(T, H, seed=H + 1, outliers=0.001)
    for v in variants_for(A.OP_NORM, H):
        P.check_rmsnorm(x, w, 1e-5, run_rms(x, w, 1e-5, v))
        q, s = run_rms_fp8(x, w, 1e-5, v)
        P.check_rmsnorm_fp8(x, w, 1e-5, q, s)
        P.check_rmsnorm_fp8_static(x, w, 1e-5, 0.0125, run_rms_static(x, w, 1e-5, 0.0125, v))


def test_rmsnorm_closed_forms_and_in_place():
    H = 1536
    w = gen.normal_bf16((H,), 0, 3, mean=1.0, std=0.1)
    x = np.full((4, H), oracle.bf16_from_f64(0.75), np.uint16)
    x[1] ^= 0x8000
    x[2] = 0
    x[3] = gen.normal_bf16((H,), 1, 1)
    x[3, :5] = 0x8000                                  # -0 stays -0: out = w * -0
    out = run_rms(x, w, 1e-6)
    assert np.array_equal(out[0], w) and np.array_equal(out[1], w ^ 0x8000)
    assert np.all(oracle.bf16_to_f32(out[2]) == 0)
    assert np.all(out[3, :5] == np.where(oracle.bf16_to_f32(w[:5]) > 0, 0x8000, 0))
    P.check_rmsnorm(x, w, 1e-6, out)
    # in place
    xr, _, _ = norm_case(64, H, seed=3)
    xt = bf16(xr)
    announce("rmsnorm in place", xr.shape)
    A.rmsnorm(xt, bf16(w), 1e-6, out=xt)
    torch.cuda.synchronize()
    P.check_rmsnorm(xr, w, 1e-6, bits(xt))


def test_rmsnorm_prefill4096_full():
    wl = W.NORM_PREFILL4096
    d = W.norm_inputs(wl)
    announce(P.check_rmsnorm(d["x"], d["weight"], wl.eps, run_rms(d["x"], d["weight"], wl.eps)))


def test_rmsnorm_fp8_dynamic_edge_rows():
    H = 16384
    x, _, w = norm_case(6, H, seed=21)
    x[0] = 0                                           # all-zero row: s = 0, q = 0
    x[1] = oracle.bf16_from_f64(0.5)                   # constant row
    x[2] = oracle.bf16_from_f64(1e-3)
    x[2, 7] = oracle.bf16_from_f64(300.0)              # one outlier
    q, s = run_rms_fp8(x, w, 1e-5)
    P.check_rmsnorm_fp8(x, w, 1e-5, q, s)
    assert s[0] == 0 and np.all((q[0] & 0x7F) == 0)
    assert q[2, 7] in (0x7E, 0xFE)
    dec = oracle.e4m3_table()
    assert np.all(np.abs(dec[q[1:]]).max(axis=1) == 448.0)


# ------------------------------------------------------------------ static norm + fp8

@pytest.mark.parametrize("scale", SCALES)
def test_static_norm_fp8_scales(scale):
    """Per-tensor scales on both sides of the fast quotient's range, one that
    saturates (|y| reaches about 4, 448 * 0.0125 = 5.6 is passed by the
    outliers), and zero (treated as one)."""
    x, r, w = norm_case(64, 4096, seed=22, outliers=0.002)
    q, ro = run_fused_static(x, r, w, 1e-5, scale)
    announce(P.check_norm_fp8_static(x, r, w, 1e-5, scale, q, ro))
    q2 = run_rms_static(x, w, 1e-5, scale)
    announce(P.check_rmsnorm_fp8_static(x, w, 1e-5, scale, q2))


def test_static_norm_fp8_every_variant():
    T, H = 37, 16384
    x, r, w = norm_case(T, H, seed=23, outliers=0.001)
    for v in variants_for(A.OP_NORM, H):
        q, ro = run_fused_static(x, r, w, 1e-5, 0.02, v)
        P.check_norm_fp8_static(x, r, w, 1e-5, 0.02, q, ro)


def test_static_norm_fp8_in_place_residual():
    x, r, w = norm_case(32, 2048, seed=24)
    rt = bf16(r)
    announce("fused_add_rmsnorm_quant_fp8_static residual in place", x.shape)
    q, ro = A.fused_add_rmsnorm_quant_fp8_static(bf16(x), rt, bf16(w), scale_t(0.05), 1e-5,
                                                 residual_out=rt)
    torch.cuda.synchronize()
    P.check_norm_fp8_static(x, r, w, 1e-5, 0.05, bits(q), bits(rt))


def test_static_norm_fp8_llama405b_full():
    wl = W.NORM_FP8_LLAMA405B
    d = W.norm_inputs(wl)
    q, ro = run_fused_static(d["x"], d["residual"], d["weight"], wl.eps, 0.02)
    announce(P.check_norm_fp8_static(d["x"], d["residual"], d["weight"], wl.eps, 0.02, q, ro))


# ------------------------------------------------------------------ per-token swiglu + fp8

@pytest.mark.parametrize("T,N", [(1, 8), (3, 24), (5, 1032), (64, 8960), (7, 28672), (2, 65536)])
def test_swiglu_dynamic_shapes_every_variant(T, N):
    gu = gen.normal_bf16((T, 2 * N), T + 3 * N, 4, std=2.0)
    for v in [-1] + variants_for(A.OP_SWIGLU_DYNAMIC, N):
        q, s = run_swiglu_dyn(gu, v)
        P.check_swiglu_fp8_dynamic(gu, q, s)


def test_swiglu_dynamic_edge_rows():
    T, N = 8, 8960
    gu = gen.normal_bf16((T, 2 * N), 31, 4, std=2.0)
    gu[0, :N] = 0                                      # gate 0: y = +-0, s = 0, codes zero
    gu[1, :N] = oracle.bf16_from_f64(0.01)             # small row with one large output
    gu[1, 100] = oracle.bf16_from_f64(12.0)
    gu[1, N + 100] = oracle.bf16_from_f64(5.0)
    gu[2, 17] = 0x7FC0                                 # a NaN gate: its code is NaN, amax ignores it
    gu[3, N + 5] = 0x7F80                              # an infinite up: s = inf
    gu[4, :N] = gen.normal_bf16((N,), 32, 1, std=30.0)  # gates past -16 take the exact SiLU
    q, s = run_swiglu_dyn(gu)
    P.check_swiglu_fp8_dynamic(gu, q, s)
    assert s[0] == 0 and np.all((q[0] & 0x7F) == 0)
    assert q[1, 100] == 0x7E
    assert q[2, 17] in (0x7F, 0xFF)
    dec = oracle.e4m3_table()
    assert np.abs(dec[q[5]]).max() == 448.0


def test_swiglu_dynamic_every_y():
    """gate = 8 (a = 8 exactly) and up = bf16 patterns of one binade range per
    row, so y = 8u sweeps every significand through the per-token scale."""
    N = 65536
    u = np.arange(N, dtype=np.uint16)
    finite = (u & 0x7F80) != 0x7F80
    rows = []
    for hi_exp in (0x3F80, 0x4700, 0x1000):
        uu = np.where(finite & ((u & 0x7F80) <= hi_exp), u, u & 0x807F)
        rows.append(np.concatenate([np.full(N, oracle.bf16_from_f64(8.0), np.uint16), uu]))
    gu = np.stack(rows)
    q, s = run_swiglu_dyn(gu)
    P.check_swiglu_fp8_dynamic(gu, q, s)


def test_swiglu_dynamic_llama70b_full():
    wl = W.SWIGLU_FP8_LLAMA70B
    gu = W.swiglu_inputs(wl)["gate_up"]
    q, s = run_swiglu_dyn(gu)
    P.check_swiglu_fp8_dynamic(gu, q, s)
    dec = oracle.e4m3_table()
    assert np.all(np.abs(dec[q]).max(axis=1) == 448.0)


# ------------------------------------------------------------------ MXFP4 norms

def run_fused_mx(x, r, w, eps, variant=-1):
    announce("fused_add_rmsnorm_quant_mxfp4", x.shape, "eps", eps, "variant", variant)
    q, s, ro = A.fused_add_rmsnorm_quant_mxfp4(bf16(x), bf16(r), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s), bits(ro)


def run_rms_mx(x, w, eps, variant=-1):
    announce("rmsnorm_quant_mxfp4", x.shape, "eps", eps, "variant", variant)
    q, s = A.rmsnorm_quant_mxfp4(bf16(x), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


@pytest.mark.parametrize("T,H", [(1, 32), (3, 96), (16, 1536), (257, 1536), (4, 16384), (2, 65536),
                                 (1023, 2048)])
def test_mxfp4_norms_default_variant(T, H):
    x, r, w = norm_case(T, H, seed=T + 5 * H, outliers=0.002)
    q, s, ro = run_fused_mx(x, r, w, 1e-5)
    announce(P.check_norm_mxfp4(x, r, w, 1e-5, q, s, ro))
    q, s = run_rms_mx(x, w, 1e-5)
    announce(P.check_rmsnorm_mxfp4(x, w, 1e-5, q, s))


@pytest.mark.parametrize("H", [1536, 16384])
def test_mxfp4_norms_every_variant(H):
    x, r, w = norm_case(37, H, seed=H + 9, outliers=0.002)
    for v in variants_for(A.OP_NORM, H):
        q, s, ro = run_fused_mx(x, r, w, 1e-5, v)
        P.check_norm_mxfp4(x, r, w, 1e-5, q, s, ro)
        q, s = run_rms_mx(x, w, 1e-5, v)
        P.check_rmsnorm_mxfp4(x, w, 1e-5, q, s)


def test_mxfp4_special_blocks():
    """An all-zero block, blocks whose amax is an exact power of two, a block
    of bf16-subnormal values (the smallest scale), one holding a NaN and one
    an infinity (scale 0xFF, zero codes)."""
    H = 256
    x, _, w = norm_case(6, H, seed=77)
    w[:] = oracle.bf16_from_f64(1.0)
    one = oracle.bf16_from_f64
    x[0, :32] = 0                                   # zero block, rest normal
    x[1, :] = one(0.5)
    x[1, 32:64] = one(1.0)                          # amax exact powers of two after the norm
    x[2, :] = one(1.0)
    x[2, 64:96] = 0x0001                            # bf16 subnormals beside 1.0: y tiny
    x[3, 100] = 0x7FC0                              # NaN: the whole row's norm is NaN
    x[4, 7] = 0x7F80                                # +inf
    q, s = run_rms_mx(x, w, 1e-6)
    P.check_rmsnorm_mxfp4(x, w, 1e-6, q, s)
    assert s[0, 0] == 0 and np.all((q[0, :16] & 0x77) == 0)
    assert np.all(s[3] == 0xFF) and np.all(q[3] == 0)


def test_mxfp4_norm_llama405b_full():
    wl = W.NORM_FP8_LLAMA405B
    d = W.norm_inputs(wl)
    q, s, ro = run_fused_mx(d["x"], d["residual"], d["weight"], wl.eps)
    announce(P.check_norm_mxfp4(d["x"], d["residual"], d["weight"], wl.eps, q, s, ro))
    assert np.isfinite(oracle.mxfp4_decode(q, s)).all()


# ------------------------------------------------------------------ graph capture

def test_quant_matrix_forms_under_graph_replay():
    """Every form launched from a captured HIP graph, replayed three times
    with eager work in between: each replay's outputs equal the eager ones
    bitwise (nothing in the forms allocates, synchronizes or clears memory)."""
    T, H, N = 64, 2048, 2048
    x, r, w = norm_case(T, H, seed=91, outliers=0.001)
    gu = gen.normal_bf16((T, 2 * N), 92, 4, std=2.0)
    xt, rt, wt, gut, sc = bf16(x), bf16(r), bf16(w), bf16(gu), scale_t(0.03)
    outs = dict(
        rms=torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
        rq=torch.empty((T, H), dtype=torch.uint8, device=DEV), rs=torch.empty((T,), device=DEV),
        st=torch.empty((T, H), dtype=torch.uint8, device=DEV), sro=torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
        mq=torch.empty((T, H // 2), dtype=torch.uint8, device=DEV), ms=torch.empty((T, H // 32), dtype=torch.uint8, device=DEV),
        mro=torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
        dq=torch.empty((T, N), dtype=torch.uint8, device=DEV), ds=torch.empty((T,), device=DEV))

    def launch():
        A.rmsnorm(xt, wt, 1e-5, out=outs["rms"])
        A.rmsnorm_quant_fp8(xt, wt, 1e-5, out=outs["rq"], scale_out=outs["rs"])
        A.fused_add_rmsnorm_quant_fp8_static(xt, rt, wt, sc, 1e-5, out=outs["st"], residual_out=outs["sro"])
        A.fused_add_rmsnorm_quant_mxfp4(xt, rt, wt, 1e-5, out=outs["mq"], scale_out=outs["ms"],
                                        residual_out=outs["mro"])
        A.swiglu_quant_fp8_dynamic(gut, out=outs["dq"], scale_out=outs["ds"])

    announce("quant-matrix forms, eager then graph")
    launch()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k].view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
        xt.add_(0)                                     # eager work between replays
    P.check_rmsnorm(x, w, 1e-5, bits(outs["rms"]))
    P.check_norm_mxfp4(x, r, w, 1e-5, bits(outs["mq"]), bits(outs["ms"]), bits(outs["mro"]))


# ------------------------------------------------------------------ MXFP4 swiglu

def run_swiglu_mx(gu, variant=-1):
    announce("swiglu_quant_mxfp4", gu.shape, "variant", variant)
    q, s = A.swiglu_quant_mxfp4(bf16(gu), variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


@pytest.mark.parametrize("T,N", [(1, 32), (3, 96), (5, 1056), (64, 8960), (300, 8960), (7, 28672)])
def test_swiglu_mxfp4_shapes_every_variant(T, N):
    gu = gen.normal_bf16((T, 2 * N), T + 7 * N, 4, std=2.0)
    for v in [-1] + list(range(A.variant_count(A.OP_SWIGLU))):
        q, s = run_swiglu_mx(gu, v)
        P.check_swiglu_mxfp4(gu, q, s)


def test_swiglu_mxfp4_special_blocks_and_every_y():
    N = 65536
    u = np.arange(N, dtype=np.uint16)
    finite = (u & 0x7F80) != 0x7F80
    rows = []
    for hi_exp in (0x3F80, 0x4700, 0x1000):            # y = 8u over several binade ranges
        uu = np.where(finite & ((u & 0x7F80) <= hi_exp), u, u & 0x807F)
        rows.append(np.concatenate([np.full(N, oracle.bf16_from_f64(8.0), np.uint16), uu]))
    gu = np.stack(rows + [rows[0].copy(), rows[0].copy()])
    gu[3, 40] = 0x7FC0                                 # NaN gate: its block gets 0xFF
    gu[4, N + 70] = 0x7F80                             # infinite up
    gu[4, :32] = 0                                     # a zero block
    for v in (-1, 0, 3):
        q, s = run_swiglu_mx(gu, v)
        P.check_swiglu_mxfp4(gu, q, s)
        assert s[3, 1] == 0xFF and s[4, 2] == 0xFF


def test_swiglu_mxfp4_llama70b_full():
    wl = W.SWIGLU_FP8_LLAMA70B
    gu = W.swiglu_inputs(wl)["gate_up"]
    q, s = run_swiglu_mx(gu)
    P.check_swiglu_mxfp4(gu, q, s)


# ------------------------------------------------------------------ NVFP4

NV_SCALES = [0.02, 1.0, 3.0e-4, 0.0, 2.0 ** -120, 1.0e6]


def run_fused_nv(x, r, w, eps, g, variant=-1):
    announce("fused_add_rmsnorm_quant_nvfp4", x.shape, "g", g, "variant", variant)
    q, s, ro = A.fused_add_rmsnorm_quant_nvfp4(bf16(x), bf16(r), bf16(w), scale_t(g), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s), bits(ro)


def run_rms_nv(x, w, eps, g, variant=-1):
    announce("rmsnorm_quant_nvfp4", x.shape, "g", g, "variant", variant)
    q, s = A.rmsnorm_quant_nvfp4(bf16(x), bf16(w), scale_t(g), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


def run_swiglu_nv(gu, g, variant=-1):
    announce("swiglu_quant_nvfp4", gu.shape, "g", g, "variant", variant)
    q, s = A.swiglu_quant_nvfp4(bf16(gu), scale_t(g), variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


@pytest.mark.parametrize("g", NV_SCALES)
def test_nvfp4_norms_tensor_scales(g):
    """Tensor scales from ordinary ones to g = 2^-120 (amax / 6g far past
    448: every block scale saturates) and g = 1e6 (block scales underflow to
    zero: signed-zero codes), and zero (treated as one)."""
    x, r, w = norm_case(48, 2048, seed=61, outliers=0.002)
    q, s, ro = run_fused_nv(x, r, w, 1e-5, g)
    announce(P.check_norm_nvfp4(x, r, w, 1e-5, g, q, s, ro))
    q, s = run_rms_nv(x, w, 1e-5, g)
    announce(P.check_rmsnorm_nvfp4(x, w, 1e-5, g, q, s))


@pytest.mark.parametrize("H", [1536, 16384])
def test_nvfp4_norms_every_variant(H):
    x, r, w = norm_case(37, H, seed=H + 13, outliers=0.002)
    for v in variants_for(A.OP_NORM, H):
        q, s, ro = run_fused_nv(x, r, w, 1e-5, 0.02, v)
        P.check_norm_nvfp4(x, r, w, 1e-5, 0.02, q, s, ro)
        q, s = run_rms_nv(x, w, 1e-5, 0.02, v)
        P.check_rmsnorm_nvfp4(x, w, 1e-5, 0.02, q, s)


@pytest.mark.parametrize("T,H", [(1, 16), (3, 48), (1023, 1536), (2, 65536)])
def test_nvfp4_norm_shapes(T, H):
    x, r, w = norm_case(T, H, seed=T + 3 * H)
    q, s, ro = run_fused_nv(x, r, w, 1e-6, 0.01)
    P.check_norm_nvfp4(x, r, w, 1e-6, 0.01, q, s, ro)


def test_nvfp4_norm_llama405b_full():
    wl = W.NORM_FP8_LLAMA405B
    d = W.norm_inputs(wl)
    q, s, ro = run_fused_nv(d["x"], d["residual"], d["weight"], wl.eps, 0.02)
    announce(P.check_norm_nvfp4(d["x"], d["residual"], d["weight"], wl.eps, 0.02, q, s, ro))


@pytest.mark.parametrize("T,N", [(1, 16), (3, 48), (5, 1040), (64, 8960), (300, 8960), (7, 28672)])
def test_swiglu_nvfp4_shapes_every_variant(T, N):
    gu = gen.normal_bf16((T, 2 * N), T + 11 * N, 4, std=2.0)
    for v in [-1] + list(range(A.variant_count(A.OP_SWIGLU))):
        q, s = run_swiglu_nv(gu, 0.05, v)
        P.check_swiglu_nvfp4(gu, 0.05, q, s)


def test_swiglu_nvfp4_scales_and_special_blocks():
    N = 65536
    u = np.arange(N, dtype=np.uint16)
    finite = (u & 0x7F80) != 0x7F80
    uu = np.where(finite & ((u & 0x7F80) <= 0x4700), u, u & 0x807F)
    row = np.concatenate([np.full(N, oracle.bf16_from_f64(8.0), np.uint16), uu])
    gu = np.stack([row, row.copy(), row.copy()])
    gu[1, 40] = 0x7FC0                                 # NaN gate: its block gets 0x7F
    gu[2, N + 70] = 0x7F80                             # infinite up
    gu[2, :16] = 0                                     # a zero block
    for g in NV_SCALES:
        for v in (-1, 0, 3):
            q, s = run_swiglu_nv(gu, g, v)
            P.check_swiglu_nvfp4(gu, g, q, s)
            assert s[1, 2] == 0x7F and s[2, 4] == 0x7F


def test_swiglu_nvfp4_llama70b_full():
    wl = W.SWIGLU_FP8_LLAMA70B
    gu = W.swiglu_inputs(wl)["gate_up"]
    q, s = run_swiglu_nv(gu, 0.05)
    P.check_swiglu_nvfp4(gu, 0.05, q, s)


# ------------------------------------------------------------------ per-group E4M3

def run_fused_grp(x, r, w, eps, variant=-1):
    announce("fused_add_rmsnorm_quant_fp8_group", x.shape, "eps", eps, "variant", variant)
    q, s, ro = A.fused_add_rmsnorm_quant_fp8_group(bf16(x), bf16(r), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s), bits(ro)


def run_rms_grp(x, w, eps, variant=-1):
    announce("rmsnorm_quant_fp8_group", x.shape, "eps", eps, "variant", variant)
    q, s = A.rmsnorm_quant_fp8_group(bf16(x), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


def run_swiglu_grp(gu, variant=-1):
    announce("swiglu_quant_fp8_group", gu.shape, "variant", variant)
    q, s = A.swiglu_quant_fp8_group(bf16(gu), variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s)


@pytest.mark.parametrize("T,H", [(1, 128), (3, 384), (16, 1536), (257, 1536), (4, 16384), (3, 16512),
                                 (2, 65536), (1023, 2048)])
def test_fp8_group_norms_default_variant(T, H):
    x, r, w = norm_case(T, H, seed=T + 17 * H, outliers=0.002)
    q, s, ro = run_fused_grp(x, r, w, 1e-5)
    announce(P.check_norm_fp8_group(x, r, w, 1e-5, q, s, ro))
    q, s = run_rms_grp(x, w, 1e-5)
    announce(P.check_rmsnorm_fp8_group(x, w, 1e-5, q, s))


@pytest.mark.parametrize("H", [1536, 16384])
def test_fp8_group_norms_every_variant(H):
    x, r, w = norm_case(37, H, seed=H + 19, outliers=0.002)
    for v in variants_for(A.OP_NORM, H):
        q, s, ro = run_fused_grp(x, r, w, 1e-5, v)
        P.check_norm_fp8_group(x, r, w, 1e-5, q, s, ro)
        q, s = run_rms_grp(x, w, 1e-5, v)
        P.check_rmsnorm_fp8_group(x, w, 1e-5, q, s)


def test_fp8_group_norm_special_groups():
    """An all-zero group (scale 0, zero codes), a group of bf16 subnormals
    beside groups near 1 (a tiny scale of its own), an outlier that only
    its own group's scale sees, a NaN (the whole row's norm is NaN: the
    maxima ignore it, scale 0, NaN codes) and an infinity."""
    H = 512
    x, _, w = norm_case(6, H, seed=78)
    w[:] = oracle.bf16_from_f64(1.0)
    one = oracle.bf16_from_f64
    x[0, :128] = 0
    x[1, :] = one(1.0)
    x[1, 256:384] = 0x0001
    x[2, 300] = one(200.0)
    x[3, 100] = 0x7FC0
    x[4, 7] = 0x7F80
    for v in variants_for(A.OP_NORM, H):
        q, s = run_rms_grp(x, w, 1e-6, v)
        P.check_rmsnorm_fp8_group(x, w, 1e-6, q, s)
        assert s[0, 0] == 0 and np.all((q[0, :128] & 0x7F) == 0)
        assert 0 < s[1, 2] < 1e-30 and s[1, 0] == s[1, 1] == s[1, 3]
        assert s[2, 2] > 10 * max(s[2, 0], s[2, 1], s[2, 3])
        assert np.all(s[3] == 0) and np.all(np.isin(q[3], [0x7F, 0xFF]))


def test_fp8_group_norm_in_place_residual():
    x, r, w = norm_case(32, 2048, seed=25)
    rt = bf16(r)
    announce("fused_add_rmsnorm_quant_fp8_group residual in place", x.shape)
    q, s, ro = A.fused_add_rmsnorm_quant_fp8_group(bf16(x), rt, bf16(w), 1e-5, residual_out=rt)
    torch.cuda.synchronize()
    assert ro.data_ptr() == rt.data_ptr()
    P.check_norm_fp8_group(x, r, w, 1e-5, bits(q), bits(s), bits(rt))


def test_fp8_group_norm_llama405b_full():
    wl = W.NORM_FP8_LLAMA405B
    d = W.norm_inputs(wl)
    q, s, ro = run_fused_grp(d["x"], d["residual"], d["weight"], wl.eps)
    announce(P.check_norm_fp8_group(d["x"], d["residual"], d["weight"], wl.eps, q, s, ro))
    dec = oracle.e4m3_table()
    amax = np.abs(dec[q]).reshape(q.shape[0], -1, A.FP8_GROUP).max(axis=2)
    assert np.all(amax == 448.0)


@pytest.mark.parametrize("T,N", [(1, 128), (3, 384), (5, 1152), (64, 8960), (300, 8960), (600, 8960),
                                 (7, 28672), (2, 65536)])
def test_swiglu_fp8_group_shapes_every_variant(T, N):
    gu = gen.normal_bf16((T, 2 * N), T + 13 * N, 4, std=2.0)
    for v in [-1] + list(range(A.variant_count(A.OP_SWIGLU))):
        q, s = run_swiglu_grp(gu, v)
        P.check_swiglu_fp8_group(gu, q, s)


def test_swiglu_fp8_group_special_groups_and_every_y():
    """y = 8u over several binade ranges (every bf16 significand passes
    through a group scale), a NaN gate (its code NaN, the group maximum
    ignores it), an infinite up (scale inf) and an all-zero group."""
    N = 65536
    u = np.arange(N, dtype=np.uint16)
    finite = (u & 0x7F80) != 0x7F80
    rows = []
    for hi_exp in (0x3F80, 0x4700, 0x1000):
        uu = np.where(finite & ((u & 0x7F80) <= hi_exp), u, u & 0x807F)
        rows.append(np.concatenate([np.full(N, oracle.bf16_from_f64(8.0), np.uint16), uu]))
    gu = np.stack(rows + [rows[0].copy(), rows[0].copy()])
    gu[3, 140] = 0x7FC0
    gu[4, N + 300] = 0x7F80
    gu[4, :128] = 0
    for v in [-1] + list(range(A.variant_count(A.OP_SWIGLU))):
        q, s = run_swiglu_grp(gu, v)
        P.check_swiglu_fp8_group(gu, q, s)
        assert q[3, 140] in (0x7F, 0xFF) and np.isfinite(s[3, 1])
        assert np.isinf(s[4, 2]) and s[4, 0] == 0 and np.all((q[4, :128] & 0x7F) == 0)


def test_swiglu_fp8_group_llama70b_full():
    wl = W.SWIGLU_FP8_LLAMA70B
    gu = W.swiglu_inputs(wl)["gate_up"]
    q, s = run_swiglu_grp(gu)
    P.check_swiglu_fp8_group(gu, q, s)


def test_fp8_group_forms_under_graph_replay():
    """The three per-group forms from one captured graph, replayed three
    times with eager work between: every replay equals the eager run."""
    T, H, N = 64, 2048, 2048
    x, r, w = norm_case(T, H, seed=93, outliers=0.001)
    gu = gen.normal_bf16((T, 2 * N), 94, 4, std=2.0)
    xt, rt, wt, gut = bf16(x), bf16(r), bf16(w), bf16(gu)
    u8 = dict(dtype=torch.uint8, device=DEV)
    outs = dict(fq=torch.empty((T, H), **u8), fs=torch.empty((T, H // 128), device=DEV),
                fro=torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
                rq=torch.empty((T, H), **u8), rs=torch.empty((T, H // 128), device=DEV),
                sq=torch.empty((T, N), **u8), ss=torch.empty((T, N // 128), device=DEV))

    def launch():
        A.fused_add_rmsnorm_quant_fp8_group(xt, rt, wt, 1e-5, out=outs["fq"], scale_out=outs["fs"],
                                            residual_out=outs["fro"])
        A.rmsnorm_quant_fp8_group(xt, wt, 1e-5, out=outs["rq"], scale_out=outs["rs"])
        A.swiglu_quant_fp8_group(gut, out=outs["sq"], scale_out=outs["ss"])

    announce("per-group forms, eager then graph")
    launch()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k].view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
        xt.add_(0)
    P.check_norm_fp8_group(x, r, w, 1e-5, bits(outs["fq"]), bits(outs["fs"]), bits(outs["fro"]))
    P.check_swiglu_fp8_group(gu, bits(outs["sq"]), bits(outs["ss"]))


# ------------------------------------------------------------------ seeded random shapes

def _random_shapes(n, seed):
    rng = np.random.default_rng([2024, seed])
    out = []
    for _ in range(n):
        T = int(rng.integers(1, 300))
        W = 8 * int(rng.integers(1, 1025))          # 8 .. 8,192, any multiple of 8
        if rng.random() < 0.3:
            W = 128 * int(rng.integers(1, 65))      # whole 128-value groups
        out.append((T, W))
    return out


@pytest.mark.parametrize("T,H", _random_shapes(24, 1))
def test_random_shapes_every_norm_form(T, H):
    x, r, w = norm_case(T, H, seed=T * 131 + H, outliers=0.002)
    xt, rt, wt = bf16(x), bf16(r), bf16(w)
    g = scale_t(0.02)
    announce("norm forms", (T, H))
    out, ro = A.fused_add_rmsnorm(xt, rt, wt, 1e-5)
    P.check_norm(x, r, w, 1e-5, bits(out), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8(xt, rt, wt, 1e-5)
    P.check_norm_fp8(x, r, w, 1e-5, bits(q), bits(s), bits(ro))
    q, ro = A.fused_add_rmsnorm_quant_fp8_static(xt, rt, wt, g, 1e-5)
    P.check_norm_fp8_static(x, r, w, 1e-5, 0.02, bits(q), bits(ro))
    P.check_rmsnorm(x, w, 1e-5, bits(A.rmsnorm(xt, wt, 1e-5)))
    q, s = A.rmsnorm_quant_fp8(xt, wt, 1e-5)
    P.check_rmsnorm_fp8(x, w, 1e-5, bits(q), bits(s))
    if H % 16 == 0:
        q, s, ro = A.fused_add_rmsnorm_quant_nvfp4(xt, rt, wt, g, 1e-5)
        P.check_norm_nvfp4(x, r, w, 1e-5, 0.02, bits(q), bits(s), bits(ro))
    if H % 32 == 0:
        q, s, ro = A.fused_add_rmsnorm_quant_mxfp4(xt, rt, wt, 1e-5)
        P.check_norm_mxfp4(x, r, w, 1e-5, bits(q), bits(s), bits(ro))
    if H % A.FP8_GROUP == 0:
        q, s, ro = A.fused_add_rmsnorm_quant_fp8_group(xt, rt, wt, 1e-5)
        P.check_norm_fp8_group(x, r, w, 1e-5, bits(q), bits(s), bits(ro))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,N", _random_shapes(24, 2))
def test_random_shapes_every_swiglu_form(T, N):
    gu = gen.normal_bf16((T, 2 * N), T * 137 + N, 4, std=2.0)
    gt = bf16(gu)
    s = scale_t(0.05)
    announce("swiglu forms", (T, N))
    P.check_swiglu(gu, bits(A.swiglu(gt)))
    P.check_swiglu_fp8(gu, 0.05, bits(A.swiglu_quant_fp8(gt, s)))
    q, sc = A.swiglu_quant_fp8_dynamic(gt)
    P.check_swiglu_fp8_dynamic(gu, bits(q), bits(sc))
    if N % 16 == 0:
        q, sc = A.swiglu_quant_nvfp4(gt, s)
        P.check_swiglu_nvfp4(gu, 0.05, bits(q), bits(sc))
    if N % 32 == 0:
        q, sc = A.swiglu_quant_mxfp4(gt)
        P.check_swiglu_mxfp4(gu, bits(q), bits(sc))
    if N % A.FP8_GROUP == 0:
        q, sc = A.swiglu_quant_fp8_group(gt)
        P.check_swiglu_fp8_group(gu, bits(q), bits(sc))
    torch.cuda.synchronize()


def _large_shapes(n, seed, max_width, max_outputs, whole_blocks):
    """Seeded shapes from a few hundred tokens up, where the default picks
    change with the token count and width (two jobs per lane, pipelined and
    few-wave norms, more waves per row): tokens x width between about two
    million and `max_outputs`; with probability 0.4 a width that is a
    multiple of `whole_blocks`."""
    rng = np.random.default_rng([2025, seed])
    out = []
    for _ in range(n):
        if rng.random() < 0.4:
            W = whole_blocks * int(rng.integers(1, max_width // whole_blocks + 1))
        else:
            W = 8 * int(rng.integers(64, max_width // 8 + 1))
        lo = max(1, (2 << 20) // W)
        hi = max(lo + 1, max_outputs // W)
        out.append((int(rng.integers(lo, hi)), W))
    return out


@pytest.mark.parametrize("T,H", _large_shapes(8, 1, 16384, 24 << 20, 2048))
def test_large_random_shapes_every_norm_form(T, H):
    x, r, w = norm_case(T, H, seed=T * 7 + H, outliers=0.001)
    xt, rt, wt = bf16(x), bf16(r), bf16(w)
    g = scale_t(0.02)
    announce("norm forms", (T, H), A.variant_name(A.OP_NORM, A.pick_variant(A.OP_NORM, T, H, 0)),
             A.variant_name(A.OP_NORM, A.pick_variant(A.OP_NORM, T, H, 1)))
    out, ro = A.fused_add_rmsnorm(xt, rt, wt, 1e-6)
    P.check_norm(x, r, w, 1e-6, bits(out), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8(xt, rt, wt, 1e-6)
    P.check_norm_fp8(x, r, w, 1e-6, bits(q), bits(s), bits(ro))
    q, ro = A.fused_add_rmsnorm_quant_fp8_static(xt, rt, wt, g, 1e-6)
    P.check_norm_fp8_static(x, r, w, 1e-6, 0.02, bits(q), bits(ro))
    P.check_rmsnorm(x, w, 1e-6, bits(A.rmsnorm(xt, wt, 1e-6)))
    q, s = A.rmsnorm_quant_fp8(xt, wt, 1e-6)
    P.check_rmsnorm_fp8(x, w, 1e-6, bits(q), bits(s))
    if H % 16 == 0:
        q, s, ro = A.fused_add_rmsnorm_quant_nvfp4(xt, rt, wt, g, 1e-6)
        P.check_norm_nvfp4(x, r, w, 1e-6, 0.02, bits(q), bits(s), bits(ro))
    if H % 32 == 0:
        q, s, ro = A.fused_add_rmsnorm_quant_mxfp4(xt, rt, wt, 1e-6)
        P.check_norm_mxfp4(x, r, w, 1e-6, bits(q), bits(s), bits(ro))
    if H % A.FP8_GROUP == 0:
        q, s, ro = A.fused_add_rmsnorm_quant_fp8_group(xt, rt, wt, 1e-6)
        P.check_norm_fp8_group(x, r, w, 1e-6, bits(q), bits(s), bits(ro))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,N", _large_shapes(8, 2, 28672, 48 << 20, 4096))
def test_large_random_shapes_every_swiglu_form(T, N):
    gu = gen.normal_bf16((T, 2 * N), T * 11 + N, 4, std=2.0)
    gt = bf16(gu)
    s = scale_t(0.05)
    announce("swiglu forms", (T, N), *(A.variant_name(A.OP_SWIGLU, A.pick_variant(A.OP_SWIGLU, T, N, f))
                                      for f in range(5)))
    P.check_swiglu(gu, bits(A.swiglu(gt)))
    P.check_swiglu_fp8(gu, 0.05, bits(A.swiglu_quant_fp8(gt, s)))
    q, sc = A.swiglu_quant_fp8_dynamic(gt)
    P.check_swiglu_fp8_dynamic(gu, bits(q), bits(sc))
    if N % 16 == 0:
        q, sc = A.swiglu_quant_nvfp4(gt, s)
        P.check_swiglu_nvfp4(gu, 0.05, bits(q), bits(sc))
    if N % 32 == 0:
        q, sc = A.swiglu_quant_mxfp4(gt)
        P.check_swiglu_mxfp4(gu, bits(q), bits(sc))
    if N % A.FP8_GROUP == 0:
        q, sc = A.swiglu_quant_fp8_group(gt)
        P.check_swiglu_fp8_group(gu, bits(q), bits(sc))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,H", [(256, 16384), (512, 16384), (1024, 4096)])
def test_fused_quant_forms_one_generation_late_residual(T, H):
    """Launches whose blocks are all resident at once and that read 12 MB or
    more: there the quantised forms store the updated residual in the
    epilogue, after its last use, instead of right after the add.  Every
    quantised form with the residual add, default variant, against the
    oracle (residual bit-exact, codes and scales to the usual bar)."""
    x, r, w = norm_case(T, H, seed=T + H, outliers=0.001)
    eps = 1e-5
    announce("fused_add_rmsnorm_quant_fp8 one generation", (T, H))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8(bf16(x), bf16(r), bf16(w), eps)
    torch.cuda.synchronize()
    P.check_norm_fp8(x, r, w, eps, bits(q), bits(s), bits(ro))
    q, ro = run_fused_static(x, r, w, eps, 0.02)
    P.check_norm_fp8_static(x, r, w, eps, 0.02, q, ro)
    q, s, ro = run_fused_mx(x, r, w, eps)
    P.check_norm_mxfp4(x, r, w, eps, q, s, ro)
    q, s, ro = run_fused_nv(x, r, w, eps, 0.02)
    P.check_norm_nvfp4(x, r, w, eps, 0.02, q, s, ro)
    q, s, ro = run_fused_grp(x, r, w, eps)
    P.check_norm_fp8_group(x, r, w, eps, q, s, ro)
