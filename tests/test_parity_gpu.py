"""GPU parity: the HIP kernels, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Bar: the updated residual bit-exact; the norm output equal to an admissible
oracle value (tests/parity.py: bit-exact except at reduction-order
knife-edges); SwiGLU and its static FP8 form bit-exact (the SiLU is correctly
rounded on both sides); dynamic FP8 bit-exact, with the stated tolerances
(scales 1e-6 relative, codes 1 E4M3 ulp) applied at knife-edges.
"""

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


def announce(*what):
    print("[gpu]", *what, flush=True)


def bf16(bits):
    return P.to_gpu_bf16(bits, DEV)


def bits(t):
    return P.from_gpu_bits(t)


def norm_case(T, H, seed=0, eps=1e-6, outliers=0.0, std=1.0):
    x = gen.normal_bf16((T, H), seed, 1, std=std, outlier_frac=outliers)
    r = gen.normal_bf16((T, H), seed, 2, outlier_frac=outliers)
    w = gen.normal_bf16((H,), seed, 3, mean=1.0, std=0.1)
    return x, r, w


def run_norm(x, r, w, eps, variant=-1):
    announce("fused_add_rmsnorm", x.shape, "eps", eps, "variant", variant)
    out, res_out = A.fused_add_rmsnorm(bf16(x), bf16(r), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(out), bits(res_out)


def run_norm_fp8(x, r, w, eps, variant=-1):
    announce("fused_add_rmsnorm_quant_fp8", x.shape, "eps", eps, "variant", variant)
    q, s, res_out = A.fused_add_rmsnorm_quant_fp8(bf16(x), bf16(r), bf16(w), eps, variant=variant)
    torch.cuda.synchronize()
    return bits(q), bits(s), bits(res_out)


def run_swiglu(gu, variant=-1):
    announce("swiglu", gu.shape, "variant", variant)
    y = A.swiglu(bf16(gu), variant=variant)
    torch.cuda.synchronize()
    return bits(y)


def run_swiglu_fp8(gu, scale, variant=-1):
    announce("swiglu_quant_fp8", gu.shape, "scale", scale, "variant", variant)
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    q = A.swiglu_quant_fp8(bf16(gu), s, variant=variant)
    torch.cuda.synchronize()
    return bits(q)


def norm_variants_for(H):
    return [v for v in range(A.variant_count(A.OP_NORM)) if A.variant_fits(A.OP_NORM, v, H)]


# ------------------------------------------------------------------ library

def test_native_library_is_loaded():
    lib = A.load()
    assert lib._name == A.lib_path()
    assert torch.cuda.is_available()
    announce("device", torch.cuda.get_device_name(0), torch.cuda.get_device_properties(0).gcnArchName)


# ------------------------------------------------------------------ norm

@pytest.mark.parametrize("T,H", [(1, 8), (3, 24), (16, 1536), (5, 520), (257, 1536), (7, 4104),
                                 (33, 8192), (4, 16384), (3, 16392), (2, 40000), (1, 65536),
                                 (1023, 1536), (1024, 1536)])
def test_norm_shapes_default_variant(T, H):
    x, r, w = norm_case(T, H, seed=T + H)
    out, res_out = run_norm(x, r, w, 1e-6)
    rep = P.check_norm(x, r, w, 1e-6, out, res_out)
    announce(rep)


@pytest.mark.parametrize("H", [512, 1536, 4096, 16384])
def test_norm_every_variant(H):
    T = 37
    x, r, w = norm_case(T, H, seed=H)
    for v in norm_variants_for(H):
        out, res_out = run_norm(x, r, w, 1e-5, variant=v)
        P.check_norm(x, r, w, 1e-5, out, res_out)
        q, s, res_q = run_norm_fp8(x, r, w, 1e-5, variant=v)
        P.check_norm_fp8(x, r, w, 1e-5, q, s, res_q)


def test_norm_pipelined_variants_walk_several_rows():
    """Persistent variants: T larger than the grid covers, so every block
    walks at least two rows (and some a third), through the public API."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for v in range(A.variant_count(A.OP_NORM)):
        name = A.variant_name(A.OP_NORM, v)
        if "pipelined" not in name:
            continue
        w = 1 if name.startswith("wave/row") else int(name.split()[0])
        vec = int(name.split("x")[-1].split()[0])
        bpc = int(name.split("pipelined")[1].split()[0])
        rows_per_block = 4 if w == 1 else 1
        H = min(w * 64 * vec * 8, 16384) if w > 1 else 1536
        T = 2 * cus * bpc * rows_per_block + 37
        x, r, wt = norm_case(T, H, seed=v)
        out, res_out = run_norm(x, r, wt, 1e-5, variant=v)
        P.check_norm(x, r, wt, 1e-5, out, res_out)
        q, s, res_q = run_norm_fp8(x, r, wt, 1e-5, variant=v)
        P.check_norm_fp8(x, r, wt, 1e-5, q, s, res_q)


@pytest.mark.parametrize("T,H", [(768, 5120), (1024, 8192), (1536, 6144), (1000, 7168)])
def test_norm_default_variant_mid_batches(T, H):
    """Batches where the library picks the persistent, pipelined variant for
    the bf16 form (each block walks several rows)."""
    x, r, w = norm_case(T, H, seed=T + H, outliers=0.001)
    out, res_out = run_norm(x, r, w, 1e-6)
    P.check_norm(x, r, w, 1e-6, out, res_out)


def test_norm_decode16_full():
    wl = W.NORM_DECODE16
    d = W.norm_inputs(wl)
    out, res_out = run_norm(d["x"], d["residual"], d["weight"], wl.eps)
    announce(P.check_norm(d["x"], d["residual"], d["weight"], wl.eps, out, res_out))


def test_norm_prefill4096_full():
    wl = W.NORM_PREFILL4096
    d = W.norm_inputs(wl)
    out, res_out = run_norm(d["x"], d["residual"], d["weight"], wl.eps)
    announce(P.check_norm(d["x"], d["residual"], d["weight"], wl.eps, out, res_out))


def test_norm_prefill4096_full_every_variant():
    """Every variant that fits the row, at the full Qwen2.5-1.5B prefill
    shape: start-up tuning may install any of them for this shape."""
    wl = W.NORM_PREFILL4096
    d = W.norm_inputs(wl)
    expect = P.NormExpectation(d["x"], d["residual"], d["weight"], wl.eps)
    xt, rt, wt = bf16(d["x"]), bf16(d["residual"]), bf16(d["weight"])
    for v in norm_variants_for(wl.hidden):
        announce("fused_add_rmsnorm", (wl.tokens, wl.hidden), "variant", v, A.variant_name(A.OP_NORM, v))
        out, res_out = A.fused_add_rmsnorm(xt, rt, wt, wl.eps, variant=v)
        torch.cuda.synchronize()
        expect.check(bits(out), bits(res_out))


def test_norm_closed_forms_on_gpu():
    H = 1536
    w = gen.normal_bf16((H,), 0, 3, mean=1.0, std=0.1)
    c = oracle.bf16_from_f64(0.75)
    x = np.full((4, H), c, np.uint16)
    x[1] ^= 0x8000
    x[2] = 0
    z = np.zeros_like(x)
    out, res_out = run_norm(x, z, w, 1e-6)
    assert np.array_equal(out[0], w) and np.array_equal(out[1], w ^ 0x8000)
    assert np.all(oracle.bf16_to_f32(out[2]) == 0)
    # scale invariance, eps = 0
    xr = gen.normal_bf16((8, H), 1, 1)
    base, _ = run_norm(xr, np.zeros_like(xr), w, 0.0)
    for k in (-5, 3):
        xs = gen.bf16_bits_from_f32(oracle.bf16_to_f32(xr) * np.float32(2.0 ** k))
        o, _ = run_norm(xs, np.zeros_like(xs), w, 0.0)
        assert np.array_equal(o, base)


def test_norm_in_place():
    T, H = 64, 1536
    x, r, w = norm_case(T, H, seed=9)
    xt, rt = bf16(x), bf16(r)
    announce("fused_add_rmsnorm in place", (T, H))
    A.fused_add_rmsnorm(xt, rt, bf16(w), 1e-6, out=xt, residual_out=rt)
    torch.cuda.synchronize()
    P.check_norm(x, r, w, 1e-6, bits(xt), bits(rt))


# ------------------------------------------------------------------ norm + fp8

def test_norm_fp8_llama405b_full():
    wl = W.NORM_FP8_LLAMA405B
    d = W.norm_inputs(wl)
    q, s, res_out = run_norm_fp8(d["x"], d["residual"], d["weight"], wl.eps)
    rep = P.check_norm_fp8(d["x"], d["residual"], d["weight"], wl.eps, q, s, res_out)
    announce(rep)
    dec = oracle.e4m3_table()
    assert np.all(np.nanmax(np.abs(dec[q]), axis=1) == 448.0)


@pytest.mark.parametrize("H", [1536, 16384])
def test_norm_fp8_edge_rows(H):
    T = 6
    x, r, w = norm_case(T, H, seed=5)
    x[0] = 0
    r[0] = 0                                           # all-zero row: s = 0, q = 0
    x[1] = oracle.bf16_from_f64(0.5)
    r[1] = 0                                           # constant row
    x[2] = oracle.bf16_from_f64(1e-3)
    r[2] = 0
    x[2, 7] = oracle.bf16_from_f64(300.0)              # one outlier
    x[3, 11] = oracle.bf16_from_f64(64.0)
    x[3, 12] = oracle.bf16_from_f64(-64.0)             # +-amax tie (equal weights)
    r[3, 11] = r[3, 12] = 0
    w[12] = w[11]
    q, s, res_out = run_norm_fp8(x, r, w, 1e-5)
    P.check_norm_fp8(x, r, w, 1e-5, q, s, res_out)
    assert s[0] == 0 and np.all((q[0] & 0x7F) == 0)
    assert q[2, 7] in (0x7E, 0xFE)


def test_norm_fp8_ragged_and_tiny():
    for T, H in [(1, 8), (2, 24), (9, 1000 * 8 + 8), (5, 16392)]:
        x, r, w = norm_case(T, H, seed=H, outliers=0.01)
        q, s, res_out = run_norm_fp8(x, r, w, 1e-5)
        P.check_norm_fp8(x, r, w, 1e-5, q, s, res_out)


# ------------------------------------------------------------------ swiglu

@pytest.mark.parametrize("variant", [-1, 0, 1, 2, 3, 4])
def test_swiglu_silu_table_exhaustive(variant):
    """One row: gate = every bf16 pattern, up = 1, so the output is the
    GPU's bf16(silu(g)) for all 65,536 gates: it must equal the oracle's
    correctly rounded table everywhere (NaN positions as NaN), in every
    kernel variant."""
    if variant >= A.variant_count(A.OP_SWIGLU):
        pytest.skip("no such variant")
    g = np.arange(65536, dtype=np.uint16)
    one = np.full(65536, oracle.bf16_from_f64(1.0), np.uint16)
    gu = np.concatenate([g, one])[None, :]
    y = run_swiglu(gu, variant=variant)[0]
    tab = oracle.silu_table()
    bad = ~P.same_bf16(y, tab)
    assert not bad.any(), "gates %s: gpu %s oracle %s" % (
        [hex(v) for v in g[bad][:8]], [hex(v) for v in y[bad][:8]], [hex(v) for v in tab[bad][:8]])


@pytest.mark.parametrize("T,N", [(1, 8), (3, 24), (5, 1032), (64, 8960), (7, 28672), (333, 136)])
def test_swiglu_shapes(T, N):
    gu = gen.normal_bf16((T, 2 * N), T * N, 4, std=3.0)
    for v in range(A.variant_count(A.OP_SWIGLU)):
        y = run_swiglu(gu, variant=v)
        P.check_swiglu(gu, y)


def test_swiglu_prefill4096_full():
    wl = W.SWIGLU_PREFILL4096
    gu = W.swiglu_inputs(wl)["gate_up"]
    y = run_swiglu(gu)
    P.check_swiglu(gu, y)


def test_swiglu_prefill4096_full_every_variant():
    wl = W.SWIGLU_PREFILL4096
    gu = W.swiglu_inputs(wl)["gate_up"]
    y_o = oracle.swiglu(gu)
    gt = bf16(gu)
    for v in range(A.variant_count(A.OP_SWIGLU)):
        announce("swiglu", gu.shape, "variant", v, A.variant_name(A.OP_SWIGLU, v))
        y = bits(A.swiglu(gt, variant=v))
        bad = ~P.same_bf16(y, y_o)
        assert not bad.any(), "variant %d differs at %d positions" % (v, bad.sum())


def test_swiglu_forms_past_65535_rows():
    """More rows than one grid dimension holds: rows continue in grid z."""
    T = 2 * 65535 + 7
    for N in (16, 32, 128):
        gu = gen.normal_bf16((T, 2 * N), N, 4, std=2.0)
        gt = bf16(gu)
        announce("swiglu forms", (T, N))
        for v in range(A.variant_count(A.OP_SWIGLU)):
            P.check_swiglu(gu, bits(A.swiglu(gt, variant=v)))
        s = torch.tensor([0.05], dtype=torch.float32, device=DEV)
        P.check_swiglu_fp8(gu, 0.05, bits(A.swiglu_quant_fp8(gt, s)))
        q, sc = A.swiglu_quant_fp8_dynamic(gt)
        P.check_swiglu_fp8_dynamic(gu, bits(q), bits(sc))
        q, sc = A.swiglu_quant_nvfp4(gt, s)
        P.check_swiglu_nvfp4(gu, 0.05, bits(q), bits(sc))
        if N % 32 == 0:
            q, sc = A.swiglu_quant_mxfp4(gt)
            P.check_swiglu_mxfp4(gu, bits(q), bits(sc))
        if N % A.FP8_GROUP == 0:
            q, sc = A.swiglu_quant_fp8_group(gt)
            P.check_swiglu_fp8_group(gu, bits(q), bits(sc))
        torch.cuda.synchronize()


def test_norm_many_narrow_rows():
    T, H = 3 * 65535 + 5, 8
    x, r, w = norm_case(T, H, seed=77)
    for v in norm_variants_for(H)[:6]:
        out, res_out = run_norm(x, r, w, 1e-6, variant=v)
        P.check_norm(x, r, w, 1e-6, out, res_out)


def test_quantised_norms_many_narrow_rows():
    """300,000 rows of 128 (75,000 four-row blocks): every quantised norm
    form, with and without the residual add, at the library's variant."""
    T, H = 300000, 128
    x, r, w = norm_case(T, H, seed=78, outliers=0.001)
    xt, rt, wt = bf16(x), bf16(r), bf16(w)
    g = torch.tensor([0.02], dtype=torch.float32, device=DEV)
    announce("quantised norms", (T, H))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8(xt, rt, wt, 1e-5)
    P.check_norm_fp8(x, r, w, 1e-5, bits(q), bits(s), bits(ro))
    q, ro = A.fused_add_rmsnorm_quant_fp8_static(xt, rt, wt, g, 1e-5)
    P.check_norm_fp8_static(x, r, w, 1e-5, 0.02, bits(q), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_fp8_group(xt, rt, wt, 1e-5)
    P.check_norm_fp8_group(x, r, w, 1e-5, bits(q), bits(s), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_mxfp4(xt, rt, wt, 1e-5)
    P.check_norm_mxfp4(x, r, w, 1e-5, bits(q), bits(s), bits(ro))
    q, s, ro = A.fused_add_rmsnorm_quant_nvfp4(xt, rt, wt, g, 1e-5)
    P.check_norm_nvfp4(x, r, w, 1e-5, 0.02, bits(q), bits(s), bits(ro))
    q, s = A.rmsnorm_quant_fp8(xt, wt, 1e-5)
    P.check_rmsnorm_fp8(x, w, 1e-5, bits(q), bits(s))
    q, s = A.rmsnorm_quant_fp8_group(xt, wt, 1e-5)
    P.check_rmsnorm_fp8_group(x, w, 1e-5, bits(q), bits(s))
    torch.cuda.synchronize()


# ------------------------------------------------------------------ swiglu + fp8

def _all_y_rows():
    """gate = 8 (bf16(silu(8)) = 8 exactly), up = every bf16, so y = 8u:
    every bf16 y except the top three binades reaches the quantiser."""
    u = np.arange(65536, dtype=np.uint16)
    g = np.full(65536, oracle.bf16_from_f64(8.0), np.uint16)
    return np.concatenate([g, u])[None, :]


@pytest.mark.parametrize("scale", [0.05, 1.0, 0.1, 3.0e-3, 17.5, 2.0 ** -10, 1.0e-40, 2.0 ** 120, 2.0 ** -126])
def test_swiglu_fp8_every_y(scale):
    gu = _all_y_rows()
    q = run_swiglu_fp8(gu, scale)
    P.check_swiglu_fp8(gu, scale, q)


def test_swiglu_fp8_every_y_every_variant():
    gu = _all_y_rows()
    for v in range(A.variant_count(A.OP_SWIGLU)):
        for scale in (0.05, 2.0 ** -126):
            q = run_swiglu_fp8(gu, scale, variant=v)
            P.check_swiglu_fp8(gu, scale, q)


def test_swiglu_fp8_zero_scale_is_one():
    gu = _all_y_rows()
    q0 = run_swiglu_fp8(gu, 0.0)
    q1 = run_swiglu_fp8(gu, 1.0)
    assert np.array_equal(q0, q1)


@pytest.mark.parametrize("T,N", [(1, 8), (5, 1032), (64, 8960), (3, 28672)])
def test_swiglu_fp8_shapes(T, N):
    gu = gen.normal_bf16((T, 2 * N), T + N, 4, std=2.0)
    for v in range(A.variant_count(A.OP_SWIGLU)):
        q = run_swiglu_fp8(gu, 0.05, variant=v)
        P.check_swiglu_fp8(gu, 0.05, q)


def test_swiglu_fp8_llama70b_full():
    wl = W.SWIGLU_FP8_LLAMA70B
    gu = W.swiglu_inputs(wl)["gate_up"]
    q = run_swiglu_fp8(gu, wl.scale)
    P.check_swiglu_fp8(gu, wl.scale, q)


# ------------------------------------------------------------------ one GPU's share

def test_norm_fp8_llama405b_sequence_parallel_share():
    """[256, 16384]: the 405B norm's rows on one of 8 sequence-parallel GPUs
    (a quarter of a wave of blocks, at the variant the library picks)."""
    wl = W.NORM_FP8_LLAMA405B_SP8
    d = W.norm_inputs(wl)
    q, s, res_out = run_norm_fp8(d["x"], d["residual"], d["weight"], wl.eps)
    announce(P.check_norm_fp8(d["x"], d["residual"], d["weight"], wl.eps, q, s, res_out))


def test_swiglu_fp8_llama70b_tensor_parallel_share():
    """[8192, 7168] -> [8192, 3584]: the 70B MLP activation on one of 8
    tensor-parallel GPUs, static and per-token scales."""
    wl = W.SWIGLU_FP8_LLAMA70B_TP8
    gu = W.swiglu_inputs(wl)["gate_up"]
    q = run_swiglu_fp8(gu, wl.scale)
    P.check_swiglu_fp8(gu, wl.scale, q)
    announce("swiglu_quant_fp8_dynamic", gu.shape)
    qd, sd = A.swiglu_quant_fp8_dynamic(bf16(gu))
    torch.cuda.synchronize()
    P.check_swiglu_fp8_dynamic(gu, bits(qd), bits(sd))


# ------------------------------------------------------------------ determinism

def test_repeat_runs_are_bitwise_identical():
    x, r, w = norm_case(512, 16384, seed=3, outliers=0.001)
    xt, rt, wt = bf16(x), bf16(r), bf16(w)
    gu = bf16(gen.normal_bf16((256, 2 * 8960), 3, 4))
    scale = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    announce("determinism: 20 repeats of each op")
    ref = None
    for i in range(20):
        o, ro = A.fused_add_rmsnorm(xt, rt, wt, 1e-5)
        q, s, rq = A.fused_add_rmsnorm_quant_fp8(xt, rt, wt, 1e-5)
        y = A.swiglu(gu)
        yq = A.swiglu_quant_fp8(gu, scale)
        got = [bits(t) for t in (o, ro, q, s, rq, y, yq)]
        if ref is None:
            ref = got
        else:
            for a, b in zip(ref, got):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
