"""Comparison of GPU results with the oracle (numpy only, no GPU calls).

The reading of "within 1 bf16 ulp / 1 E4M3 ulp" used here: the pages leave
the order of the row reduction open and say a fused kernel's results may
differ from the unfused ones in the last bits for that reason.  So a GPU norm
output is correct when it equals the oracle's value for *some* per-row
multiplier rho within relative distance DELTA of the exact 1/sqrt(mean+eps)
(the "admissible" values; one or two per element).  Outside such knife-edges
the admissible set is the single nominal value, so these checks demand
bit-exactness there.  The residual output has no freedom at all.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

# Relative window for the row multiplier.  A binary64 accumulation over any
# order, one rounding to binary32 for the mean, one for mean + eps and one for
# the reciprocal square root stay far inside 2^-18.
DELTA = 2.0 ** -18


# ----------------------------------------------------------------- tensors

def to_gpu_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def from_gpu_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


# ----------------------------------------------------------------- ulps

def bf16_ordered(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def e4m3_ordered(q: np.ndarray) -> np.ndarray:
    q = q.astype(np.int64)
    mag = q & 0x7F
    return np.where(q & 0x80, -mag, mag)


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordered(a) - bf16_ordered(b))


def e4m3_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(e4m3_ordered(a) - e4m3_ordered(b))


def same_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Bitwise equal, with every NaN equal to every NaN."""
    fa, fb = oracle.bf16_to_f32(a), oracle.bf16_to_f32(b)
    return (a == b) | (np.isnan(fa) & np.isnan(fb))


# ----------------------------------------------------------------- norm

class NormReport(dict):
    pass


def norm_admissible(res_out: np.ndarray, weight: np.ndarray, eps: float):
    """Nominal oracle output and the two window-end alternatives."""
    rs, rs_exact = oracle.rms_scale(res_out, eps)
    lo, hi = oracle.rms_window(rs_exact, DELTA)
    nominal = oracle.rmsnorm_apply(res_out, weight, rs)
    alt_lo = oracle.rmsnorm_apply(res_out, weight, lo)
    alt_hi = oracle.rmsnorm_apply(res_out, weight, hi)
    return nominal, alt_lo, alt_hi


def check_norm(x, residual, weight, eps, out_gpu, res_out_gpu) -> NormReport:
    """Assert the GPU's fused_add_rmsnorm results; return statistics."""
    res_out = oracle.residual_add(x, residual)
    bad_res = ~same_bf16(res_out_gpu, res_out)
    assert not bad_res.any(), "residual_out differs at %d positions, first %s" % (
        bad_res.sum(), np.argwhere(bad_res)[:5].tolist())
    nominal, alt_lo, alt_hi = norm_admissible(res_out, weight, eps)
    exact = same_bf16(out_gpu, nominal)
    admissible = exact | same_bf16(out_gpu, alt_lo) | same_bf16(out_gpu, alt_hi)
    bad = ~admissible
    assert not bad.any(), "out outside the admissible set at %d positions, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), out_gpu[bad][:5], nominal[bad][:5])
    finite = np.isfinite(oracle.bf16_to_f32(nominal))
    ulps = bf16_ulps(out_gpu[finite], nominal[finite])
    return NormReport(elements=int(out_gpu.size), not_nominal=int((~exact).sum()),
                      max_ulps_vs_nominal=int(ulps.max()) if ulps.size else 0)


class NormExpectation:
    """The oracle's results for one fused_add_rmsnorm input, computed once,
    to check the outputs of many launches (every kernel variant) against."""

    def __init__(self, x, residual, weight, eps):
        self.res_out = oracle.residual_add(x, residual)
        self.nominal, self.alt_lo, self.alt_hi = norm_admissible(self.res_out, weight, eps)

    def check(self, out_gpu, res_out_gpu) -> NormReport:
        bad_res = ~same_bf16(res_out_gpu, self.res_out)
        assert not bad_res.any(), "residual_out differs at %d positions, first %s" % (
            bad_res.sum(), np.argwhere(bad_res)[:5].tolist())
        exact = same_bf16(out_gpu, self.nominal)
        bad = ~(exact | same_bf16(out_gpu, self.alt_lo) | same_bf16(out_gpu, self.alt_hi))
        assert not bad.any(), "out outside the admissible set at %d positions, first %s" % (
            bad.sum(), np.argwhere(bad)[:5].tolist())
        return NormReport(elements=int(out_gpu.size), not_nominal=int((~exact).sum()))


def check_rmsnorm(x, weight, eps, out_gpu) -> NormReport:
    """Assert the GPU's rmsnorm (no residual add) results."""
    nominal, alt_lo, alt_hi = norm_admissible(x, weight, eps)
    exact = same_bf16(out_gpu, nominal)
    admissible = exact | same_bf16(out_gpu, alt_lo) | same_bf16(out_gpu, alt_hi)
    bad = ~admissible
    assert not bad.any(), "out outside the admissible set at %d positions, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), out_gpu[bad][:5], nominal[bad][:5])
    return NormReport(elements=int(out_gpu.size), not_nominal=int((~exact).sum()))


def _check_dynamic_codes(rows_in, weight, eps, q_gpu, s_gpu, q_o, s_o) -> NormReport:
    """Per-token E4M3 codes and scales of a norm of rows_in (the rows the
    norm normalizes), against the oracle's q_o, s_o.  A NaN code matches any
    NaN code and a NaN scale any NaN scale (a NaN's sign carries nothing)."""
    same_s = (s_gpu.view(np.uint32) == s_o.view(np.uint32)) | (np.isnan(s_gpu) & np.isnan(s_o))
    rows_s = np.flatnonzero(~same_s)
    bad_q = ~_same_codes(q_gpu, q_o)
    rows_q = np.flatnonzero(bad_q.any(axis=1))
    rows = np.union1d(rows_s, rows_q)
    if len(rows):
        _, lo, hi = norm_admissible(rows_in[rows], weight, eps)
        ylo, yhi = oracle.bf16_to_f32(lo), oracle.bf16_to_f32(hi)
        amax_lo = np.minimum(np.abs(ylo), np.abs(yhi)).max(axis=1)
        amax_hi = np.maximum(np.abs(ylo), np.abs(yhi)).max(axis=1)
        s_lo = (amax_lo.astype(np.float32) / np.float32(448)).astype(np.float32)
        s_hi = (amax_hi.astype(np.float32) / np.float32(448)).astype(np.float32)
        sg = s_gpu[rows]
        ok_s = (sg >= s_lo * (1 - 1e-6)) & (sg <= s_hi * (1 + 1e-6))
        assert ok_s.all(), "scale outside tolerance in rows %s" % rows[~ok_s][:5].tolist()
        for k, r in enumerate(rows):
            cand = [oracle.quant_fp8_static(lo[k], float(sg[k])), oracle.quant_fp8_static(hi[k], float(sg[k]))]
            d = np.minimum(e4m3_ulps(q_gpu[r], cand[0]), e4m3_ulps(q_gpu[r], cand[1]))
            d[_same_codes(q_gpu[r], q_o[r])] = 0
            assert d.max() <= 1, "row %d: code off by %d e4m3 ulps" % (r, d.max())
    return NormReport(rows=int(q_gpu.shape[0]), rows_not_nominal=int(len(rows)),
                      codes_not_nominal=int(bad_q.sum()),
                      scales_not_nominal=int(len(rows_s)))


def check_norm_fp8(x, residual, weight, eps, q_gpu, s_gpu, res_out_gpu) -> NormReport:
    """Assert fused_add_rmsnorm_quant_fp8 results.

    Bit-exact is expected; the stated tolerances (scales within 1e-6
    relative, codes within 1 E4M3 ulp) are applied against admissible values
    where the norm output itself sits on a knife-edge."""
    q_o, s_o, res_o, y_o, _ = oracle.fused_add_rmsnorm_quant_fp8(x, residual, weight, eps)
    bad_res = ~same_bf16(res_out_gpu, res_o)
    assert not bad_res.any(), "residual_out differs at %d positions" % bad_res.sum()
    return _check_dynamic_codes(res_o, weight, eps, q_gpu, s_gpu, q_o, s_o)


def check_rmsnorm_fp8(x, weight, eps, q_gpu, s_gpu) -> NormReport:
    """Assert rmsnorm_quant_fp8 (no residual add, per-token scale) results."""
    q_o, s_o, _, _ = oracle.rmsnorm_quant_fp8(x, weight, eps)
    return _check_dynamic_codes(x, weight, eps, q_gpu, s_gpu, q_o, s_o)


def _same_codes(a, b):
    """Equal E4M3 codes, with every NaN code equal to every NaN code."""
    nan_a, nan_b = np.isin(a, [0x7F, 0xFF]), np.isin(b, [0x7F, 0xFF])
    return (a == b) | (nan_a & nan_b)


def _check_static_codes(rows_in, weight, eps, scale, q_gpu, q_o) -> NormReport:
    bad = ~_same_codes(q_gpu, q_o)
    rows = np.flatnonzero(bad.any(axis=1))
    if len(rows):
        _, lo, hi = norm_admissible(rows_in[rows], weight, eps)
        for k, r in enumerate(rows):
            cand = [oracle.quant_fp8_static(lo[k], scale), oracle.quant_fp8_static(hi[k], scale)]
            d = np.minimum(e4m3_ulps(q_gpu[r], cand[0]), e4m3_ulps(q_gpu[r], cand[1]))
            d[_same_codes(q_gpu[r], q_o[r])] = 0
            assert d.max() <= 1, "row %d: code off by %d e4m3 ulps" % (r, d.max())
    return NormReport(rows=int(q_gpu.shape[0]), rows_not_nominal=int(len(rows)),
                      codes_not_nominal=int(bad.sum()))


def check_norm_fp8_static(x, residual, weight, eps, scale, q_gpu, res_out_gpu) -> NormReport:
    """Assert fused_add_rmsnorm_quant_fp8_static results (codes bit-exact
    except where the norm output sits on a knife-edge, then within 1 E4M3 ulp
    of an admissible value)."""
    q_o, res_o, _, _ = oracle.fused_add_rmsnorm_quant_fp8_static(x, residual, weight, eps, scale)
    bad_res = ~same_bf16(res_out_gpu, res_o)
    assert not bad_res.any(), "residual_out differs at %d positions" % bad_res.sum()
    return _check_static_codes(res_o, weight, eps, scale, q_gpu, q_o)


def check_rmsnorm_fp8_static(x, weight, eps, scale, q_gpu) -> NormReport:
    q_o, _, _ = oracle.rmsnorm_quant_fp8_static(x, weight, eps, scale)
    return _check_static_codes(x, weight, eps, scale, q_gpu, q_o)



# ----------------------------------------------------------------- per-group E4M3

def _same_scales(a, b):
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))


def _check_group_codes(rows_in, weight, eps, q_gpu, s_gpu, q_o, s_o) -> NormReport:
    """Per-group E4M3 codes and fp32 group scales of a norm of rows_in against
    the oracle.  Rows that differ: each group scale lies between the scales of
    the smallest and largest admissible group amax (1e-6 relative slack), and
    each code is within 1 E4M3 ulp of the code of an admissible value under
    the GPU's own group scale."""
    groups = s_gpu.shape[1]
    G = q_gpu.shape[1] // groups
    same_s = _same_scales(s_gpu, s_o)
    same_q = _same_codes(q_gpu, q_o)
    rows = np.flatnonzero(~same_s.all(axis=1) | ~same_q.all(axis=1))
    if len(rows):
        _, lo, hi = norm_admissible(rows_in[rows], weight, eps)
        alo, ahi = np.abs(oracle.bf16_to_f32(lo)), np.abs(oracle.bf16_to_f32(hi))
        n = len(rows)
        amin = np.fmax.reduce(np.fmin(alo, ahi).reshape(n, groups, G), axis=2, initial=0.0)
        amax = np.fmax.reduce(np.fmax(alo, ahi).reshape(n, groups, G), axis=2, initial=0.0)
        s_lo = (amin.astype(np.float32) / np.float32(448)).astype(np.float32)
        s_hi = (amax.astype(np.float32) / np.float32(448)).astype(np.float32)
        sg = s_gpu[rows]
        ok_s = same_s[rows] | ((sg >= s_lo * (1 - 1e-6)) & (sg <= s_hi * (1 + 1e-6)))
        assert ok_s.all(), "group scale outside tolerance in rows %s" % rows[~ok_s.all(axis=1)][:5].tolist()
        for k, r in enumerate(rows):
            for g in np.flatnonzero(~same_q[r].reshape(groups, G).all(axis=1)):
                sl = slice(g * G, (g + 1) * G)
                sc = float(sg[k, g])
                d = np.minimum(e4m3_ulps(q_gpu[r, sl], oracle.quant_fp8_static(lo[k, sl], sc)),
                               e4m3_ulps(q_gpu[r, sl], oracle.quant_fp8_static(hi[k, sl], sc)))
                d[same_q[r, sl]] = 0
                assert d.max() <= 1, "row %d group %d: code off by %d e4m3 ulps" % (r, g, d.max())
    return NormReport(rows=int(q_gpu.shape[0]), rows_not_nominal=int(len(rows)),
                      codes_not_nominal=int((~same_q).sum()),
                      scales_not_nominal=int((~same_s).sum()))


def check_norm_fp8_group(x, residual, weight, eps, q_gpu, s_gpu, res_out_gpu) -> NormReport:
    """Assert fused_add_rmsnorm_quant_fp8_group results: residual_out
    bit-exact, codes and group scales bit-exact except where the norm output
    sits on a knife-edge (then to the tolerances above)."""
    q_o, s_o, res_o, _, _ = oracle.fused_add_rmsnorm_quant_fp8_group(x, residual, weight, eps)
    bad_res = ~same_bf16(res_out_gpu, res_o)
    assert not bad_res.any(), "residual_out differs at %d positions" % bad_res.sum()
    return _check_group_codes(res_o, weight, eps, q_gpu, s_gpu, q_o, s_o)


def check_rmsnorm_fp8_group(x, weight, eps, q_gpu, s_gpu) -> NormReport:
    q_o, s_o, _, _ = oracle.rmsnorm_quant_fp8_group(x, weight, eps)
    return _check_group_codes(x, weight, eps, q_gpu, s_gpu, q_o, s_o)

# ----------------------------------------------------------------- swiglu

def check_swiglu(gate_up, y_gpu):
    y_o = oracle.swiglu(gate_up)
    bad = ~same_bf16(y_gpu, y_o)
    assert not bad.any(), "swiglu differs at %d positions, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), y_gpu[bad][:5], y_o[bad][:5])


def check_swiglu_fp8(gate_up, scale, q_gpu):
    q_o = oracle.swiglu_quant_fp8(gate_up, scale)
    nan_o = np.isin(q_o, [0x7F, 0xFF])
    nan_g = np.isin(q_gpu, [0x7F, 0xFF])
    assert np.array_equal(nan_o, nan_g), "NaN codes differ at %d positions" % (nan_o != nan_g).sum()
    bad = (q_gpu != q_o) & ~nan_o
    assert not bad.any(), "swiglu_quant_fp8 differs at %d positions, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), q_gpu[bad][:5], q_o[bad][:5])


def check_swiglu_fp8_dynamic(gate_up, q_gpu, s_gpu):
    """Per-token E4M3 SwiGLU: the SwiGLU output has no knife-edges (its
    SiLU is correctly rounded), so scales and codes must be bit-exact."""
    q_o, s_o, _ = oracle.swiglu_quant_fp8_dynamic(gate_up)
    bad_s = ~((s_gpu.view(np.uint32) == s_o.view(np.uint32)) | (np.isnan(s_gpu) & np.isnan(s_o)))
    assert not bad_s.any(), "scales differ in %d rows, first %s: gpu %s oracle %s" % (
        bad_s.sum(), np.flatnonzero(bad_s)[:5].tolist(), s_gpu[bad_s][:5], s_o[bad_s][:5])
    bad = ~_same_codes(q_gpu, q_o)
    assert not bad.any(), "codes differ at %d positions, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), q_gpu[bad][:5], q_o[bad][:5])


# ----------------------------------------------------------------- mxfp4

def e2m1_ordered(q: np.ndarray) -> np.ndarray:
    q = q.astype(np.int64)
    mag = q & 0x7
    return np.where(q & 0x8, -mag, mag)


def _unpack_e2m1(q: np.ndarray) -> np.ndarray:
    return np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1)


def _check_mx_codes(rows_in, weight, eps, q_gpu, s_gpu, q_o, s_o) -> NormReport:
    """MXFP4 codes and E8M0 scales of a norm of rows_in against the oracle;
    rows that differ must match the oracle's MXFP4 of an admissible norm
    output (scales exactly, codes within one E2M1 step)."""
    rows = np.flatnonzero((q_gpu != q_o).any(axis=1) | (s_gpu != s_o).any(axis=1))
    if len(rows):
        _, lo, hi = norm_admissible(rows_in[rows], weight, eps)
        cands = [oracle.quant_mxfp4(lo), oracle.quant_mxfp4(hi)]
        for k, r in enumerate(rows):
            ok_s = np.zeros(s_gpu.shape[1], bool)
            d = np.full(q_gpu.shape[1] * 2, 99)
            for cq, cs in cands:
                same_s = s_gpu[r] == cs[k]
                ok_s |= same_s
                dd = np.abs(e2m1_ordered(_unpack_e2m1(q_gpu[r][None])[0]) -
                            e2m1_ordered(_unpack_e2m1(cq[k][None])[0]))
                dd[~np.repeat(same_s, 32)] = 99
                d = np.minimum(d, dd)
            assert ok_s.all(), "row %d: block scales outside the admissible set" % r
            assert d.max() <= 1, "row %d: code off by %d E2M1 steps" % (r, d.max())
    return NormReport(rows=int(q_gpu.shape[0]), rows_not_nominal=int(len(rows)),
                      codes_not_nominal=int((q_gpu != q_o).sum()),
                      scales_not_nominal=int((s_gpu != s_o).sum()))


def _check_fp4_codes(rows_in, weight, eps, q_gpu, s_gpu, q_o, s_o, quant) -> NormReport:
    """Block-scaled FP4 codes of a norm of rows_in against the oracle; rows
    that differ must match the oracle's encoding (quant) of an admissible
    norm output (scales exactly, codes within one E2M1 step)."""
    rows = np.flatnonzero((q_gpu != q_o).any(axis=1) | (s_gpu != s_o).any(axis=1))
    blk = (q_gpu.shape[1] * 2) // s_gpu.shape[1]
    if len(rows):
        _, lo, hi = norm_admissible(rows_in[rows], weight, eps)
        cands = [quant(lo), quant(hi)]
        for k, r in enumerate(rows):
            ok_s = np.zeros(s_gpu.shape[1], bool)
            d = np.full(q_gpu.shape[1] * 2, 99)
            for cq, cs in cands:
                same_s = s_gpu[r] == cs[k]
                ok_s |= same_s
                dd = np.abs(e2m1_ordered(_unpack_e2m1(q_gpu[r][None])[0]) -
                            e2m1_ordered(_unpack_e2m1(cq[k][None])[0]))
                dd[~np.repeat(same_s, blk)] = 99
                d = np.minimum(d, dd)
            assert ok_s.all(), "row %d: block scales outside the admissible set" % r
            assert d.max() <= 1, "row %d: code off by %d E2M1 steps" % (r, d.max())
    return NormReport(rows=int(q_gpu.shape[0]), rows_not_nominal=int(len(rows)),
                      codes_not_nominal=int((q_gpu != q_o).sum()),
                      scales_not_nominal=int((s_gpu != s_o).sum()))


def check_norm_nvfp4(x, residual, weight, eps, g, q_gpu, s_gpu, res_out_gpu) -> NormReport:
    q_o, s_o, res_o, _, _ = oracle.fused_add_rmsnorm_quant_nvfp4(x, residual, weight, eps, g)
    bad_res = ~same_bf16(res_out_gpu, res_o)
    assert not bad_res.any(), "residual_out differs at %d positions" % bad_res.sum()
    return _check_fp4_codes(res_o, weight, eps, q_gpu, s_gpu, q_o, s_o, lambda y: oracle.quant_nvfp4(y, g))


def check_rmsnorm_nvfp4(x, weight, eps, g, q_gpu, s_gpu) -> NormReport:
    q_o, s_o, _, _ = oracle.rmsnorm_quant_nvfp4(x, weight, eps, g)
    return _check_fp4_codes(x, weight, eps, q_gpu, s_gpu, q_o, s_o, lambda y: oracle.quant_nvfp4(y, g))


def check_norm_mxfp4(x, residual, weight, eps, q_gpu, s_gpu, res_out_gpu) -> NormReport:
    q_o, s_o, res_o, _, _ = oracle.fused_add_rmsnorm_quant_mxfp4(x, residual, weight, eps)
    bad_res = ~same_bf16(res_out_gpu, res_o)
    assert not bad_res.any(), "residual_out differs at %d positions" % bad_res.sum()
    return _check_mx_codes(res_o, weight, eps, q_gpu, s_gpu, q_o, s_o)


def check_rmsnorm_mxfp4(x, weight, eps, q_gpu, s_gpu) -> NormReport:
    q_o, s_o, _, _ = oracle.rmsnorm_quant_mxfp4(x, weight, eps)
    return _check_mx_codes(x, weight, eps, q_gpu, s_gpu, q_o, s_o)


def check_swiglu_mxfp4(gate_up, q_gpu, s_gpu):
    """MXFP4 SwiGLU: the SwiGLU output has no knife-edges, so scales and codes
    must be bit-exact."""
    q_o, s_o, _ = oracle.swiglu_quant_mxfp4(gate_up)
    bad_s = s_gpu != s_o
    assert not bad_s.any(), "block scales differ at %d blocks, first %s: gpu %s oracle %s" % (
        bad_s.sum(), np.argwhere(bad_s)[:5].tolist(), s_gpu[bad_s][:5], s_o[bad_s][:5])
    bad = q_gpu != q_o
    assert not bad.any(), "codes differ at %d bytes, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), q_gpu[bad][:5], q_o[bad][:5])


def check_swiglu_nvfp4(gate_up, g, q_gpu, s_gpu):
    """NVFP4 SwiGLU: bit-exact scales and codes (no knife-edges in y)."""
    q_o, s_o, _ = oracle.swiglu_quant_nvfp4(gate_up, g)
    bad_s = s_gpu != s_o
    assert not bad_s.any(), "block scales differ at %d blocks, first %s: gpu %s oracle %s" % (
        bad_s.sum(), np.argwhere(bad_s)[:5].tolist(), s_gpu[bad_s][:5], s_o[bad_s][:5])
    bad = q_gpu != q_o
    assert not bad.any(), "codes differ at %d bytes, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), q_gpu[bad][:5], q_o[bad][:5])


def check_swiglu_fp8_group(gate_up, q_gpu, s_gpu):
    """Per-group E4M3 SwiGLU: no knife-edges in y, so group scales and codes
    are bit-exact."""
    q_o, s_o, _ = oracle.swiglu_quant_fp8_group(gate_up)
    bad_s = ~_same_scales(s_gpu, s_o)
    assert not bad_s.any(), "group scales differ at %d groups, first %s: gpu %s oracle %s" % (
        bad_s.sum(), np.argwhere(bad_s)[:5].tolist(), s_gpu[bad_s][:5], s_o[bad_s][:5])
    bad = ~_same_codes(q_gpu, q_o)
    assert not bad.any(), "codes differ at %d positions, first %s: gpu %s oracle %s" % (
        bad.sum(), np.argwhere(bad)[:5].tolist(), q_gpu[bad][:5], q_o[bad][:5])
