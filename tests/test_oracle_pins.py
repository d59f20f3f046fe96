"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties one step of the oracle to a closed form, an invariant, an
exact brute-force computation (tests/exact.py) or an independent library
routine (torch CPU conversions and eager ops), chosen so that a plausible
mistake -- a dropped term, a wrong rounding point, swapped gate/up halves, a
sum in place of a mean, a multiply in place of a divide -- fails one of them.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests import exact
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_of(bits):
    return oracle.bf16_to_f32(bits)


def bf16_t(bits) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


ALL_BF16 = np.arange(65536, dtype=np.uint16)
FINITE_BF16 = ALL_BF16[np.isfinite(oracle.bf16_to_f32(ALL_BF16))]


# ------------------------------------------------------------------ formats

def test_bf16_rounding_matches_torch_cast():
    """bf16 rounding of binary32 values == torch's fp32->bf16 cast, bitwise,
    over every top half combined with low halves around the tie point."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    f = u.view(np.float32)
    ref = bits_of(torch.from_numpy(f.copy()).to(torch.bfloat16))
    lib = oracle._lib()
    got = np.array([lib.aarms_oracle_bf16_from_f64(float(v)) for v in f], dtype=np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(f32_of(got[nan])))


def test_bf16_rounding_of_binary64_exact():
    """Values between binary32 points (the SiLU path rounds binary64 directly):
    brute-force nearest-even search with exact rationals."""
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(400) * np.exp2(rng.integers(-140, 120, 400)))
    # exact bf16 midpoints and their binary64 neighbours
    for b in [0x3F80, 0x0001, 0x0080, 0x7F7E, 0x3F81, 0x00FF]:
        a, c = exact.bf16_value(b), exact.bf16_value(b + 1)
        m = (a + c) / 2
        vals += [m, np.nextafter(m, 0), np.nextafter(m, np.inf), -m]
    vals += [float.fromhex("0x1.FEp127") * (1 + 2.0 ** -9), float.fromhex("0x1.FEp127") * (1 + 2.0 ** -8.5), 2.0 ** -134, 2.0 ** -134 * 1.0001]
    for v in vals:
        assert oracle.bf16_from_f64(v) == exact.round_to_bf16(Fraction(float(v))), v


def test_e4m3_decode_matches_torch():
    table = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(table), nan)
    assert np.array_equal(table[~nan], ref[~nan])
    assert table[0x7E] == 448.0 and np.nanmax(table) == 448.0
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}


def test_e4m3_encode_exhaustive_vs_bruteforce():
    """Every binary32 value on a fine grid in [-448, 448] (all bf16 values
    there, plus every E4M3 midpoint and its neighbours): oracle encode ==
    exact nearest-even search == torch's cast."""
    v = oracle.bf16_to_f32(FINITE_BF16).astype(np.float64)
    v = v[np.abs(v) <= 448]
    grid = np.array(sorted(set(oracle.e4m3_table()[:0x7F])))
    mids = (grid[1:] + grid[:-1]) / 2
    mids = np.concatenate([mids, -mids])
    extra = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                            np.nextafter(mids.astype(np.float32), np.float32(-np.inf))])
    v = np.concatenate([v, extra.astype(np.float64)])
    lib = oracle._lib()
    got = np.array([lib.aarms_oracle_e4m3_from_f64(float(x)) for x in v], dtype=np.uint8)
    ref_t = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref_t)
    sample = np.random.default_rng(3).choice(len(v), 3000, replace=False)
    for i in list(sample) + list(range(len(v) - len(extra), len(v))):
        assert got[i] == exact.round_to_e4m3(Fraction(float(v[i]))), v[i]


# ------------------------------------------------------------------ residual add

def test_residual_add_matches_torch_and_exact():
    rng = np.random.default_rng(11)
    n = 200_000
    x = gen.bf16_bits_from_f32((rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32))
    r = gen.bf16_bits_from_f32((rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32))
    got = oracle.residual_add(x, r)
    ref = bits_of(bf16_t(x) + bf16_t(r))
    assert np.array_equal(got, ref)
    # closed form: the binary32 sum of two bf16 rounds to the correctly
    # rounded bf16 sum (checked exactly on a sample)
    for i in rng.choice(n, 2000, replace=False):
        s = Fraction(float(f32_of(x[i]))) + Fraction(float(f32_of(r[i])))
        assert got[i] == exact.round_to_bf16(s)


# ------------------------------------------------------------------ RMSNorm

def _norm(x, res, w, eps):
    out, res_out, rs = oracle.fused_add_rmsnorm(x, res, w, eps)
    return out, res_out, rs


def test_rmsnorm_constant_row_gives_weight_times_sign():
    """x = c, residual = 0: mean = c^2 exactly, and t rounds to sign(c) when
    c^2 >= 512*eps, so out = w * sign(c) bit-exactly."""
    H = 1536
    w = gen.normal_bf16((H,), 0, 3, mean=1.0, std=0.1)
    cs = [1.0, -1.0, 0.5, 3.0, -0.0625, 100.0, 2.0 ** -20]
    for eps in [1e-6, 1e-5, 0.0]:
        for c in cs:
            if eps and c * c < 512 * eps:
                continue
            x = np.full((2, H), oracle.bf16_from_f64(c), np.uint16)
            z = np.zeros((2, H), np.uint16)
            out, _, _ = _norm(x, z, w, eps)
            want = w if c > 0 else (w ^ 0x8000)
            assert np.array_equal(out[0], want) and np.array_equal(out[1], want), (c, eps)
    # c = 0 with eps > 0: out = 0 (signs follow w)
    out, _, _ = _norm(np.zeros((1, H), np.uint16), np.zeros((1, H), np.uint16), w, 1e-6)
    assert np.all(f32_of(out) == 0)


def test_rmsnorm_scale_invariance():
    """eps = 0, x scaled by 2^k: every step scales exactly, output bitwise equal."""
    x = gen.normal_bf16((8, 1536), 5, 1)
    w = gen.normal_bf16((1536,), 5, 3, mean=1.0, std=0.1)
    z = np.zeros_like(x)
    base, _, _ = _norm(x, z, w, 0.0)
    for k in [-12, -3, -1, 1, 4, 9]:
        xs = gen.bf16_bits_from_f32(f32_of(x) * np.float32(2.0 ** k))
        out, _, _ = _norm(xs, z, w, 0.0)
        assert np.array_equal(out, base), k


def test_rmsnorm_unit_rms_and_weight_one():
    """w = 1: out is the normalized row; its RMS is 1 within 1e-3 (a sum in
    place of the mean, or a missing rsqrt, fails this)."""
    for H in [64, 100, 1536, 16384]:
        x = gen.normal_bf16((16, H), 2, 1, std=3.0)
        r = gen.normal_bf16((16, H), 2, 2)
        w = np.full(H, oracle.bf16_from_f64(1.0), np.uint16)
        out, res_out, _ = _norm(x, r, w, 1e-6)
        t = f32_of(out).astype(np.float64)
        rms = np.sqrt((t ** 2).mean(axis=1))
        assert np.all(np.abs(rms - 1) < 1e-3), (H, rms)
        # w = 0 gives zeros
        out0, _, _ = _norm(x, r, np.zeros(H, np.uint16), 1e-6)
        assert np.all(f32_of(out0) == 0)


def test_rmsnorm_matches_torch_eager_eight_ops():
    """torch CPU eager, the eight operations as the pages list them, on the
    residual sum.  torch sums in its own order, so the only differences
    allowed are at rounding knife-edges, inside the admissible window."""
    T, H, eps = 256, 1536, 1e-6
    x = gen.normal_bf16((T, H), 9, 1)
    res = gen.normal_bf16((T, H), 9, 2)
    w = gen.normal_bf16((H,), 9, 3, mean=1.0, std=0.1)
    out, res_out, rs = _norm(x, res, w, eps)
    hs = bf16_t(res_out)
    h = hs.to(torch.float32)                                  # cast to float
    var = h.pow(2).mean(-1, keepdim=True)                     # square, mean
    hn = h * torch.rsqrt(var + eps)                           # add eps, rsqrt, multiply
    ref = bits_of(bf16_t(w) * hn.to(torch.bfloat16))          # cast back, weight
    diff = np.flatnonzero(ref.reshape(-1) != out.reshape(-1))
    assert len(diff) < 0.005 * out.size
    _, rs_exact = oracle.rms_scale(res_out, eps)
    lo, hi = oracle.rms_window(rs_exact, 2.0 ** -18)
    alt_lo = oracle.rmsnorm_apply(res_out, w, lo).reshape(-1)
    alt_hi = oracle.rmsnorm_apply(res_out, w, hi).reshape(-1)
    r = ref.reshape(-1)
    assert np.all((r[diff] == alt_lo[diff]) | (r[diff] == alt_hi[diff]))
    # the rounding points: rounding t before the weight (the pages' order)
    # differs from a single rounding of w*h*rs on a sizeable fraction
    one_round = bits_of((bf16_t(w).float() * hn).to(torch.bfloat16))
    assert (one_round != out).mean() > 0.05


def test_rms_scale_brute_force_exact():
    """Tiny rows: mean by exact rationals, rsqrt to 60 digits, each rounded to
    binary32 by nearest-value search."""
    rng = np.random.default_rng(1)
    for H in [1, 2, 3, 5, 8]:
        for _ in range(40):
            r = gen.bf16_bits_from_f32((rng.standard_normal((1, H)) * np.exp2(rng.integers(-20, 20))).astype(np.float32))
            eps = float(np.float32([0.0, 1e-6, 1e-5, 0.25][rng.integers(4)]))
            rs, _ = oracle.rms_scale(r, eps)
            hs = [Fraction(float(v)) for v in f32_of(r[0])]
            m = exact.round_to_f32(sum(h * h for h in hs) / H)
            v = np.float32(np.float32(m) + np.float32(eps))
            if v == 0:
                continue
            want = exact.round_to_f32(exact.rsqrt_exact(Fraction(float(v))))
            assert rs[0] == np.float32(want), (H, r, eps)


# ------------------------------------------------------------------ SiLU

@pytest.fixture(scope="module")
def silu_table():
    return oracle.silu_table()


def test_silu_table_exhaustive_vs_60_digit(silu_table):
    """All 65,536 gates: the oracle's bf16(silu(g)) equals the correctly
    rounded value of silu computed to 60 digits.  Also checks that no gate's
    exact silu lies close enough to a bf16 midpoint for the oracle's binary64
    evaluation to matter (distance > 2^-40 relative) where the oracle uses it
    (|g| >= 2^-24; below that the value is g/2 up to a tie-breaking term).

    Outside [-200, 100] the exact value needs no evaluation: for g > 100,
    silu(g) = g(1 - d) with 0 < d < e^-100, which rounds to g; for g < -200,
    -e^-199 < silu(g) < 0, below half the smallest bf16 subnormal: -0."""
    closest = Fraction(1)
    for g in FINITE_BF16:
        gv = exact.bf16_value(int(g))
        if gv == 0:
            assert silu_table[g] == g  # silu(+-0) = +-0
            continue
        if gv > 100:
            assert silu_table[g] == g
            continue
        if gv < -200:
            assert silu_table[g] == 0x8000
            continue
        s = exact.silu_exact(gv)
        want = exact.round_to_bf16(s)
        assert silu_table[g] == want, hex(g)
        if abs(gv) < 2.0 ** -24 or abs(s) < Fraction(1, 2 ** 120):
            continue
        # relative distance of the exact value to the nearest bf16 midpoint
        v = Fraction(exact.bf16_value(want & 0x7FFF))
        nb = exact.bf16_value((want & 0x7FFF) + 1) if abs(s) >= v else exact.bf16_value((want & 0x7FFF) - 1)
        mid = (v + Fraction(nb)) / 2
        closest = min(closest, abs(abs(s) - mid) / abs(s))
    assert closest > Fraction(1, 2 ** 40), float(closest)


def test_silu_special_values(silu_table):
    assert silu_table[0x0000] == 0x0000 and silu_table[0x8000] == 0x8000
    assert silu_table[0x7F80] == 0x7F80              # +inf
    assert silu_table[0xFF80] == 0x8000              # -inf -> -0
    assert np.isnan(f32_of(silu_table[0x7FC0]))
    g = f32_of(ALL_BF16)
    big = np.isfinite(g) & (g >= 8)
    assert np.array_equal(silu_table[big], ALL_BF16[big])   # silu(g) rounds to g
    # silu(-g) = silu(g) - g: check on the exact values for a sample
    for gb in [0x3F80, 0x4000, 0x3E00, 0x40A0, 0x3C00]:
        gv = exact.bf16_value(gb)
        assert abs(exact.silu_exact(-gv) - (exact.silu_exact(gv) - Fraction(gv))) < Fraction(1, 10 ** 50)


def test_silu_vs_torch_differs_only_where_float_cannot_see(silu_table):
    """torch CPU F.silu on bf16 (binary32 math, one rounding) agrees with the
    oracle on every gate except two known classes, where the 60-digit pin
    above shows the oracle is the correctly rounded one:
      * |g| < 2^-24: binary32 returns g/2 exactly, an exact tie for odd
        subnormal results, and ties-to-even ignores the g^2/4 term;
      * g < -88: binary32 exp(-g) overflows and the quotient becomes -0,
        while the exact value is a bf16 subnormal.
    Any other difference must sit at a knife-edge (within 2^-18 relative of a
    bf16 midpoint)."""
    g = bf16_t(FINITE_BF16)
    ref = bits_of(F.silu(g))
    got = silu_table[FINITE_BF16]
    gv = f32_of(FINITE_BF16)
    bad = np.flatnonzero(ref != got)
    tiny = np.abs(gv[bad]) < 2.0 ** -24
    overflow = gv[bad] < -88
    assert 0 < tiny.sum() <= 254 and 0 < overflow.sum() <= 20
    for i in bad[tiny]:
        # torch's value is the even neighbour of the tie at g/2
        assert ref[i] == oracle.bf16_from_f64(float(gv[i]) / 2)
    assert np.all(f32_of(ref[bad[overflow]]) == 0)
    for i in bad[~tiny & ~overflow]:
        s = exact.silu_exact(float(gv[i]))
        a, b = Fraction(exact.bf16_value(int(got[i]))), Fraction(exact.bf16_value(int(ref[i])))
        assert abs(s - (a + b) / 2) / abs(s) < Fraction(1, 2 ** 18), hex(FINITE_BF16[i])


# ------------------------------------------------------------------ SwiGLU

def test_swiglu_layout_and_product():
    """gate is the first half of each row, up the second; y = bf16(a * u)
    with a = bf16(silu(gate)): compared with torch's bf16 multiply of the
    table value and up."""
    tab = oracle.silu_table()
    gu = gen.normal_bf16((64, 2 * 320), 4, 4, std=3.0)
    y = oracle.swiglu(gu)
    g, u = gu[:, :320], gu[:, 320:]
    ref = bits_of(bf16_t(tab[g]) * bf16_t(u))
    assert np.array_equal(y, ref)
    swapped = bits_of(bf16_t(tab[u]) * bf16_t(g))
    assert (swapped != y).mean() > 0.5


def test_swiglu_product_special_cases():
    tab = oracle.silu_table()
    n = FINITE_BF16.size
    one = np.full(n, oracle.bf16_from_f64(1.0), np.uint16)
    gu = np.concatenate([FINITE_BF16, one])[None, :]
    assert np.array_equal(oracle.swiglu(gu)[0], tab[FINITE_BF16])
    zero = np.zeros(n, np.uint16)
    y0 = oracle.swiglu(np.concatenate([FINITE_BF16, zero])[None, :])[0]
    assert np.all(f32_of(y0[np.isfinite(f32_of(tab[FINITE_BF16]))]) == 0)
    four = np.full(n, oracle.bf16_from_f64(4.0), np.uint16)
    y4 = oracle.swiglu(np.concatenate([FINITE_BF16, four])[None, :])[0]
    a = f32_of(tab[FINITE_BF16])
    ok = np.isfinite(a) & (np.abs(a) < 1e37) & ((np.abs(a) > 1e-37) | (a == 0))
    with np.errstate(over="ignore"):
        assert np.array_equal(f32_of(y4)[ok], (a * 4)[ok])


# ------------------------------------------------------------------ FP8

@pytest.mark.parametrize("scale", [0.05, 1.0, 0.1, 3.0e-3, 17.5])
def test_static_quant_exhaustive_vs_torch(scale):
    """Every bf16 y: oracle == torch clamp(y.float() / scale).to(e4m3fn)."""
    y = ALL_BF16
    q = oracle.quant_fp8_static(y, scale)
    yf = torch.from_numpy(oracle.bf16_to_f32(y).copy())
    z = torch.clamp(yf / torch.tensor(scale, dtype=torch.float32), -448.0, 448.0)
    ref = z.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(oracle.bf16_to_f32(y))
    assert np.array_equal(q[~nan], ref[~nan])
    assert np.all(np.isin(q[nan], [0x7F, 0xFF]))


def test_static_quant_saturation_and_ties():
    y = FINITE_BF16
    yf = f32_of(y)
    q = oracle.quant_fp8_static(y, 0.05)
    assert np.all(q[yf >= 22.4] == 0x7E) and np.all(q[yf <= -22.4] == 0xFE)
    inf = np.array([0x7F80, 0xFF80], np.uint16)
    assert list(oracle.quant_fp8_static(inf, 0.05)) == [0x7E, 0xFE]
    # exact ties: y / 0.05 in binary32 lands on an E4M3 midpoint; the result
    # must be the even code (checked with exact rationals)
    with np.errstate(over="ignore"):
        z = (yf / np.float32(0.05)).astype(np.float32)
    grid = np.array(sorted(set(oracle.e4m3_table()[:0x7F])))
    mids = (grid[1:] + grid[:-1]) / 2
    ties = np.flatnonzero(np.isin(np.abs(z.astype(np.float64)), mids))
    assert len(ties) > 10
    for i in ties:
        assert q[i] == exact.round_to_e4m3(Fraction(float(z[i])))
        assert q[i] % 2 == 0


def test_per_row_quant_invariants():
    y = gen.normal_bf16((64, 4096), 6, 1, outlier_frac=0.001)
    y[3] = 0                                    # all-zero row
    y[4] = oracle.bf16_from_f64(1e-3)           # tiny row with one outlier
    y[4, 17] = oracle.bf16_from_f64(37.5)
    q, s = oracle.quant_fp8_per_row(y)
    dec = oracle.e4m3_table()
    qa = np.abs(dec[q])
    amax = np.abs(f32_of(y)).max(axis=1)
    for i in range(64):
        if i == 3:
            assert s[i] == 0 and np.all(qa[i] == 0)
            continue
        assert qa[i].max() == 448.0                  # max |q| = 448 exactly
        assert s[i] == np.float32(amax[i]) / np.float32(448)
        assert abs(float(s[i]) * 448 - amax[i]) <= np.spacing(np.float32(amax[i]))
    assert q[4, 17] == 0x7E
    # torch: s = amax / 448, q = clamp(y / s).to(e4m3fn)
    yt = torch.from_numpy(f32_of(y).copy())
    st = yt.abs().amax(dim=1, keepdim=True) / 448.0
    z = torch.where(st == 0, yt, yt / torch.where(st == 0, torch.ones_like(st), st))
    ref = torch.clamp(z, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    assert np.array_equal(s, st.squeeze(1).numpy())


def test_norm_quant_is_composition():
    x = gen.normal_bf16((32, 2048), 8, 1, outlier_frac=0.001)
    r = gen.normal_bf16((32, 2048), 8, 2, outlier_frac=0.001)
    w = gen.normal_bf16((2048,), 8, 3, mean=1.0, std=0.1)
    q, s, res_out, y, rs = oracle.fused_add_rmsnorm_quant_fp8(x, r, w, 1e-5)
    out, res_out2, _ = _norm(x, r, w, 1e-5)
    q2, s2 = oracle.quant_fp8_per_row(out)
    assert np.array_equal(y, out) and np.array_equal(res_out, res_out2)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ------------------------------------------------------------------ the rest of the quant matrix
#
# RMSNorm without the residual add (the first page's Metal norm), the norm
# with a per-tensor (static) E4M3 scale, and SwiGLU with a per-token
# (dynamic) scale: the same steps as above, composed differently.

def test_plain_rmsnorm_constant_row_and_signed_zero():
    H = 1536
    w = gen.normal_bf16((H,), 10, 3, mean=1.0, std=0.1)
    for eps in [1e-6, 1e-5, 0.0]:
        for c in [1.0, -1.0, 0.5, 3.0, -0.0625, 100.0, 2.0 ** -20]:
            if eps and c * c < 512 * eps:
                continue
            x = np.full((2, H), oracle.bf16_from_f64(c), np.uint16)
            out, _ = oracle.rmsnorm(x, w, eps)
            want = w if c > 0 else (w ^ 0x8000)
            assert np.array_equal(out[0], want) and np.array_equal(out[1], want), (c, eps)
    # no add in front: a -0 input reaches the multiply as -0, so out = w * -0
    # (a residual add of +0 would have turned it into +0)
    x = gen.normal_bf16((1, H), 10, 1)
    x[0, :7] = 0x8000
    out, _ = oracle.rmsnorm(x, w, 1e-6)
    want = np.where(f32_of(w[:7]) > 0, 0x8000, 0x0000).astype(np.uint16)
    assert np.array_equal(out[0, :7], want)


def test_plain_rmsnorm_scale_invariance():
    x = gen.normal_bf16((8, 2048), 11, 1)
    w = gen.normal_bf16((2048,), 11, 3, mean=1.0, std=0.1)
    base, _ = oracle.rmsnorm(x, w, 0.0)
    for k in [-9, -2, 1, 5]:
        xs = gen.bf16_bits_from_f32(f32_of(x) * np.float32(2.0 ** k))
        out, _ = oracle.rmsnorm(xs, w, 0.0)
        assert np.array_equal(out, base), k


def test_plain_rmsnorm_matches_torch_eager_eight_ops():
    """torch CPU eager on x itself (no residual): equal except at knife-edges,
    which lie inside the admissible window."""
    T, H, eps = 256, 1536, 1e-6
    x = gen.normal_bf16((T, H), 12, 1, std=2.0)
    w = gen.normal_bf16((H,), 12, 3, mean=1.0, std=0.1)
    out, rs = oracle.rmsnorm(x, w, eps)
    h = bf16_t(x).to(torch.float32)
    hn = h * torch.rsqrt(h.pow(2).mean(-1, keepdim=True) + eps)
    ref = bits_of(bf16_t(w) * hn.to(torch.bfloat16))
    diff = np.flatnonzero(ref.reshape(-1) != out.reshape(-1))
    assert len(diff) < 0.005 * out.size
    _, rs_exact = oracle.rms_scale(x, eps)
    lo, hi = oracle.rms_window(rs_exact, 2.0 ** -18)
    alt_lo = oracle.rmsnorm_apply(x, w, lo).reshape(-1)
    alt_hi = oracle.rmsnorm_apply(x, w, hi).reshape(-1)
    r = ref.reshape(-1)
    assert np.all((r[diff] == alt_lo[diff]) | (r[diff] == alt_hi[diff]))


@pytest.mark.parametrize("scale", [0.05, 0.0125, 1.0])
def test_static_norm_quant_vs_torch(scale):
    """Per-tensor E4M3 on the norm output: the codes are torch's
    clamp(y / scale).to(e4m3fn) of the bf16 norm output, with and without
    the residual add."""
    x = gen.normal_bf16((32, 2048), 13, 1, outlier_frac=0.001)
    r = gen.normal_bf16((32, 2048), 13, 2, outlier_frac=0.001)
    w = gen.normal_bf16((2048,), 13, 3, mean=1.0, std=0.1)
    q, res_out, y, _ = oracle.fused_add_rmsnorm_quant_fp8_static(x, r, w, 1e-5, scale)
    out, res_out2, _ = _norm(x, r, w, 1e-5)
    assert np.array_equal(y, out) and np.array_equal(res_out, res_out2)
    q2, y2, _ = oracle.rmsnorm_quant_fp8_static(x, w, 1e-5, scale)
    assert np.array_equal(y2, oracle.rmsnorm(x, w, 1e-5)[0])
    for qq, yy in ((q, y), (q2, y2)):
        z = torch.clamp(torch.from_numpy(f32_of(yy).copy()) / torch.tensor(scale, dtype=torch.float32), -448, 448)
        assert np.array_equal(qq, z.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    # saturation reached: with scale 0.0125 the largest |y| (about 4) lands
    # beyond 448 and must give the largest code, not NaN
    if scale == 0.0125:
        big = np.abs(f32_of(y)) >= 448 * 0.0125
        assert big.any() and np.all((q[big] & 0x7F) == 0x7E)


def test_dynamic_norm_quant_without_residual():
    x = gen.normal_bf16((32, 4096), 14, 1, outlier_frac=0.001)
    w = gen.normal_bf16((4096,), 14, 3, mean=1.0, std=0.1)
    q, s, y, _ = oracle.rmsnorm_quant_fp8(x, w, 1e-5)
    assert np.array_equal(y, oracle.rmsnorm(x, w, 1e-5)[0])
    amax = np.abs(f32_of(y)).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    assert np.all(np.abs(oracle.e4m3_table()[q]).max(axis=1) == 448.0)


def test_dynamic_swiglu_quant_invariants_and_torch():
    """Per-token E4M3 on the SwiGLU output: s = f32(max|y| / 448), every
    non-zero row reaches 448 exactly, an all-zero row gives s = 0 and zero
    codes, and the codes are torch's conversion of clamp(y / s)."""
    T, N = 64, 4096
    gu = gen.normal_bf16((T, 2 * N), 15, 4, std=2.0)
    gu[5, :N] = 0                                  # gate 0: silu = 0, y = +-0
    gu[6, :N] = oracle.bf16_from_f64(0.01)         # small row with one large output
    gu[6, 100] = oracle.bf16_from_f64(12.0)
    gu[6, N + 100] = oracle.bf16_from_f64(5.0)
    q, s, y = oracle.swiglu_quant_fp8_dynamic(gu)
    assert np.array_equal(y, oracle.swiglu(gu))
    yf = f32_of(y)
    amax = np.abs(yf).max(axis=1)
    qa = np.abs(oracle.e4m3_table()[q])
    for i in range(T):
        if i == 5:
            assert s[i] == 0 and np.all(qa[i] == 0)
            continue
        assert s[i] == np.float32(amax[i]) / np.float32(448)
        assert qa[i].max() == 448.0
    assert q[6, 100] == 0x7E
    yt = torch.from_numpy(yf.copy())
    st = yt.abs().amax(dim=1, keepdim=True) / 448.0
    z = torch.where(st == 0, yt, yt / torch.where(st == 0, torch.ones_like(st), st))
    ref = torch.clamp(z, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


# ------------------------------------------------------------------ MXFP4

E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e2m1_brute(v: float) -> int:
    """Nearest E2M1 magnitude by search (ties to the even code), saturating."""
    a = min(abs(v), 6.0)
    d = [abs(a - g) for g in E2M1_GRID]
    best = min(d)
    cands = [i for i, x in enumerate(d) if x == best]
    code = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return code | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_values_and_rounding_exhaustive():
    assert [oracle.e2m1_to_f64(q) for q in range(8)] == E2M1_GRID
    assert [oracle.e2m1_to_f64(q | 8) for q in range(8)] == [-g for g in E2M1_GRID]
    # every finite bf16, scaled into the E2M1 range by a few powers of two
    f = f32_of(FINITE_BF16).astype(np.float64)
    for k in (0, -3, 3):
        v = np.ldexp(f, k)
        v = v[np.abs(v) < 16]
        for x in v:
            assert oracle.e2m1_from_f64(float(x)) == _e2m1_brute(float(x)), x
    # the ties exactly
    for t, want in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6), (7.0, 7)]:
        assert oracle.e2m1_from_f64(t) == want and oracle.e2m1_from_f64(-t) == want | 8


def test_e8m0_decode_matches_torch():
    b = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    mine = np.array([oracle.e8m0_to_f64(int(x)) for x in b])
    # torch decodes byte 0 as 2^-127 like every other byte
    assert np.array_equal(mine, ref)
    assert math.isnan(oracle.e8m0_to_f64(255))


def test_mxfp4_scale_rule_and_nearest_elements():
    """Per 32-value block: 4 X <= amax < 8 X for the power of two X the scale
    byte encodes, the block's largest element is at 4 or 6 (times X), and
    every element decodes to the nearest point of X times the E2M1 grid
    (ties to the even code, saturating at 6 X)."""
    rng = np.random.default_rng(7)
    rows = []
    for k in (-20, -5, 0, 3, 9, 40):
        rows.append(gen.bf16_bits_from_f32((rng.standard_normal(256) * 2.0 ** k).astype(np.float32)))
    y = np.stack(rows)
    q, s = oracle.quant_mxfp4(y)
    X = np.array([[oracle.e8m0_to_f64(int(b)) for b in r] for r in s])
    yf = f32_of(y).astype(np.float64).reshape(len(rows), -1, 32)
    amax = np.abs(yf).max(axis=2)
    assert np.all(4 * X <= amax) and np.all(amax < 8 * X)
    dec = oracle.mxfp4_decode(q, s).reshape(yf.shape)
    assert np.all(np.isin(np.abs(dec).max(axis=2) / X, [4.0, 6.0]))
    for r in range(len(rows)):
        for b in range(yf.shape[1]):
            for i in range(32):
                want = _e2m1_brute(yf[r, b, i] / X[r, b])
                code = (q[r, b * 16 + i // 2] >> (4 * (i % 2))) & 0xF
                assert code == want or (code & 7) == (want & 7) == 0, (r, b, i)


def test_mxfp4_packing_zero_and_special_blocks():
    one = oracle.bf16_from_f64
    y = np.zeros((3, 64), np.uint16)
    y[0, 0], y[0, 1] = one(1.0), one(6.0)          # X = 2^(2 - 2) = 1: codes 2 (1.0) and 7 (6.0)
    y[1, 32 + 5] = 0x7FC0                          # NaN in the second block
    y[2, 3] = 0x7F80                               # +inf
    q, s = oracle.quant_mxfp4(y)
    assert q[0, 0] == 0x72                         # first element in the low nibble
    assert s[0, 0] == 127 and s[0, 1] == 0         # all-zero block: smallest scale
    assert np.all(q[0, 16:] == 0)
    assert s[1, 0] == 0 and s[1, 1] == 0xFF and s[2, 0] == 0xFF
    assert np.all(q[1, 16:] == 0) and np.all(q[2, :16] == 0)


def test_mxfp4_norm_is_composition():
    x = gen.normal_bf16((16, 2048), 16, 1, outlier_frac=0.001)
    r = gen.normal_bf16((16, 2048), 16, 2)
    w = gen.normal_bf16((2048,), 16, 3, mean=1.0, std=0.1)
    q, s, res_out, y, _ = oracle.fused_add_rmsnorm_quant_mxfp4(x, r, w, 1e-5)
    out, res2, _ = _norm(x, r, w, 1e-5)
    assert np.array_equal(y, out) and np.array_equal(res_out, res2)
    q2, s2 = oracle.quant_mxfp4(out)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    q3, s3, y3, _ = oracle.rmsnorm_quant_mxfp4(x, w, 1e-5)
    assert np.array_equal(y3, oracle.rmsnorm(x, w, 1e-5)[0])
    gu = gen.normal_bf16((8, 2 * 1024), 16, 4, std=2.0)
    q4, s4, y4 = oracle.swiglu_quant_mxfp4(gu)
    assert np.array_equal(y4, oracle.swiglu(gu))
    q5, s5 = oracle.quant_mxfp4(y4)
    assert np.array_equal(q4, q5) and np.array_equal(s4, s5)


# ------------------------------------------------------------------ NVFP4

@pytest.mark.parametrize("g", [0.01, 1.0, 3.0e-4, 0.0])
def test_nvfp4_scales_and_elements_vs_numpy_and_exact(g):
    """Block scale: the E4M3 nearest (exact rationals) to numpy's binary32
    amax / (6 g), saturated at 448; elements: brute-force E2M1 of numpy's
    binary32 v / (scale * g).  g = 0 behaves as 1."""
    rng = np.random.default_rng(11)
    rows = [gen.bf16_bits_from_f32((rng.standard_normal(128) * 2.0 ** k).astype(np.float32)) for k in (-12, 0, 6)]
    y = np.stack(rows)
    y[1, 16:32] = 0                                 # a zero block: scale 0, signed-zero codes
    q, s = oracle.quant_nvfp4(y, g)
    gg = np.float32(g) if g else np.float32(1.0)
    six_g = np.float32(6.0) * gg
    yf = f32_of(y).reshape(len(rows), -1, 16)
    e4m3 = oracle.e4m3_table()
    for r in range(len(rows)):
        for b in range(yf.shape[1]):
            amax = np.float32(np.abs(yf[r, b]).max())
            t = np.float32(amax / six_g)
            t = min(t, np.float32(448.0))
            assert s[r, b] == exact.round_to_e4m3(Fraction(float(t))), (r, b)
            S = np.float32(np.float32(e4m3[s[r, b]]) * gg)
            for i in range(16):
                v = np.float32(yf[r, b, i])
                z = np.float32(v * np.float32(0.0)) if S == 0 else np.float32(v / S)
                code = (q[r, b * 8 + i // 2] >> (4 * (i % 2))) & 0xF
                assert code == _e2m1_brute(float(z)), (r, b, i)
    assert s[1, 1] == 0 and np.all((q[1, 8:16] & 0x77) == 0)


def test_nvfp4_special_blocks_and_composition():
    one = oracle.bf16_from_f64
    y = np.zeros((2, 64), np.uint16)
    y[0, 3] = 0x7FC0                                # NaN block
    y[1, 20] = 0xFF80                               # -inf block
    y[1, 40] = one(600.0)                           # amax / (6 g) beyond 448: saturated scale
    q, s = oracle.quant_nvfp4(y, 0.1)
    assert s[0, 0] == 0x7F and np.all(q[0, :8] == 0)
    assert s[1, 1] == 0x7F and s[1, 2] == 0x7E
    assert (q[1, 20] & 0xF) == 0x7                  # 600 / (448 * 0.1) > 6: saturates at 6
    x = gen.normal_bf16((8, 1024), 17, 1)
    r = gen.normal_bf16((8, 1024), 17, 2)
    w = gen.normal_bf16((1024,), 17, 3, mean=1.0, std=0.1)
    q1, s1, ro, yy, _ = oracle.fused_add_rmsnorm_quant_nvfp4(x, r, w, 1e-5, 0.02)
    assert np.array_equal(yy, _norm(x, r, w, 1e-5)[0])
    q2, s2 = oracle.quant_nvfp4(yy, 0.02)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    gu = gen.normal_bf16((4, 2 * 512), 17, 4, std=2.0)
    q3, s3, y3 = oracle.swiglu_quant_nvfp4(gu, 0.05)
    assert np.array_equal(y3, oracle.swiglu(gu))
    dec = oracle.nvfp4_decode(q3, s3, 0.05)
    yf = f32_of(y3).astype(np.float64)
    # a block's largest value is represented within one E2M1 step of its scale
    blk = np.abs(yf).reshape(4, -1, 16).max(axis=2)
    db = np.abs(dec).reshape(4, -1, 16).max(axis=2)
    sc = oracle.e4m3_table()[s3] * 0.05
    assert np.all(np.abs(db - blk) <= 2 * sc + 1e-12)


# ------------------------------------------------------------------ the pages' shapes

def test_golden_workload_shapes_from_pages():
    """Shapes and byte counts the first page prints, against the workloads."""
    with open(os.path.join(GOLDEN, "pages_workloads.json")) as f:
        gold = json.load(f)
    from workloads import configs as C
    q = gold["qwen2.5-1.5b"]
    assert C.NORM_PREFILL4096.hidden == q["hidden"]
    assert C.SWIGLU_PREFILL4096.inter == q["intermediate"]
    assert C.DECODE_GRAPH.layers == q["layers"]
    tune = gold["rmsnorm_tuning"]
    # the tuning study gives 25 MB moved by every variant at 4,096 rows of
    # 1,536 fp16: one read and one write of the rows
    moved = tune["rows"][-1] * tune["hidden"] * 2 * 2
    assert round(moved / 1e6) == tune["megabytes_moved_at_4096_rows"]
    prefill = gold["prefill_intermediate"]
    assert prefill["rows"] * prefill["cols"] == 2048 * C.SWIGLU_PREFILL4096.inter


# ------------------------------------------------------------------ per-group FP8

def _torch_group_quant(yf: np.ndarray, G: int):
    """torch: per group of G values, s = amax / 448, q = clamp(y / s) -> E4M3."""
    T, H = yf.shape
    yt = torch.from_numpy(yf.copy()).reshape(T, H // G, G)
    st = yt.abs().amax(dim=2, keepdim=True) / 448.0
    z = torch.where(st == 0, yt, yt / torch.where(st == 0, torch.ones_like(st), st))
    q = torch.clamp(z, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(T, H).numpy()
    return q, st.reshape(T, H // G).numpy()


def test_per_group_quant_against_torch_and_invariants():
    """Per-group (block) E4M3, groups of 128: every non-zero group reaches 448
    exactly, its scale is f32(amax / 448), all-zero groups give s = 0 and zero
    codes; the codes equal torch's per-group clamp-and-convert."""
    G = oracle.FP8_GROUP
    assert G == 128
    y = gen.normal_bf16((16, 1024), 21, 1, outlier_frac=0.001)
    y[2, 128:256] = 0                                  # one all-zero group
    y[3, :] = oracle.bf16_from_f64(1e-3)
    y[3, 300] = oracle.bf16_from_f64(37.5)             # one outlier in group 2 only
    q, s = oracle.quant_fp8_per_group(y)
    assert q.shape == y.shape and s.shape == (16, 1024 // G)
    yf = f32_of(y)
    amax = np.abs(yf).reshape(16, -1, G).max(axis=2)
    qa = np.abs(oracle.e4m3_table()[q]).reshape(16, -1, G)
    assert s[2, 1] == 0 and np.all(qa[2, 1] == 0)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz].astype(np.float32) / np.float32(448)).astype(np.float32))
    assert np.all(qa.max(axis=2)[nz] == 448.0)
    assert q[3, 300] == 0x7E and s[3, 2] == np.float32(37.5) / np.float32(448)
    assert s[3, 0] == np.float32(oracle.bf16_to_f32(oracle.bf16_from_f64(1e-3))) / np.float32(448)
    qt, st = _torch_group_quant(yf, G)
    assert np.array_equal(q, qt) and np.array_equal(s, st)


def test_per_group_quant_reduces_to_per_row_and_catches_swapped_groups():
    y = gen.normal_bf16((8, 512), 22, 1, std=3.0)
    # one group the width of the row is the per-token form
    qg, sg = oracle.quant_fp8_per_group(y, 512)
    qr, sr = oracle.quant_fp8_per_row(y)
    assert np.array_equal(qg, qr) and np.array_equal(sg[:, 0], sr)
    # per-group codes differ from per-row codes (the scales are the groups')
    q, s = oracle.quant_fp8_per_group(y)
    assert not np.array_equal(q, qr)
    # a group quantised with its neighbour's scale is wrong somewhere
    yf = f32_of(y)
    swapped = np.concatenate([s[:, 1:2], s[:, 0:1], s[:, 2:]], axis=1)
    z = yf / np.repeat(swapped, 128, axis=1)
    wrong = torch.from_numpy(np.clip(z, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(q, wrong)


def test_per_group_quant_exact_on_a_small_case():
    """Brute force: q = nearest-even E4M3 of the binary32 quotient y / s, with
    s the binary32 rounding of amax / 448, all in exact rationals."""
    y = gen.normal_bf16((3, 256), 23, 1, std=5.0)
    y[1, 5] = oracle.bf16_from_f64(-300.0)
    q, s = oracle.quant_fp8_per_group(y)
    yf = f32_of(y)
    for r in range(3):
        for g in range(2):
            vals = [Fraction(float(v)) for v in yf[r, g * 128:(g + 1) * 128]]
            amax = max(abs(v) for v in vals)
            sc = exact.round_to_f32(amax / 448)
            assert float(s[r, g]) == sc
            for j, v in enumerate(vals):
                z = exact.round_to_f32(v / Fraction(sc))
                z = max(min(Fraction(z), Fraction(448)), Fraction(-448))
                code = exact.round_to_e4m3(z)              # sign bit included
                got = int(q[r, g * 128 + j])
                if z == 0:
                    assert got & 0x7F == 0                     # a signed zero
                else:
                    assert got == code


def test_per_group_quant_special_values():
    y = np.full((2, 256), oracle.bf16_from_f64(0.5), np.uint16)
    y[0, 3] = 0x7FC0                                   # NaN: ignored by the group amax, stays NaN
    y[1, 130] = 0x7F80                                 # +inf: the group's scale is inf
    q, s = oracle.quant_fp8_per_group(y)
    assert s[0, 0] == np.float32(0.5) / np.float32(448) and (q[0, 3] & 0x7F) == 0x7F
    assert q[0, 4] == 0x7E                              # 0.5 / s = 448
    assert np.isinf(s[1, 1]) and s[1, 0] == np.float32(0.5) / np.float32(448)
    assert np.all((q[1, 128:256] & 0x7F)[np.arange(128) != 2] == 0)   # finite / inf = 0
    assert (q[1, 130] & 0x7F) == 0x7F                   # inf / inf = NaN


def test_per_group_compositions():
    x = gen.normal_bf16((16, 1024), 24, 1)
    r = gen.normal_bf16((16, 1024), 24, 2)
    w = gen.normal_bf16((1024,), 24, 3, mean=1.0, std=0.1)
    q, s, ro, y, _ = oracle.fused_add_rmsnorm_quant_fp8_group(x, r, w, 1e-5)
    out, ro2, _ = oracle.fused_add_rmsnorm(x, r, w, 1e-5)
    assert np.array_equal(y, out) and np.array_equal(ro, ro2)
    assert all(np.array_equal(a, b) for a, b in zip((q, s), oracle.quant_fp8_per_group(out)))
    q, s, y, _ = oracle.rmsnorm_quant_fp8_group(x, w, 1e-5)
    assert np.array_equal(y, oracle.rmsnorm(x, w, 1e-5)[0])
    gu = gen.normal_bf16((8, 2048), 24, 4, std=2.0)
    q, s, y = oracle.swiglu_quant_fp8_group(gu)
    assert np.array_equal(y, oracle.swiglu(gu)) and s.shape == (8, 1024 // 128)
    assert all(np.array_equal(a, b) for a, b in zip((q, s), oracle.quant_fp8_per_group(y)))
