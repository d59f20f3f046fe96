// device.h -- gfx950 device helpers shared by the norm and SwiGLU kernels:
// bf16 / E4M3 packing, wave and block reductions, the SiLU evaluation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace aarms {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Streaming accesses: every tensor except the weight is read or written
// exactly once, so loads and stores carry the non-temporal hint (the data is
// not kept in the caches for reuse that will not come).
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_stream(T *p, T v) { __builtin_nontemporal_store(v, p); }

// The block's index in the launch's row of blocks (linear_grid): a scalar.
__device__ __forceinline__ int64_t linear_block()
{
    return ((int64_t)blockIdx.y << LINEAR_GRID_SHIFT) + (int64_t)blockIdx.x;
}

// A 16-byte vector holds 8 bf16 values: element 2e is the low half of word
// e, element 2e+1 the high half.  Widening bf16 -> binary32 is exact.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two binary32 -> one word of two bf16, round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    bf16x2 r = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// The binary32 value of bf16(a).  Rounding to nearest is monotone and
// symmetric, so the bf16 rounding of the largest |p| of a set of binary32
// values is the largest |bf16(p)|: maxima of rounded outputs are taken on the
// products before their rounding and rounded once.
__device__ __forceinline__ float round_bf16(float a)
{
    return bf_lo(pack_bf16(a, a));
}

// Saturate to the E4M3 range, keeping NaN: the conversion below turns
// anything beyond 464 into NaN, and v_med3_f32 drops a NaN operand.
__device__ __forceinline__ float clamp_e4m3(float z)
{
    float c = __builtin_amdgcn_fmed3f(z, -448.0f, 448.0f);
    return (z != z) ? z : c;
}

// Four binary32 already inside [-448, 448] (or NaN) -> four OCP E4M3 bytes,
// round to nearest even (v_cvt_pk_fp8_f32), first value in the lowest byte.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d)
{
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return (uint32_t)v;
}

// ---------------------------------------------------------------- row scale
//
// The row statistics as the unfused definition computes them in binary64,
// mean = binary32(acc / n) and rs = binary32(1 / sqrt(v)), without the
// binary64 division and square-root sequences (about 40 instructions per
// wave, run by every wave of a row).
//  - row_mean: q0 = acc * inv_n with inv_n = binary64(1 / n), then one
//    correction from the exact remainder acc - q0 n (an fma).  With inv_n
//    correctly rounded and q0 within an ulp, the corrected quotient is the
//    correctly rounded one (Markstein's theorem), so the result is
//    binary32(binary64(acc / n)) exactly.  Finite acc (the caller branches).
//  - row_rsqrt: r0 = v_rsq_f32(v), then two Newton steps
//    r <- r + r (1 - v r^2) / 2 in binary64 (r0 is within about 2^-22; the
//    steps leave an error of a few units of 2^-53, as the division of the
//    unfused form has), rounded once to binary32.  Normal v in
//    [2^-126, 2^126) (the caller branches).
__device__ __forceinline__ float row_mean(double acc, double n, double inv_n)
{
    const double q0 = acc * inv_n;
    const double rem = __builtin_fma(-q0, n, acc);
    return (float)__builtin_fma(rem, inv_n, q0);
}

__device__ __forceinline__ bool row_rsqrt_in_range(float v)
{
    return v >= 0x1p-126f && v < 0x1p126f;
}

__device__ __forceinline__ float row_rsqrt(float v)
{
    const double vd = v;
    double r = (double)__builtin_amdgcn_rsqf(v);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const double e = __builtin_fma(-(vd * r), r, 1.0);
        r = __builtin_fma(0.5 * r, e, r);
    }
    return (float)r;
}

// ---------------------------------------------------------------- MXFP4
//
// A block of 32 values shares the E8M0 scale 2^x with x = floor(log2 amax)
// - 2 clamped to [-127, 127]; each value v becomes E2M1(v / 2^x), rounded
// to nearest even and saturated at +-6.  From the binary32 bits of amax
// (exponent field e): x + 127 = max(e, 2) - 2, which also gives 2^-127 for
// a zero or binary32-subnormal amax; amax non-finite marks the block with
// the E8M0 NaN byte 0xFF.  v / 2^x is computed as v * 2^-x: 2^-x is a
// normal binary32 for every x here (x <= 125) and the product is exact
// unless it falls far below the smallest E2M1 step, where the code is a
// signed zero either way.  v_cvt_scalef32_pk_fp4_f32 (scale operand 1.0)
// does the rounding and saturation and packs the first value into the low
// nibble (checked on gfx950 at every rounding tie and past 6).

__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits)
{
    if (amax_bits >= 0x7F800000u) return 0xFFu;
    const uint32_t e = amax_bits >> 23;
    return (e > 2u ? e : 2u) - 2u;
}

// Eight values (four bf16 words) -> four bytes of E2M1 pairs, scaled by
// 2^-x given as its binary32 value.
__device__ __forceinline__ uint32_t pack_e2m1x8(const uint32_t (&w)[4], float inv_scale)
{
    uint32_t q = 0;
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, bf_lo(w[0]) * inv_scale, bf_hi(w[0]) * inv_scale, 1.0f, 0);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, bf_lo(w[1]) * inv_scale, bf_hi(w[1]) * inv_scale, 1.0f, 1);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, bf_lo(w[2]) * inv_scale, bf_hi(w[2]) * inv_scale, 1.0f, 2);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, bf_lo(w[3]) * inv_scale, bf_hi(w[3]) * inv_scale, 1.0f, 3);
    return q;
}

// ---------------------------------------------------------------- y / scale
//
// q = e4m3(clamp(binary32(y / s), -448, 448)).  A scale of exactly zero is
// treated as one.  For a scale in [2^-126, 2^118] (the usual case):
//   - y is first clamped to +-lim, lim = binary32(448 s), with the
//     NaN-propagating v_maximum3/v_minimum3: a NaN stays NaN, an infinity or
//     any |y| beyond lim gives a quotient that rounds to +-448, and no
//     quotient can overflow binary32;
//   - the quotient is y * inv (inv = binary32(1/s)), within an ulp, plus one
//     correction step from the exact remainder q0 s - y (one fma), which
//     rounds it to the nearest binary32 quotient.
// Outside that range, or for a negative scale, the IEEE division is used (a
// uniform branch).
struct E4m3Scale {
    float s, inv, lim;
};

__device__ __forceinline__ E4m3Scale make_e4m3_scale(float s)
{
    E4m3Scale q;
    q.s = (s == 0.0f) ? 1.0f : s;
    q.inv = 1.0f / q.s;
    q.lim = __builtin_fabsf(448.0f * q.s);
    return q;
}

__device__ __forceinline__ bool e4m3_scale_is_fast(const E4m3Scale &q)
{
    return q.s >= 0x1p-126f && q.s <= 0x1p118f;
}

// CLAMP = false is for per-token scales s = binary32(amax / 448), where every
// |y| <= amax gives |y / s| <= 448 (1 + 2^-24) and the input clamp is moot.
template <bool FAST, bool CLAMP = true>
__device__ __forceinline__ float e4m3_quotient(float y, const E4m3Scale &q)
{
    if constexpr (FAST) {
        float yc = y;
        if constexpr (CLAMP)
            yc = __builtin_elementwise_minimum(__builtin_elementwise_maximum(y, -q.lim), q.lim);
        const float q0 = yc * q.inv;
        // rem = q0 s - y is exact; z = q0 - rem * inv.  Written this way round
        // (rather than y - q0 s) so that a zero quotient keeps the sign of y.
        const float rem = __builtin_fmaf(q0, q.s, -yc);
        return __builtin_fmaf(rem, -q.inv, q0);
    } else {
        return clamp_e4m3(y / q.s);
    }
}

// ---------------------------------------------------------------- NVFP4
//
// A block of 16 values shares an E4M3 scale under the fp32 tensor scale g
// (0 means 1): scale = E4M3(binary32(amax / binary32(6 g))), nearest even,
// saturated at 448 (v_cvt_pk_fp8_f32 after a clamp); each value becomes
// E2M1(binary32(v / S)), S = binary32(scale * g), or a signed zero when S is
// 0; a block holding a NaN or an infinity gets the E4M3 NaN 0x7F and zero
// codes.  Both quotients are the correctly rounded ones of the E4M3 path
// (e4m3_quotient).

struct Nvfp4Tensor {
    float g;
    E4m3Scale six;           // 6 g, as the divisor of the block amax
    bool six_fast;
};

// The tensor scale as used (0 means 1), and the reciprocal of 6 g that the
// block-scale quotient takes (make_e4m3_scale's divisor and reciprocal).
__device__ __forceinline__ float nv_tensor_scale(float g)
{
    return (g == 0.0f) ? 1.0f : g;
}

__device__ __forceinline__ float nv_six_inverse(float g)
{
    return make_e4m3_scale(6.0f * nv_tensor_scale(g)).inv;
}

// six_inv = nv_six_inverse(g), passed in so that a block can compute it once.
__device__ __forceinline__ Nvfp4Tensor make_nvfp4_tensor(float g, float six_inv)
{
    Nvfp4Tensor t;
    t.g = nv_tensor_scale(g);
    const float s6 = 6.0f * t.g;
    t.six.s = (s6 == 0.0f) ? 1.0f : s6;
    t.six.inv = six_inv;
    t.six.lim = __builtin_fabsf(448.0f * t.six.s);
    t.six_fast = e4m3_scale_is_fast(t.six);
    return t;
}

__device__ __forceinline__ Nvfp4Tensor make_nvfp4_tensor(float g)
{
    return make_nvfp4_tensor(g, nv_six_inverse(g));
}

// E4M3 block scale: binary32(amax / 6g) (the correctly rounded quotient of
// the E4M3 path, its input clamped at 448 * 6g so nothing overflows),
// saturated at 448, rounded to nearest even.
__device__ __forceinline__ uint32_t nv_scale_byte(uint32_t amax_bits, const Nvfp4Tensor &t)
{
    if (amax_bits >= 0x7F800000u) return 0x7Fu;
    const float a = __uint_as_float(amax_bits);
    const float q = t.six_fast ? e4m3_quotient<true>(a, t.six) : e4m3_quotient<false>(a, t.six);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q, 0.0f, 448.0f), 0.0f, 0, false) &
           0xFFu;
}

// NW bf16 words (2 NW values) of one block -> NW bytes of E2M1 pairs, the
// first value of each pair in the low nibble.  Unless the block scale
// saturated (448), every |v| / S stays below about 12, so the quotient needs
// no input clamp; a saturated block takes the clamped form (its values can
// be arbitrarily large against S).
template <int NW, bool CLAMP>
__device__ __forceinline__ void nv_quotients(const uint32_t (&w)[NW], const E4m3Scale &qs, bool fast,
                                             float (&z)[2 * NW])
{
#pragma unroll
    for (int e = 0; e < NW; ++e) {
        const float v0 = bf_lo(w[e]), v1 = bf_hi(w[e]);
        if (fast) {
            z[2 * e] = e4m3_quotient<true, CLAMP>(v0, qs);
            z[2 * e + 1] = e4m3_quotient<true, CLAMP>(v1, qs);
        } else {
            z[2 * e] = e4m3_quotient<false, CLAMP>(v0, qs);
            z[2 * e + 1] = e4m3_quotient<false, CLAMP>(v1, qs);
        }
    }
}

// The block divisor S = binary32(E4M3(sb) * g) and its reciprocal as the
// fast quotient takes it: binary32(1 / S), or 0 when S is 0.  With divisor 1
// and reciprocal 0 the fast quotient returns the zero of v's sign for every
// finite v (q0 = v * 0, rem = -v, z = -v * -0 + q0), which is what a block
// whose scale is zero encodes, so no per-value select is needed.
__device__ __forceinline__ float nv_block_divisor(uint32_t sb, float g)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)sb, 0) * g;
}

// g as used (nv_tensor_scale)
__device__ __forceinline__ float nv_block_inverse(uint32_t sb, float g)
{
    const float S = nv_block_divisor(sb, g);
    return S == 0.0f ? 0.0f : 1.0f / S;
}

// inv = nv_block_inverse(sb, t), passed in so that a caller can take it from
// a table of the 127 finite block scales.
template <int NW>
__device__ __forceinline__ uint32_t pack_nvfp4(const uint32_t (&w)[NW], uint32_t sb, const Nvfp4Tensor &t, float inv)
{
    static_assert(NW == 2 || NW == 4, "2 or 4 words");
    const float S = nv_block_divisor(sb, t.g);
    E4m3Scale qs;
    qs.s = (S == 0.0f) ? 1.0f : S;
    qs.inv = inv;
    qs.lim = __builtin_fabsf(448.0f * qs.s);
    const bool fast = e4m3_scale_is_fast(qs);
    float z[2 * NW];
    if (sb == 0x7Eu)
        nv_quotients<NW, true>(w, qs, fast, z);
    else
        nv_quotients<NW, false>(w, qs, fast, z);
    // the byte selector of the conversion is an immediate
    uint32_t q = 0;
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, z[0], z[1], 1.0f, 0);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, z[2], z[3], 1.0f, 1);
    if constexpr (NW == 4) {
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, z[4], z[5], 1.0f, 2);
        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, z[6], z[7], 1.0f, 3);
    }
    return q;
}

// Butterfly sums and maxima over the 64 lanes of a wave, entirely in VALU
// lane permutations (no LDS round trips, which dominate a lone row's latency).
// Each step combines v with its value on a partner lane, and every
// permutation used is an involution that pairs lanes: lane ^ 1 and lane ^ 2
// (DPP quad_perm), 7 - lane within 8 (row_half_mirror, pairs the two
// quads), 15 - lane within 16 (row_mirror, pairs the two halves of a
// row), then the two 16-lane rows of each 32-lane half and the two halves
// (v_permlane16_swap / v_permlane32_swap, which hand every lane both
// operands in the same order).  So every lane ends with the same bits.
// Every lane's source lane exists under these permutations, so the move
// needs no fill value and bound_ctrl (zero for a missing source) never
// applies; without a fill value the compiler folds the move into the
// integer maxima below (v_max_u32 with DPP) and drops a register
// initialisation per step of the sums.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, (hi << 32) | lo);
}

constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // row_half_mirror
constexpr int DPP_MIRROR = 0x140;      // row_mirror

// (a, b) with a = the value of the lower 16-lane row (32-lane half) of each
// pair and b = the upper one, on every lane of the pair.
template <int SPAN>
__device__ __forceinline__ void swap_pair_u32(uint32_t v, uint32_t &a, uint32_t &b)
{
    if constexpr (SPAN == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = r[0];
        b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = r[0];
        b = r[1];
    }
}

template <int SPAN>
__device__ __forceinline__ double swap_sum_f64(double v)
{
    const uint64_t bits = __builtin_bit_cast(uint64_t, v);
    uint32_t alo, blo, ahi, bhi;
    swap_pair_u32<SPAN>((uint32_t)bits, alo, blo);
    swap_pair_u32<SPAN>((uint32_t)(bits >> 32), ahi, bhi);
    const double a = __builtin_bit_cast(double, ((uint64_t)ahi << 32) | alo);
    const double b = __builtin_bit_cast(double, ((uint64_t)bhi << 32) | blo);
    return a + b;
}

__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_f64<DPP_XOR1>(v);
    v += dpp_f64<DPP_XOR2>(v);
    v += dpp_f64<DPP_HALF_MIRROR>(v);
    v += dpp_f64<DPP_MIRROR>(v);
    v = swap_sum_f64<16>(v);
    return swap_sum_f64<32>(v);
}

// Maxima of non-negative, non-NaN binary32 values (magnitudes folded with
// fmaxf from 0, which drops NaN).  For those, the order of the bit patterns
// as unsigned integers is the order of the values, so the butterflies take
// integer maxima: the same result as fmaxf, without the NaN quieting that a
// floating-point maximum of a permuted lane needs first.
__device__ __forceinline__ uint32_t max_dpp_step(uint32_t v, uint32_t w) { return v > w ? v : w; }

template <int SPAN>
__device__ __forceinline__ uint32_t swap_max_u32(uint32_t v)
{
    uint32_t a, b;
    swap_pair_u32<SPAN>(v, a, b);
    return max_dpp_step(a, b);
}

__device__ __forceinline__ float wave_max(float x)
{
    uint32_t v = __float_as_uint(x);
    v = max_dpp_step(v, dpp_u32<DPP_XOR1>(v));
    v = max_dpp_step(v, dpp_u32<DPP_XOR2>(v));
    v = max_dpp_step(v, dpp_u32<DPP_HALF_MIRROR>(v));
    v = max_dpp_step(v, dpp_u32<DPP_MIRROR>(v));
    v = swap_max_u32<16>(v);
    return __uint_as_float(swap_max_u32<32>(v));
}

// Maximum over each group of 16 adjacent lanes (one DPP row), or with
// LANES == 32 over each aligned pair of rows, of non-negative non-NaN
// values (the group amax, NaN already dropped).  Every lane of a group ends
// with the group's value.
template <int LANES>
__device__ __forceinline__ float group_max(float x)
{
    static_assert(LANES == 16 || LANES == 32, "one or two DPP rows");
    uint32_t v = __float_as_uint(x);
    v = max_dpp_step(v, dpp_u32<DPP_XOR1>(v));
    v = max_dpp_step(v, dpp_u32<DPP_XOR2>(v));
    v = max_dpp_step(v, dpp_u32<DPP_HALF_MIRROR>(v));
    v = max_dpp_step(v, dpp_u32<DPP_MIRROR>(v));
    if constexpr (LANES == 32) v = swap_max_u32<16>(v);
    return __uint_as_float(v);
}

// Cross-wave combine of a block's per-wave partials in LDS (N <= 16 of them):
// lane i < N of every wave reads partial i, a 16-lane butterfly (same
// involutions as above) combines them, and lane 0's value is broadcast.
// Every wave runs the same steps on the same data, so every lane of the
// block ends with the same bits; registers hold one partial, not N.
template <int N>
__device__ __forceinline__ double block_sum(const double *part, int wave_lane)
{
    static_assert(N >= 1 && N <= 16, "up to 16 waves");
    double v = (wave_lane < N) ? part[wave_lane] : 0.0;
    v += dpp_f64<DPP_XOR1>(v);
    v += dpp_f64<DPP_XOR2>(v);
    v += dpp_f64<DPP_HALF_MIRROR>(v);
    v += dpp_f64<DPP_MIRROR>(v);
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 0);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 0);
    return __builtin_bit_cast(double, (hi << 32) | lo);
}

// The same for maxima of non-negative non-NaN values, integer maxima of the
// bit patterns as in wave_max (absent partials read as 0).
template <int N>
__device__ __forceinline__ float block_max(const float *part, int wave_lane)
{
    static_assert(N >= 1 && N <= 16, "up to 16 waves");
    uint32_t v = (wave_lane < N) ? __float_as_uint(part[wave_lane]) : 0u;
    v = max_dpp_step(v, dpp_u32<DPP_XOR1>(v));
    v = max_dpp_step(v, dpp_u32<DPP_XOR2>(v));
    v = max_dpp_step(v, dpp_u32<DPP_HALF_MIRROR>(v));
    v = max_dpp_step(v, dpp_u32<DPP_MIRROR>(v));
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 0));
}

// ---------------------------------------------------------------- SiLU
//
// bf16(silu(g)) must be the correctly rounded value.  The fast form below,
// g * rcp(1 + 2^(-g*log2 e)) with the hardware exp2 and reciprocal, is within
// a few units of binary32 rounding of silu(g) (analytically below 31 units
// for g >= -16; measured on gfx950 over all 65,536 gates: within 14 units
// for g in [-16, -8) and within 4 for |g| <= 4).  Because the gate is a bf16,
// the fast form is a function of 16 bits and its bf16 rounding can be
// checked against the correctly rounded value for every input: on gfx950 the
// only gates it misrounds with g >= -16 are those whose binary32 result is
// an exact bf16 midpoint (subnormal gates, where silu(g) = g/2 + g^2/4 and
// binary32 loses the g^2/4).  So a lane is recomputed by silu_exact() when
// its result lies within SILU_EDGE units of a midpoint (the low 16 bits near
// 0x8000) or when g < -16; everything else keeps the fast value.  The
// exhaustive check runs on the shipped kernel through the public API in the
// GPU parity tests.  A window this narrow is taken by about one element in
// 20,000-40,000 for normally distributed gates, so the exact path costs
// almost nothing; a window as wide as the analytic bound would send most
// waves through it.

constexpr uint32_t SILU_EDGE = 2;
// g < -16 (or g is a negative NaN) exactly when the bit pattern of g, read
// as unsigned, exceeds that of -16.0; integer compares cannot be upset by a
// signalling NaN the way a floating-point minimum can.
constexpr uint32_t SILU_FAST_MIN_BITS = 0xC1800000u;

__device__ __forceinline__ float silu_fast(float g)
{
    float e = __builtin_amdgcn_exp2f(g * -1.44269502162933349609375f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Knife-edge key of a binary32 result s: with l = the low 16 bits of s (its
// position between two bf16 values, 0x8000 being the rounding midpoint),
// key = ((l + SILU_EDGE - 0x8000) mod 2^16) << 16, which is at most
// SILU_EDGE_KEY_MAX exactly when |l - 0x8000| <= SILU_EDGE.  One
// v_lshl_add_u32.
constexpr uint32_t SILU_EDGE_KEY_MAX = (2u * SILU_EDGE) << 16;

__device__ __forceinline__ uint32_t silu_edge_key(float s)
{
    return (__float_as_uint(s) << 16) + ((SILU_EDGE - 0x8000u) << 16);
}

// The binary32 neighbour of f in direction dir (+1 up, -1 down); f != 0.
__device__ __forceinline__ float step_f32(float f, int dir)
{
    uint32_t b = __float_as_uint(f);
    bool up_in_magnitude = (dir > 0) == !(b >> 31);
    return __uint_as_float(up_in_magnitude ? b + 1u : b - 1u);
}

// Correctly rounded bf16(silu(g)), returned as a binary32 value whose
// round-to-nearest-even to bf16 is that result.
//  - |g| < 2^-24: silu(g) = g/2 + g^2/4 - ...; the binary64 value is g/2 and
//    the positive g^2/4 decides a tie (odd subnormal results).
//  - otherwise silu is evaluated in binary64 (error a few units of 2^-53).
// The binary64 value x goes to binary32 first; that rounding can only change
// the bf16 result when it lands exactly on a bf16 midpoint, and then the
// value is stepped one binary32 unit back toward x.
__device__ __attribute__((noinline)) float silu_exact(float g)
{
    if (g != g) return g;
    if (g == -__builtin_inff()) return -0.0f;
    double x;
    int dir_if_exact;
    if (__builtin_fabsf(g) < 0x1p-24f) {
        x = 0.5 * (double)g;
        dir_if_exact = +1;
    } else {
        double gd = (double)g;
        x = gd / (1.0 + exp(-gd));
        dir_if_exact = 0;
    }
    float f = (float)x;
    if ((__float_as_uint(f) & 0xFFFFu) == 0x8000u) {
        double back = (double)f;
        if (x > back) f = step_f32(f, +1);
        else if (x < back) f = step_f32(f, -1);
        else if (dir_if_exact != 0) f = step_f32(f, dir_if_exact);
    }
    return f;
}

}  // namespace aarms
