/*
 * aarms_oracle.c -- plain CPU oracle for fused residual-add + RMSNorm, SwiGLU
 * and their FP8 (E4M3) and block-scaled FP4 (MXFP4, NVFP4) epilogues.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * bench's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or constant with the HIP library, and the HIP library never
 * loads it.
 *
 * What it follows (cited by page title and section):
 *  - RMSNorm as eight operations -- cast to float, square, mean, add epsilon,
 *    reciprocal square root, multiply, cast back, multiply by the weight --
 *    and TensorRT-LLM's RMSNorm that adds the residual and normalizes in one
 *    kernel: "TensorRT-LLM: Compiling Inference Engines Ahead of Time",
 *    section "Fusing operations, measured".  FasterTransformer's residual-add
 *    glue kernel is the same add ("FasterTransformer" post, section
 *    "Weights, LayerNorm, and the Plumbing Nobody Photographs").
 *  - SwiGLU: silu(gate) * up over a gate_up projection output whose first
 *    half of each row is gate and second half is up; the activation is
 *    rounded to the storage type before the product (first page, same
 *    section, the swiglu kernel and its rounding comment).
 *  - FP8 quantisation of the SiLU-and-mul output (vLLM's activation fusion
 *    pass) and of the RMSNorm output ("Introduction to torch.compile and How
 *    It Works with vLLM", sections 3 and 4), in E4M3 ("TensorRT-LLM"
 *    walkthrough, Part V, the quantization deep dive; the FP8 formats paper,
 *    Part XI item 6).  E4M3 here is the OCP E4M3FN encoding: bias 7, three
 *    mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448.
 *
 * Arithmetic rules.  Steps the definition performs in float are IEEE binary32
 * with round-to-nearest-even; the file is built with -ffp-contract=off (no
 * fused multiply-add) and without fast-math or denormal flushing.  Where the
 * pages leave the order of operations open:
 *  - the mean of squares is summed in binary64 and rounded once to binary32;
 *  - the reciprocal square root is taken in binary64 and rounded once;
 *  - SiLU is evaluated in binary64 and rounded once, directly, to bf16.
 * Conversions to bf16 and E4M3 are written out below from the formats'
 * definitions (round to nearest, ties to even, subnormals kept).
 *
 * Conventions the pages do not fix (the configured workloads never hit them):
 *  - NaN converts to NaN; bf16 overflow gives infinity; E4M3 inputs are
 *    clamped to [-448, 448] before rounding, so infinities saturate;
 *  - silu(+inf) = +inf, silu(-inf) = -0;
 *  - the row amax ignores NaN;
 *  - a quantisation scale of zero is treated as one (an all-zero row's
 *    dynamic scale is 0 and its codes are signed zeros);
 *  - MXFP4: a block holding a NaN or an infinity gets the E8M0 NaN scale
 *    0xFF and zero codes; an all-zero block gets the smallest scale, 2^-127.
 *
 * MXFP4 follows the OCP Microscaling formats the "TensorRT-LLM" walkthrough
 * names (Part V: 32-value blocks sharing a power-of-two E8M0 scale, E2M1
 * elements): the shared exponent is floor(log2(max |v|)) minus 2 (the
 * exponent of E2M1's largest power of two), clamped to E8M0's range; each
 * element is v / 2^exponent rounded to nearest even on the E2M1 grid and
 * saturated at +-6.  Two elements per byte, the first in the low nibble.
 *
 * NVFP4 (same walkthrough: E2M1 elements in 16-value blocks sharing an E4M3
 * scale, one FP32 scale per tensor on top) with the tensor scale g given:
 * the block scale is E4M3(binary32(amax / binary32(6 g))), rounded to
 * nearest even and saturated at 448, so the block's largest value lands at
 * E2M1's largest, 6; each element is E2M1(binary32(v / S)) with
 * S = binary32(scale * g), and a signed zero when S is zero.  g = 0 is
 * treated as 1; a block holding a NaN or an infinity gets the E4M3 NaN
 * 0x7F and zero codes.
 */

#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BF16_MAX 0x1.FEp127
#define E4M3_MAX 448.0

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the top half of a binary32 word: widening is exact. */
float aarms_oracle_bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* Round a binary64 value to the grid of a binary format with p significand
 * bits (leading bit included) whose smallest normal exponent is emin.  Below
 * 2^emin the spacing stays 2^(emin-p+1) (gradual underflow).  Round to
 * nearest; an exact tie goes up when dir > 0, down when dir < 0 and to the
 * even neighbour when dir == 0.  dir is the sign of a remainder too small to
 * be held in v (see the SiLU below); ordinary rounding passes 0.  The caller
 * handles overflow. */
static double round_to_grid(double v, int p, int emin, int dir)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    (void)frexp(v, &e);              /* |v| in [2^(e-1), 2^e) */
    int lead = e - 1;
    if (lead < emin) lead = emin;
    double q = ldexp(1.0, lead - (p - 1));
    double n = v / q;                /* exact: q is a power of two */
    double fl = floor(n);
    double frac = n - fl;            /* exact */
    double k;
    if (frac > 0.5) k = fl + 1.0;
    else if (frac < 0.5) k = fl;
    else if (dir > 0) k = fl + 1.0;
    else if (dir < 0) k = fl;
    else k = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    if (k == 0.0) return copysign(0.0, v);
    return k * q;
}

static uint16_t bf16_round(double v, int dir)
{
    if (isnan(v)) return signbit(v) ? 0xFFC0u : 0x7FC0u;
    double r = round_to_grid(v, 8, -126, dir);
    if (fabs(r) > BF16_MAX) r = copysign(INFINITY, v);
    /* r lies on the bf16 grid, which is a subset of the binary32 grid */
    return (uint16_t)(bits_from_f32((float)r) >> 16);
}

/* binary64 -> bf16 (8 significand bits, emin -126), ties to even. */
uint16_t aarms_oracle_bf16_from_f64(double v) { return bf16_round(v, 0); }

/* binary64 -> OCP E4M3FN (4 significand bits, emin -6), ties to even.
 * A value that rounds beyond 448 has no encoding and gives NaN. */
uint8_t aarms_oracle_e4m3_from_f64(double v)
{
    uint8_t s = signbit(v) ? 0x80u : 0x00u;
    if (isnan(v)) return (uint8_t)(s | 0x7Fu);
    double r = fabs(round_to_grid(v, 4, -6, 0));
    if (r > E4M3_MAX) return (uint8_t)(s | 0x7Fu);
    if (r == 0.0) return s;
    int e;
    (void)frexp(r, &e);
    int lead = e - 1;
    if (lead < -6)                               /* subnormal: m * 2^-9 */
        return (uint8_t)(s | (uint8_t)(r * 512.0));
    int E = lead + 7;                            /* biased exponent 1..15 */
    int M = (int)((ldexp(r, -lead) - 1.0) * 8.0);
    return (uint8_t)(s | (E << 3) | M);
}

double aarms_oracle_e4m3_to_f64(uint8_t q)
{
    double sgn = (q & 0x80u) ? -1.0 : 1.0;
    int E = (q >> 3) & 0xF, M = q & 7;
    if (E == 15 && M == 7) return NAN;
    if (E == 0) return sgn * ldexp((double)M, -9);
    return sgn * ldexp(1.0 + M / 8.0, E - 7);
}

/* binary64 -> E2M1 (2 significand bits, emin 0, largest finite 6), ties to
 * even, saturating at +-6.  Code: sign in bit 3, then the magnitudes 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6 as 0..7.  NaN gives 0 (its block is marked by the
 * scale instead). */
uint8_t aarms_oracle_e2m1_from_f64(double v)
{
    if (isnan(v)) return 0;
    uint8_t s = signbit(v) ? 0x8u : 0x0u;
    double r = fabs(round_to_grid(v, 2, 0, 0));
    if (r > 6.0) r = 6.0;
    if (r == 0.0) return s;
    if (r < 1.0) return (uint8_t)(s | 1u);          /* 0.5, the only subnormal */
    int e;
    (void)frexp(r, &e);
    int lead = e - 1;                                /* 0, 1 or 2 */
    int E = lead + 1;                                /* biased exponent 1..3 */
    int M = (int)((ldexp(r, -lead) - 1.0) * 2.0);
    return (uint8_t)(s | (E << 1) | M);
}

double aarms_oracle_e2m1_to_f64(uint8_t q)
{
    double sgn = (q & 0x8u) ? -1.0 : 1.0;
    int E = (q >> 1) & 3, M = q & 1;
    if (E == 0) return sgn * 0.5 * M;
    return sgn * ldexp(1.0 + M / 2.0, E - 1);
}

/* E8M0 byte -> its value 2^(b - 127); 0xFF is NaN. */
double aarms_oracle_e8m0_to_f64(uint8_t b)
{
    return b == 0xFFu ? NAN : ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------------------ */
/* residual add + RMSNorm                                              */
/* ------------------------------------------------------------------ */

/* Residual add: r = bf16(f32(x) + f32(residual)), one binary32 add. */
void aarms_oracle_residual_add(const uint16_t *x, const uint16_t *res, int64_t n, uint16_t *r_out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float s = aarms_oracle_bf16_to_f32(x[i]) + aarms_oracle_bf16_to_f32(res[i]);
        r_out[i] = aarms_oracle_bf16_from_f64((double)s);
    }
}

/* Per-row scale of the norm: cast to float, square, mean, add epsilon,
 * reciprocal square root.  rs[row] is the binary32 value the normalization
 * multiplies by; rs_exact[row] (optional) is the same quantity kept in
 * binary64 without the binary32 roundings, the centre of the window of
 * correct results when the summation order is left open. */
void aarms_oracle_rms_scale(const uint16_t *r, int64_t T, int64_t H, float eps,
                            float *rs, double *rs_exact)
{
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row) {
        const uint16_t *rr = r + row * H;
        double acc = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double h = (double)aarms_oracle_bf16_to_f32(rr[j]);
            acc += h * h;
        }
        float m = (float)(acc / (double)H);          /* mean, rounded to float */
        float v = m + eps;                           /* add epsilon in float   */
        rs[row] = (float)(1.0 / sqrt((double)v));    /* rsqrt, rounded once    */
        if (rs_exact) rs_exact[row] = 1.0 / sqrt(acc / (double)H + (double)eps);
    }
}

/* Normalize and weight with a given per-row multiplier rho:
 * t = bf16(f32(h * rho)) (the multiply and the cast back to the tensor type),
 * y = bf16(f32(w) * f32(t)) (the weight multiply; the product of two bf16 is
 * exact in binary32). */
void aarms_oracle_rmsnorm_apply(const uint16_t *r, const uint16_t *w, const float *rho,
                                int64_t T, int64_t H, uint16_t *y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row) {
        for (int64_t j = 0; j < H; ++j) {
            float h = aarms_oracle_bf16_to_f32(r[row * H + j]);
            float p = h * rho[row];
            uint16_t t = aarms_oracle_bf16_from_f64((double)p);
            float tw = aarms_oracle_bf16_to_f32(w[j]) * aarms_oracle_bf16_to_f32(t);
            y[row * H + j] = aarms_oracle_bf16_from_f64((double)tw);
        }
    }
}

/* The window of per-row multipliers a correct fused kernel may use: binary32
 * values within relative distance delta of the exact 1/sqrt(mean + eps).
 * rho_lo is rounded down and rho_hi up, so the window is never narrower. */
void aarms_oracle_rms_window(const double *rs_exact, int64_t T, double delta,
                             float *rho_lo, float *rho_hi)
{
    for (int64_t row = 0; row < T; ++row) {
        double lo = rs_exact[row] * (1.0 - delta), hi = rs_exact[row] * (1.0 + delta);
        float flo = (float)lo, fhi = (float)hi;
        if ((double)flo > lo) flo = nextafterf(flo, -INFINITY);
        if ((double)fhi < hi) fhi = nextafterf(fhi, INFINITY);
        rho_lo[row] = flo;
        rho_hi[row] = fhi;
    }
}

/* fused_add_rmsnorm: residual_out = x + residual; out = RMSNorm(residual_out) * w. */
void aarms_oracle_fused_add_rmsnorm(const uint16_t *x, const uint16_t *res, const uint16_t *w,
                                    int64_t T, int64_t H, float eps,
                                    uint16_t *out, uint16_t *res_out, float *rs)
{
    aarms_oracle_residual_add(x, res, T * H, res_out);
    aarms_oracle_rms_scale(res_out, T, H, eps, rs, 0);
    aarms_oracle_rmsnorm_apply(res_out, w, rs, T, H, out);
}

/* rmsnorm without the residual add (the form of the first page's own Metal
 * norm, same section): out = RMSNorm(x) * w on x as given. */
void aarms_oracle_rmsnorm(const uint16_t *x, const uint16_t *w, int64_t T, int64_t H, float eps,
                          uint16_t *out, float *rs)
{
    aarms_oracle_rms_scale(x, T, H, eps, rs, 0);
    aarms_oracle_rmsnorm_apply(x, w, rs, T, H, out);
}

/* ------------------------------------------------------------------ */
/* FP8 quantisation                                                    */
/* ------------------------------------------------------------------ */

/* q = e4m3(clamp(f32(y) / scale, -448, 448)): divide, saturate, round. */
static uint8_t quant_e4m3(float y, float scale)
{
    float z = (scale == 0.0f) ? y : y / scale;      /* binary32 division */
    if (z > 448.0f) z = 448.0f;
    if (z < -448.0f) z = -448.0f;
    return aarms_oracle_e4m3_from_f64((double)z);
}

/* Per-tensor (static) scale: one scale for all n values. */
void aarms_oracle_quant_fp8_static(const uint16_t *y, int64_t n, float scale, uint8_t *q)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        q[i] = quant_e4m3(aarms_oracle_bf16_to_f32(y[i]), scale);
}

/* Per-token (dynamic) scale: s[row] = f32(max_j |y_j| / 448), then each
 * element is divided by its row's scale. */
void aarms_oracle_quant_fp8_per_row(const uint16_t *y, int64_t T, int64_t H,
                                    uint8_t *q, float *s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row) {
        float a = 0.0f;
        for (int64_t j = 0; j < H; ++j)
            a = fmaxf(a, fabsf(aarms_oracle_bf16_to_f32(y[row * H + j])));
        float sc = a / 448.0f;
        s[row] = sc;
        for (int64_t j = 0; j < H; ++j)
            q[row * H + j] = quant_e4m3(aarms_oracle_bf16_to_f32(y[row * H + j]), sc);
    }
}

/* Per-group (dynamic, block) scales: each row in groups of G consecutive
 * values; s[row, g] = f32(max |y| over the group / 448), and each element is
 * divided by its group's scale -- the per-token rule above, applied to each
 * group ("TensorRT-LLM" walkthrough, Part V: FP8 scales per tensor or per
 * block).  H is a multiple of G; s is [T, H / G]. */
void aarms_oracle_quant_fp8_per_group(const uint16_t *y, int64_t T, int64_t H, int64_t G,
                                      uint8_t *q, float *s)
{
    const int64_t groups = H / G;
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row) {
        for (int64_t g = 0; g < groups; ++g) {
            const int64_t first = row * H + g * G;
            float a = 0.0f;
            for (int64_t j = 0; j < G; ++j)
                a = fmaxf(a, fabsf(aarms_oracle_bf16_to_f32(y[first + j])));
            const float sc = a / 448.0f;
            s[row * groups + g] = sc;
            for (int64_t j = 0; j < G; ++j)
                q[first + j] = quant_e4m3(aarms_oracle_bf16_to_f32(y[first + j]), sc);
        }
    }
}

/* fused_add_rmsnorm_quant_fp8: the norm as above, its bf16 output quantised
 * per token. */
void aarms_oracle_fused_add_rmsnorm_quant_fp8(const uint16_t *x, const uint16_t *res,
                                              const uint16_t *w, int64_t T, int64_t H, float eps,
                                              uint16_t *y_scratch, uint8_t *q, float *s,
                                              uint16_t *res_out, float *rs)
{
    aarms_oracle_fused_add_rmsnorm(x, res, w, T, H, eps, y_scratch, res_out, rs);
    aarms_oracle_quant_fp8_per_row(y_scratch, T, H, q, s);
}

/* MXFP4: each row of H values (H a multiple of 32) in blocks of 32, one E8M0
 * scale byte per block, two E2M1 codes per byte (first in the low nibble). */
void aarms_oracle_quant_mxfp4(const uint16_t *y, int64_t T, int64_t H, uint8_t *q, uint8_t *s)
{
    const int64_t nb = H / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t *yb = y + row * H + b * 32;
            double amax = 0.0;
            int bad = 0;
            for (int i = 0; i < 32; ++i) {
                double v = (double)aarms_oracle_bf16_to_f32(yb[i]);
                if (!isfinite(v)) bad = 1;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            uint8_t *qb = q + row * (H / 2) + b * 16;
            if (bad) {
                s[row * nb + b] = 0xFFu;
                for (int i = 0; i < 16; ++i) qb[i] = 0;
                continue;
            }
            int x = -127;                              /* all-zero block */
            if (amax > 0.0) {
                int e;
                (void)frexp(amax, &e);                 /* amax in [2^(e-1), 2^e) */
                x = (e - 1) - 2;
                if (x < -127) x = -127;
                if (x > 127) x = 127;
            }
            s[row * nb + b] = (uint8_t)(x + 127);
            for (int i = 0; i < 16; ++i) {
                double v0 = ldexp((double)aarms_oracle_bf16_to_f32(yb[2 * i]), -x);
                double v1 = ldexp((double)aarms_oracle_bf16_to_f32(yb[2 * i + 1]), -x);
                qb[i] = (uint8_t)(aarms_oracle_e2m1_from_f64(v0) | (aarms_oracle_e2m1_from_f64(v1) << 4));
            }
        }
    }
}

/* NVFP4: each row of H values (H a multiple of 16) in blocks of 16, one E4M3
 * scale byte per block, two E2M1 codes per byte (first in the low nibble),
 * under the tensor scale g. */
void aarms_oracle_quant_nvfp4(const uint16_t *y, int64_t T, int64_t H, float g, uint8_t *q, uint8_t *s)
{
    const int64_t nb = H / 16;
    const float gg = (g == 0.0f) ? 1.0f : g;
    const float six_g = 6.0f * gg;                     /* binary32 product */
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t *yb = y + row * H + b * 16;
            float amax = 0.0f;
            int bad = 0;
            for (int i = 0; i < 16; ++i) {
                float v = aarms_oracle_bf16_to_f32(yb[i]);
                if (!isfinite(v)) bad = 1;
                else if (fabsf(v) > amax) amax = fabsf(v);
            }
            uint8_t *qb = q + row * (H / 2) + b * 8;
            if (bad) {
                s[row * nb + b] = 0x7Fu;
                for (int i = 0; i < 8; ++i) qb[i] = 0;
                continue;
            }
            float t = amax / six_g;                      /* binary32 quotient */
            if (t > 448.0f) t = 448.0f;
            const uint8_t sb = aarms_oracle_e4m3_from_f64((double)t);
            s[row * nb + b] = sb;
            const float S = (float)aarms_oracle_e4m3_to_f64(sb) * gg;   /* binary32 product */
            for (int i = 0; i < 8; ++i) {
                uint8_t c[2];
                for (int h = 0; h < 2; ++h) {
                    const float v = aarms_oracle_bf16_to_f32(yb[2 * i + h]);
                    const float z = (S == 0.0f) ? v * 0.0f : v / S;         /* binary32 quotient */
                    c[h] = aarms_oracle_e2m1_from_f64((double)z);
                }
                qb[i] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* SwiGLU                                                              */
/* ------------------------------------------------------------------ */

/* a = bf16(silu(g)) with silu(g) = g / (1 + exp(-g)), rounded once.
 * For |g| >= 2^-24 silu is evaluated in binary64 (its error, a few units of
 * 2^-53, is far from deciding any bf16 rounding; the pin tests check this
 * against a 60-digit evaluation of every gate).  Below that binary64 cannot
 * hold the second term of silu(g) = g/2 + g^2/4 - g^4/96 + ...: the value is
 * g/2, and the positive g^2/4 only decides ties (subnormal results). */
uint16_t aarms_oracle_silu_bf16(uint16_t g_bits)
{
    double g = (double)aarms_oracle_bf16_to_f32(g_bits);
    if (isnan(g)) return 0x7FC0u;
    if (fabs(g) < 0x1p-24) return bf16_round(g / 2.0, +1);
    double s = (g == -INFINITY) ? -0.0 : g / (1.0 + exp(-g));
    return bf16_round(s, 0);
}

/* y = bf16(f32(a) * f32(u)) with a = bf16(silu(gate)); gate = gu[row, j],
 * up = gu[row, N + j].  The product of two bf16 is exact in binary32. */
static uint16_t swiglu_one(uint16_t g, uint16_t u)
{
    float p = aarms_oracle_bf16_to_f32(aarms_oracle_silu_bf16(g)) * aarms_oracle_bf16_to_f32(u);
    return aarms_oracle_bf16_from_f64((double)p);
}

void aarms_oracle_swiglu(const uint16_t *gu, int64_t T, int64_t N, uint16_t *y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row)
        for (int64_t j = 0; j < N; ++j)
            y[row * N + j] = swiglu_one(gu[row * 2 * N + j], gu[row * 2 * N + N + j]);
}

/* SwiGLU output (bf16) quantised with a per-tensor scale. */
void aarms_oracle_swiglu_quant_fp8(const uint16_t *gu, int64_t T, int64_t N, float scale, uint8_t *q)
{
    #pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < T; ++row)
        for (int64_t j = 0; j < N; ++j) {
            uint16_t y = swiglu_one(gu[row * 2 * N + j], gu[row * 2 * N + N + j]);
            q[row * N + j] = quant_e4m3(aarms_oracle_bf16_to_f32(y), scale);
        }
}

/* SwiGLU output (bf16) quantised with a per-token scale:
 * s[row] = f32(max_j |y_j| / 448), q = e4m3(clamp(y / s)). */
void aarms_oracle_swiglu_quant_fp8_per_row(const uint16_t *gu, int64_t T, int64_t N,
                                           uint16_t *y_scratch, uint8_t *q, float *s)
{
    aarms_oracle_swiglu(gu, T, N, y_scratch);
    aarms_oracle_quant_fp8_per_row(y_scratch, T, N, q, s);
}

/* Threads for the OpenMP loops above (0 or less: leave as is). */
void aarms_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int aarms_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
