/*
 * aarms.h -- C ABI of libaarms.so: fused residual-add + RMSNorm, SwiGLU, and
 * their FP8 (E4M3) and block-scaled FP4 (MXFP4, NVFP4) epilogues, as
 * hand-written HIP kernels for gfx950 (MI355X).
 *
 * Data formats
 *   bf16  : 16-bit bit pattern (the top half of an IEEE binary32), passed as
 *           uint16 storage.
 *   fp8   : one byte, OCP E4M3FN (exponent bias 7, 3 mantissa bits, no
 *           infinities, 0x7F/0xFF are NaN, largest finite 448).
 *   fp4   : E2M1 codes (sign, 2 exponent bits, 1 mantissa bit: 0, 0.5, 1,
 *           1.5, 2, 3, 4, 6), two per byte, the first value of each pair in
 *           the low nibble.
 *   e8m0  : one byte, a power of two 2^(b - 127); 0xFF is NaN (MXFP4 block
 *           scales, one per 32 values).
 *   NVFP4 block scales are fp8 E4M3 bytes, one per 16 values.
 *   All tensors are dense and row-major; a "row" is one token.
 *
 * Conventions common to every entry point
 *   - Every pointer is a device pointer.  The caller allocates, owns and frees
 *     all memory; the library never allocates, frees or synchronizes, and
 *     keeps no pointer after it returns.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs
 *     asynchronously; every entry point may be captured into a hipGraph.
 *   - num_tokens == 0 is a no-op that returns AARMS_OK without checking the
 *     pointers.
 *   - Arguments are validated before anything is enqueued; on any error code
 *     nothing has been launched.  No C++ exception crosses this interface.
 *   - Tensor pointers must be 16-byte aligned; fp32 scale pointers 4-byte
 *     aligned; block-scale byte arrays (E8M0, E4M3) may have any alignment.
 *   - Outputs may not overlap any other argument, except the in-place pairs
 *     each entry point names.  Inputs may overlap each other.
 *   - Results are deterministic: the same inputs give the same bits on every
 *     run (reductions use a fixed order).
 *
 * Arithmetic (identical across entry points; the oracle-parity tests pin it)
 *   - Residual add: r = bf16(f32(x) + f32(residual)), one binary32 add.
 *   - RMSNorm: h = f32(r); mean of h^2 accumulated in binary64 and rounded
 *     once to binary32; v = binary32(mean + eps); rs = binary32(1/sqrt(v))
 *     from binary64; t = bf16(f32(h * rs)); y = bf16(f32(w) * f32(t)).
 *   - SiLU: a = bf16(silu(gate)) correctly rounded (silu(g) = g/(1+e^-g));
 *     y = bf16(f32(a) * f32(up)).
 *   - FP8: q = e4m3(clamp(f32(y) / scale, -448, 448)), the quotient rounded
 *     once to binary32, then round-to-nearest-even to E4M3.  NaN stays NaN
 *     (0x7F or 0xFF: the sign of a NaN is not specified), infinities
 *     saturate.  A scale of exactly zero is treated as one.
 */
#ifndef AARMS_H
#define AARMS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; everything declared
 * here is exported. */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

/* Return codes. */
enum aarms_status {
    AARMS_OK = 0,
    AARMS_ERR_NULL_POINTER = 1,      /* a required pointer is NULL                 */
    AARMS_ERR_BAD_SHAPE = 2,         /* negative size, zero width, width % 8 != 0
                                        (% 32 for MXFP4, % 16 for NVFP4)          */
    AARMS_ERR_UNSUPPORTED_SHAPE = 3, /* width, rows or element count beyond the limits */
    AARMS_ERR_MISALIGNED = 4,        /* pointer alignment not met                  */
    AARMS_ERR_ALIAS = 5,             /* an output overlaps another argument        */
    AARMS_ERR_BAD_EPS = 6,           /* eps negative, NaN or infinite              */
    AARMS_ERR_HIP = 7,               /* the HIP runtime refused the launch         */
    AARMS_ERR_BAD_VARIANT = 8        /* *_ex: unknown variant, or too narrow for H */
};

/* Limits. */
#define AARMS_MAX_HIDDEN 65536            /* norms: row width kept in registers    */
#define AARMS_MAX_ELEMENTS (1LL << 40)    /* tokens x width, per tensor            */
#define AARMS_MAX_TOKENS 2147483647LL     /* rows per call (the launch grids)     */
#define AARMS_MAX_INTER (1LL << 33)       /* swiglu: output row width              */
#define AARMS_MAX_INTER_PER_TOKEN 65536   /* swiglu_quant_fp8_dynamic: row kept in
                                             registers until its amax is known    */

/*
 * fused_add_rmsnorm -- residual add followed by RMSNorm in one pass.
 *
 * TensorRT-LLM folds the residual add into its normalization kernel; the
 * norm itself is the eight operations of Hugging Face's RMSNorm (cast to
 * float, square, mean, add epsilon, reciprocal square root, multiply, cast
 * back, multiply by the weight): "TensorRT-LLM: Compiling Inference Engines
 * Ahead of Time", section "Fusing operations, measured".
 *
 *   out          [num_tokens, hidden] bf16   written: the normalized, weighted row
 *   residual_out [num_tokens, hidden] bf16   written: x + residual (the updated
 *                                            residual stream)
 *   x            [num_tokens, hidden] bf16   read
 *   residual     [num_tokens, hidden] bf16   read
 *   weight       [hidden]             bf16   read
 *   hidden       > 0, multiple of 8, <= AARMS_MAX_HIDDEN
 *   eps          >= 0 and finite, added to the binary32 mean
 * In place: out == x and/or residual_out == residual are allowed.
 */
int fused_add_rmsnorm(void *out, void *residual_out,
                      const void *x, const void *residual, const void *weight,
                      int64_t num_tokens, int64_t hidden, float eps,
                      hipStream_t stream);

/*
 * fused_add_rmsnorm_quant_fp8 -- fused_add_rmsnorm whose bf16 output is
 * quantised to E4M3 with a dynamic per-token scale, in the same pass.
 *
 * The fused RMSNorm + FP8 quant is one of vLLM's fusion passes, and the
 * format is FP8 E4M3 with per-tensor or finer scaling: "Introduction to
 * torch.compile and How It Works with vLLM", section 4; "TensorRT-LLM"
 * walkthrough, Part V (quantization deep dive).
 *
 *   out_fp8      [num_tokens, hidden] fp8    written: e4m3(clamp(y / s_row))
 *   scale_out    [num_tokens]         fp32   written: s_row = binary32(max_j |y_j| / 448)
 *                                            (0 for an all-zero row, whose codes are zeros)
 *   residual_out [num_tokens, hidden] bf16   written: x + residual
 *   x, residual, weight, hidden, eps         as for fused_add_rmsnorm
 * y is the bf16 value fused_add_rmsnorm would write to `out`; every non-zero
 * row has max |q| = 448.  In place: residual_out == residual is allowed.
 */
int fused_add_rmsnorm_quant_fp8(void *out_fp8, float *scale_out, void *residual_out,
                                const void *x, const void *residual, const void *weight,
                                int64_t num_tokens, int64_t hidden, float eps,
                                hipStream_t stream);

/*
 * fused_add_rmsnorm_quant_fp8_static -- fused_add_rmsnorm whose bf16 output
 * is quantised to E4M3 with a given per-tensor scale, in the same pass
 * (vLLM's RMSNorm + quant fusion with the per-tensor scaling of the
 * "TensorRT-LLM" walkthrough, Part V).
 *
 *   out_fp8      [num_tokens, hidden] fp8    written: e4m3(clamp(y / *scale, -448, 448))
 *   residual_out [num_tokens, hidden] bf16   written: x + residual
 *   scale        [1] fp32, device memory,    read by the kernel; positive and
 *                finite, except that exactly zero is treated as one
 *   x, residual, weight, hidden, eps         as for fused_add_rmsnorm
 * In place: residual_out == residual is allowed.
 */
int fused_add_rmsnorm_quant_fp8_static(void *out_fp8, void *residual_out,
                                       const void *x, const void *residual, const void *weight,
                                       const float *scale, int64_t num_tokens, int64_t hidden,
                                       float eps, hipStream_t stream);

/*
 * rmsnorm -- RMSNorm without the residual add: the form of the first page's
 * own Metal norm ("TensorRT-LLM: Compiling Inference Engines Ahead of Time",
 * section "Fusing operations, measured": the laptop fusions have no add).
 *
 *   out      [num_tokens, hidden] bf16   written: bf16(w * bf16(x * rs))
 *   x        [num_tokens, hidden] bf16   read
 *   weight, hidden, eps                  as for fused_add_rmsnorm
 * In place: out == x is allowed.
 */
int rmsnorm(void *out, const void *x, const void *weight, int64_t num_tokens, int64_t hidden,
            float eps, hipStream_t stream);

/*
 * rmsnorm_quant_fp8 / rmsnorm_quant_fp8_static -- rmsnorm with the dynamic
 * per-token or the static per-tensor E4M3 epilogue of the two
 * fused_add_rmsnorm_quant_fp8 forms above (same outputs, no residual).
 * No in-place form.
 */
int rmsnorm_quant_fp8(void *out_fp8, float *scale_out, const void *x, const void *weight,
                      int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream);
int rmsnorm_quant_fp8_static(void *out_fp8, const void *x, const void *weight, const float *scale,
                             int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream);

/*
 * fused_add_rmsnorm_quant_mxfp4 / rmsnorm_quant_mxfp4 -- the norm (with or
 * without the residual add) whose bf16 output is written as OCP MXFP4 in the
 * same pass: blocks of 32 values along a row share an E8M0 (power-of-two)
 * scale and each value is an E2M1 code ("TensorRT-LLM" walkthrough, Part V,
 * the OCP MXFP4 standard; vLLM's AllReduce + RMSNorm + Quant (FP4) fusion,
 * "Introduction to torch.compile and How It Works with vLLM", section 4).
 *
 *   out_fp4      [num_tokens, hidden / 2]  uint8  written: two E2M1 codes per byte,
 *                                                 the first value in the low nibble
 *   scale_out    [num_tokens, hidden / 32] uint8  written: E8M0 byte b (2^(b - 127)) per
 *                                                 block, b = clamp(floor(log2 max|y|) - 2 + 127,
 *                                                 0, 254); 0xFF for a block holding a
 *                                                 NaN or an infinity (its codes are 0)
 *   residual_out, x, residual, weight, eps   as for fused_add_rmsnorm / rmsnorm
 *   hidden       multiple of 32, <= AARMS_MAX_HIDDEN
 * A code is E2M1(y / 2^(b - 127)) rounded to nearest even, saturated at +-6.
 * In place: residual_out == residual is allowed.  scale_out has no
 * alignment requirement.
 */
int fused_add_rmsnorm_quant_mxfp4(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                  const void *x, const void *residual, const void *weight,
                                  int64_t num_tokens, int64_t hidden, float eps,
                                  hipStream_t stream);
int rmsnorm_quant_mxfp4(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                        int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream);

/*
 * fused_add_rmsnorm_quant_nvfp4 / rmsnorm_quant_nvfp4 -- the norm (with or
 * without the residual add) whose bf16 output is written as NVFP4 in the
 * same pass: E2M1 codes in blocks of 16 along a row sharing an E4M3 scale,
 * under a given FP32 tensor scale ("TensorRT-LLM" walkthrough, Part V; vLLM
 * post, section 4).  The pages give the format, not the scale recipe; this
 * library's:
 *   block scale  E4M3(binary32(max|y| / binary32(6 g))), nearest even,
 *                saturated at 448 (the block's largest value maps to 6)
 *   code         E2M1(binary32(y / S)), S = binary32(block scale * g),
 *                nearest even, saturated at +-6; a signed zero when S = 0
 *
 *   out_fp4      [num_tokens, hidden / 2]  uint8  written: two E2M1 codes per byte,
 *                                                 the first value in the low nibble
 *   scale_out    [num_tokens, hidden / 16] uint8  written: E4M3 block scales; 0x7F
 *                                                 for a block holding a NaN or an
 *                                                 infinity (its codes are 0)
 *   tensor_scale [1] fp32, device memory  read: g, positive and finite; 0 means 1
 *   residual_out, x, residual, weight, eps   as for fused_add_rmsnorm / rmsnorm
 *   hidden       multiple of 16, <= AARMS_MAX_HIDDEN
 * In place: residual_out == residual is allowed.
 */
int fused_add_rmsnorm_quant_nvfp4(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                  const void *x, const void *residual, const void *weight,
                                  const float *tensor_scale, int64_t num_tokens, int64_t hidden,
                                  float eps, hipStream_t stream);
int rmsnorm_quant_nvfp4(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                        const float *tensor_scale, int64_t num_tokens, int64_t hidden, float eps,
                        hipStream_t stream);

/*
 * swiglu -- silu(gate) * up over a concatenated gate_up projection output.
 *
 * TensorRT-LLM's gated MLP runs one gate_up_proj matmul followed by a fused
 * swiglu; the activation reads the two halves of each row, gate first, and
 * rounds the SiLU to the storage type before the product: first page,
 * section "Fusing operations, measured" (the swiglu kernel).
 *
 *   out      [num_tokens, inter]     bf16   written
 *   gate_up  [num_tokens, 2 * inter] bf16   read; gate = columns [0, inter),
 *                                           up = columns [inter, 2*inter)
 *   inter    > 0, multiple of 8, at most AARMS_MAX_INTER
 * No in-place form: out may not overlap gate_up.
 */
int swiglu(void *out, const void *gate_up, int64_t num_tokens, int64_t inter,
           hipStream_t stream);

/*
 * swiglu_quant_fp8 -- swiglu whose bf16 output is quantised to E4M3 with a
 * given per-tensor scale, in the same pass (vLLM's SiLU-and-mul + quant
 * fusion: "Introduction to torch.compile and How It Works with vLLM",
 * sections 3 and 4).
 *
 *   out_fp8  [num_tokens, inter]     fp8    written: e4m3(clamp(y / *scale))
 *   gate_up  [num_tokens, 2 * inter] bf16   read, as for swiglu
 *   scale    [1] fp32, device memory,       read by the kernel (so it may be
 *            changed between graph replays); must be positive and finite,
 *            except that exactly zero is treated as one
 *   inter    > 0, multiple of 8, at most AARMS_MAX_INTER
 */
int swiglu_quant_fp8(void *out_fp8, const void *gate_up, const float *scale,
                     int64_t num_tokens, int64_t inter, hipStream_t stream);

/*
 * swiglu_quant_mxfp4 -- swiglu whose bf16 output is written as OCP MXFP4 in
 * the same pass, with the block rules of the MXFP4 norms above (blocks of 32
 * along a row).
 *
 *   out_fp4   [num_tokens, inter / 2]  uint8  written: two E2M1 codes per byte
 *   scale_out [num_tokens, inter / 32] uint8  written: E8M0 block scales
 *   gate_up   [num_tokens, 2 * inter]  bf16   read, as for swiglu
 *   inter     multiple of 32, at most AARMS_MAX_INTER
 * No in-place form.
 */
int swiglu_quant_mxfp4(void *out_fp4, uint8_t *scale_out, const void *gate_up,
                       int64_t num_tokens, int64_t inter, hipStream_t stream);

/*
 * swiglu_quant_nvfp4 -- swiglu whose bf16 output is written as NVFP4 in the
 * same pass, with the block rules of the NVFP4 norms above.
 *
 *   out_fp4      [num_tokens, inter / 2]  uint8
 *   scale_out    [num_tokens, inter / 16] uint8  E4M3 block scales
 *   gate_up      [num_tokens, 2 * inter]  bf16   read, as for swiglu
 *   tensor_scale [1] fp32, device memory
 *   inter        multiple of 16, at most AARMS_MAX_INTER
 * No in-place form.
 */
int swiglu_quant_nvfp4(void *out_fp4, uint8_t *scale_out, const void *gate_up,
                       const float *tensor_scale, int64_t num_tokens, int64_t inter,
                       hipStream_t stream);

/*
 * swiglu_quant_fp8_dynamic -- swiglu whose bf16 output is quantised to E4M3
 * with a dynamic per-token scale, in the same pass (vLLM's SiLU-and-mul +
 * quant fusion, sections 3 and 4 of its post, with per-token scaling as in
 * the norm above).
 *
 *   out_fp8   [num_tokens, inter]     fp8    written: e4m3(clamp(y / s_row))
 *   scale_out [num_tokens]            fp32   written: s_row = binary32(max_j |y_j| / 448)
 *                                            (0 for an all-zero row, whose codes are zeros)
 *   gate_up   [num_tokens, 2 * inter] bf16   read, as for swiglu
 *   inter     > 0, multiple of 8, at most AARMS_MAX_INTER_PER_TOKEN
 * y is the bf16 value swiglu would write.  No in-place form.
 */
int swiglu_quant_fp8_dynamic(void *out_fp8, float *scale_out, const void *gate_up,
                             int64_t num_tokens, int64_t inter, hipStream_t stream);

/* Human-readable name of a return code (static storage, never NULL). */
const char *aarms_status_string(int status);

/*
 * fused_add_rmsnorm_quant_fp8_group, rmsnorm_quant_fp8_group,
 * swiglu_quant_fp8_group -- the norm (with or without the residual add) or
 * swiglu, then E4M3 codes under one fp32 scale per group of
 * AARMS_FP8_GROUP (128) consecutive values of a row: the per-block FP8
 * scaling of the "TensorRT-LLM" walkthrough, Part V, with the per-token rule
 * of fused_add_rmsnorm_quant_fp8 applied to each group.
 *
 *   out_fp8      [num_tokens, width]       fp8    written: e4m3(clamp(y / s_g))
 *   scale_out    [num_tokens, width / 128] fp32   written: s_g = binary32(max |y| over
 *                                                  the group / 448), NaN values
 *                                                  ignored (0 for an all-zero group,
 *                                                  whose codes are zeros); 4-byte aligned
 *   residual_out, x, residual, weight, hidden, eps   as for fused_add_rmsnorm
 *   gate_up, inter                                    as for swiglu
 * width (hidden or inter) must be a multiple of 128 (else
 * AARMS_ERR_BAD_SHAPE).  y is the bf16 value the bf16 form would write; every
 * non-zero group has max |q| = 448.  In place (norm with the residual):
 * residual_out == residual is allowed.
 */
#define AARMS_FP8_GROUP 128
int fused_add_rmsnorm_quant_fp8_group(void *out_fp8, float *scale_out, void *residual_out,
                                      const void *x, const void *residual, const void *weight,
                                      int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream);
int rmsnorm_quant_fp8_group(void *out_fp8, float *scale_out, const void *x, const void *weight,
                            int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream);
int swiglu_quant_fp8_group(void *out_fp8, float *scale_out, const void *gate_up, int64_t num_tokens,
                           int64_t inter, hipStream_t stream);

/*
 * Kernel variants, for tuning sweeps.  The plain entry points pick a variant
 * from (num_tokens, width, output format); the *_ex forms take it
 * explicitly.  A variant id is an index into the op's table;
 * aarms_variant_name() describes it (static storage) and returns NULL past
 * the end.  ops: 0 = the norms with the residual add (fused_add_rmsnorm*),
 * 3 = the norms without it (rmsnorm*), both on one variant table (quant = the
 * output format: 0 bf16, 1 E4M3 per token, 2 E4M3 per tensor (the _static
 * forms), 3 MXFP4, 4 NVFP4, 5 E4M3 per 128-value group); 1 = swiglu,
 * swiglu_quant_fp8, swiglu_quant_mxfp4, swiglu_quant_nvfp4 and
 * swiglu_quant_fp8_group (quant = the output format: 0 bf16, 1 E4M3, 2 MXFP4,
 * 3 NVFP4, 4 E4M3 per 128-value group); 2 = swiglu_quant_fp8_dynamic.  -1
 * is returned for a format code outside these.
 * aarms_pick_variant() returns the id the plain entry point would use, or -1
 * for an unsupported shape.  Variant -1 in an *_ex call means "pick".
 * aarms_variant_fits() returns 1 if the variant runs rows of `width` values
 * (hidden for the norms, inter for the SwiGLU ops), 0 if an *_ex call with it
 * would return AARMS_ERR_BAD_VARIANT for that width (too narrow, or, for the
 * norm variants named "resident", a width that is not a multiple of 512).
 */
int aarms_variant_count(int op);
const char *aarms_variant_name(int op, int variant);
int aarms_pick_variant(int op, int64_t num_tokens, int64_t width, int quant);
int aarms_variant_fits(int op, int variant, int64_t width);

int fused_add_rmsnorm_ex(void *out, void *residual_out,
                         const void *x, const void *residual, const void *weight,
                         int64_t num_tokens, int64_t hidden, float eps,
                         int variant, hipStream_t stream);
int fused_add_rmsnorm_quant_fp8_ex(void *out_fp8, float *scale_out, void *residual_out,
                                   const void *x, const void *residual, const void *weight,
                                   int64_t num_tokens, int64_t hidden, float eps,
                                   int variant, hipStream_t stream);
int swiglu_ex(void *out, const void *gate_up, int64_t num_tokens, int64_t inter,
              int variant, hipStream_t stream);
int swiglu_quant_fp8_ex(void *out_fp8, const void *gate_up, const float *scale,
                        int64_t num_tokens, int64_t inter, int variant, hipStream_t stream);
int fused_add_rmsnorm_quant_fp8_static_ex(void *out_fp8, void *residual_out,
                                          const void *x, const void *residual, const void *weight,
                                          const float *scale, int64_t num_tokens, int64_t hidden,
                                          float eps, int variant, hipStream_t stream);
int rmsnorm_ex(void *out, const void *x, const void *weight, int64_t num_tokens, int64_t hidden,
               float eps, int variant, hipStream_t stream);
int rmsnorm_quant_fp8_ex(void *out_fp8, float *scale_out, const void *x, const void *weight,
                         int64_t num_tokens, int64_t hidden, float eps, int variant,
                         hipStream_t stream);
int rmsnorm_quant_fp8_static_ex(void *out_fp8, const void *x, const void *weight,
                                const float *scale, int64_t num_tokens, int64_t hidden, float eps,
                                int variant, hipStream_t stream);
int swiglu_quant_fp8_dynamic_ex(void *out_fp8, float *scale_out, const void *gate_up,
                                int64_t num_tokens, int64_t inter, int variant, hipStream_t stream);
int fused_add_rmsnorm_quant_fp8_group_ex(void *out_fp8, float *scale_out, void *residual_out,
                                         const void *x, const void *residual, const void *weight,
                                         int64_t num_tokens, int64_t hidden, float eps, int variant,
                                         hipStream_t stream);
int rmsnorm_quant_fp8_group_ex(void *out_fp8, float *scale_out, const void *x, const void *weight,
                               int64_t num_tokens, int64_t hidden, float eps, int variant,
                               hipStream_t stream);
int swiglu_quant_fp8_group_ex(void *out_fp8, float *scale_out, const void *gate_up, int64_t num_tokens,
                              int64_t inter, int variant, hipStream_t stream);
int swiglu_quant_mxfp4_ex(void *out_fp4, uint8_t *scale_out, const void *gate_up,
                          int64_t num_tokens, int64_t inter, int variant, hipStream_t stream);
int swiglu_quant_nvfp4_ex(void *out_fp4, uint8_t *scale_out, const void *gate_up,
                          const float *tensor_scale, int64_t num_tokens, int64_t inter, int variant,
                          hipStream_t stream);
int fused_add_rmsnorm_quant_nvfp4_ex(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                     const void *x, const void *residual, const void *weight,
                                     const float *tensor_scale, int64_t num_tokens, int64_t hidden,
                                     float eps, int variant, hipStream_t stream);
int rmsnorm_quant_nvfp4_ex(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                           const float *tensor_scale, int64_t num_tokens, int64_t hidden, float eps,
                           int variant, hipStream_t stream);
int fused_add_rmsnorm_quant_mxfp4_ex(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                     const void *x, const void *residual, const void *weight,
                                     int64_t num_tokens, int64_t hidden, float eps, int variant,
                                     hipStream_t stream);
int rmsnorm_quant_mxfp4_ex(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                           int64_t num_tokens, int64_t hidden, float eps, int variant,
                           hipStream_t stream);

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* AARMS_H */
