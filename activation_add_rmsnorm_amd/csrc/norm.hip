// norm.hip -- RMSNorm for gfx950, with or without the residual add in front,
// and with a bf16 epilogue or a quantised one: E4M3 with a per-token, a
// per-tensor or a per-128-value scale, MXFP4 or NVFP4.
//
// One pass over HBM: x (and the residual) are read once with 16-byte
// streaming loads, the updated residual and the output are written once, and
// the row stays in registers between the reduction and the epilogue.  A row
// is handled by one wave (narrow rows, four rows per 256-thread block) or by
// a whole block of 2..16 waves (wide rows); a persistent, software-pipelined
// form walks several rows per block.  The sum of squares is accumulated per
// lane in binary64, reduced with a wave butterfly and, across waves, through
// LDS in a fixed order, so results are bitwise reproducible.  One-generation
// bf16 launches hold their stores until the launch's reads are served (see
// hold_stores).
//
// The arithmetic follows the eight-operation RMSNorm with the residual add
// in front ("TensorRT-LLM: Compiling Inference Engines Ahead of Time",
// section "Fusing operations, measured"; the same page's own Metal norm has
// no add); the FP8 epilogues follow vLLM's RMSNorm + quant fusion
// ("Introduction to torch.compile and How It Works with vLLM", section 4)
// with the per-token or per-tensor scaling of the TensorRT-LLM walkthrough's
// quantization deep dive (Part V).

#include "device.h"
#include "launch.h"

#include <atomic>

namespace aarms {

// q = e4m3(clamp(y / s)) for this lane's slices of the row (y as binary32
// values of bf16), stored as 8-byte groups.
template <int WPR, int VPT, bool FAST, bool CLAMP>
__device__ __forceinline__ void quantize_row(const float (&yf)[VPT][8], const E4m3Scale &qs,
                                             uint8_t *qo, int lane, int nvec)
{
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * WPR * 64;
        if (v >= nvec) continue;
        float z[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = e4m3_quotient<FAST, CLAMP>(yf[k][j], qs);
        u32x2 q;
        q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
        q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
        st_stream((u32x2 *)(qo + (size_t)v * 8), q);
    }
}

// x into xv and, with RES, the residual into rv.
template <int WPR, int VPT, bool RES>
__device__ __forceinline__ void load_row(const NormParams &p, int64_t row, int lane, int nvec,
                                         u32x4 (&xv)[VPT], u32x4 (&rv)[VPT])
{
    const size_t base = (size_t)row * (size_t)p.hidden;
    const u32x4 *xr = (const u32x4 *)((const uint16_t *)p.x + base);
    const u32x4 *rr = (const u32x4 *)((const uint16_t *)p.residual + base);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * WPR * 64;
        const bool ok = v < nvec;
        xv[k] = ok ? ld_stream(xr + v) : (u32x4)0u;
        if constexpr (RES) rv[k] = ok ? ld_stream(rr + v) : (u32x4)0u;
    }
}

// y = bf16(w * bf16(h * rs)) for the two bf16 of one word of the row.
__device__ __forceinline__ uint32_t norm_word(uint32_t r, uint32_t w, float rs)
{
    const uint32_t t = pack_bf16(bf_lo(r) * rs, bf_hi(r) * rs);
    return pack_bf16(bf_lo(w) * bf_lo(t), bf_hi(w) * bf_hi(t));
}

// The same, also handing back the binary32 products p0 = w t before their
// rounding.  Rounding to nearest is monotone and symmetric, so the largest
// |p| rounds to the largest |y|: amax reductions run on the products (one
// three-operand maximum per word) and round once at the end.
__device__ __forceinline__ uint32_t norm_word(uint32_t r, uint32_t w, float rs, float &p0, float &p1)
{
    const uint32_t t = pack_bf16(bf_lo(r) * rs, bf_hi(r) * rs);
    p0 = bf_lo(w) * bf_lo(t);
    p1 = bf_hi(w) * bf_hi(t);
    return pack_bf16(p0, p1);
}

// Static per-tensor E4M3 epilogue: q = e4m3(clamp(y / s)) straight from the
// row, 8 bytes per 16-byte slice.
// With late_ro, slice k of the updated residual is stored there once it has
// been read (the late residual stores of finish_row).
template <int WPR, int VPT, bool FAST>
__device__ __forceinline__ void store_static_fp8(const u32x4 (&rv)[VPT], const u32x4 (&wv)[VPT], float rs,
                                                 const E4m3Scale &qs, uint8_t *qo, int lane, int nvec,
                                                 u32x4 *late_ro)
{
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * WPR * 64;
        if (v >= nvec) continue;
        float z[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t y = norm_word(rv[k][e], wv[k][e], rs);
            z[2 * e] = e4m3_quotient<FAST, true>(bf_lo(y), qs);
            z[2 * e + 1] = e4m3_quotient<FAST, true>(bf_hi(y), qs);
        }
        if (late_ro) st_stream(late_ro + v, rv[k]);
        u32x2 q;
        q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
        q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
        st_stream((u32x2 *)(qo + (size_t)v * 8), q);
    }
}

template <int WPR, int VPT>
__device__ __forceinline__ void load_weight(const NormParams &p, int lane, int nvec, u32x4 (&wv)[VPT])
{
    const u32x4 *wr = (const u32x4 *)p.weight;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * WPR * 64;
        wv[k] = (v < nvec) ? wr[v] : (u32x4)0u;
    }
}

// Phase stamps (measurement build only, -DAARMS_PHASE_STAMPS): lane 0 of
// each wave records the real-time clock (100 MHz) when the wave reaches slot
// k, after dep has been computed, into stamps[(row * WPR + wave) * 16 + k]:
// 0 start, 1 row loads consumed, 2 wave sum, 3 first barrier passed, 4 row
// amax (per-token E4M3) or outputs computed, 5 wave maximum, 6 second
// barrier passed, 7 last store issued; 8 and 9 hold the HW_ID and XCC_ID
// registers (which CU ran the wave); with stamp_detail, per-token E4M3 with
// several waves per row also 10 row sum combined, 11 mean and 1/sqrt
// computed, 12 weight in registers, 13 row amax combined, 14 scale and its
// reciprocal computed.
#ifdef AARMS_PHASE_STAMPS
__device__ __forceinline__ uint64_t stamp_after(float dep)
{
    asm volatile("" : : "v"(dep));
    return __builtin_amdgcn_s_memrealtime();
}
#define AARMS_STAMP(k, dep)                                                                        \
    do {                                                                                           \
        if (p.stamps) {                                                                            \
            const uint64_t t_ = stamp_after(dep);                                                  \
            if ((lane & 63) == 0) p.stamps[((size_t)row * WPR + (size_t)(lane >> 6)) * 16 + (k)] = t_; \
        }                                                                                          \
    } while (0)
#define AARMS_STAMP_DETAIL(k, dep)                                                                 \
    do {                                                                                           \
        if (p.stamp_detail) AARMS_STAMP(k, dep);                                                   \
    } while (0)
#else
#define AARMS_STAMP(k, dep) do {} while (0)
#define AARMS_STAMP_DETAIL(k, dep) do {} while (0)
#endif

// Store hold.  In a launch whose blocks are all resident at once, every
// wave issues its loads at the start and would store its row as soon as the
// row is done, so the writes of the first rows finished compete in HBM with
// the reads still outstanding for the rest.  Holding each row's stores until
// a fixed time after its wave started (about the time the launch's reads
// take) serves the reads first and the writes after them, with fewer
// read/write turnarounds (measured 16-19% faster on one-wave-per-row bf16
// launches of 25-38 MB of reads).  The wait is bounded: it ends once the
// real-time clock (100 MHz, s_memrealtime) has advanced hold_ticks past
// t_start, or if the clock reads below t_start.  dep ties the wait to a
// value computed from the row, so it starts after the row's loads landed.
__device__ __forceinline__ void hold_stores(uint64_t t_start, uint32_t hold_ticks, double dep)
{
    if (hold_ticks == 0) return;
    asm volatile("" : : "v"(dep));
    while (true) {
        const uint64_t now = __builtin_amdgcn_s_memrealtime();
        if (now < t_start || now - t_start >= hold_ticks) break;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Everything after the row's loads: residual add and store (RES), sum of
// squares, the row reduction (through psum when the row spans several
// waves), the normalization and the epilogue.  With W_LATE the weight is
// loaded here, after the first pass, so that its registers are not live
// while the row loads are in flight.
// t_start: the wave's start on the real-time clock, for the store hold (the
// stores issued after the sum of squares: all of them in the bf16 form).
template <int WPR, int VPT, int EPI, bool RES, bool W_LATE>
__device__ __forceinline__ void finish_row(const NormParams &p, int64_t row, int lane, int nvec,
                                           const u32x4 (&xv)[VPT], u32x4 (&rv)[VPT],
                                           u32x4 (&wv)[VPT], double *psum, float *pmax,
                                           const float *nv_inv, uint64_t t_start = 0)
{
    constexpr bool QUANT = EPI == NORM_EPI_FP8_DYNAMIC;
    const size_t base = (size_t)row * (size_t)p.hidden;
    u32x4 *ro = (u32x4 *)((uint16_t *)p.residual_out + base);

    // ---- residual add (binary32, one rounding), store, sum of squares.
    // One counter tracks both loads and stores on gfx9, so a load waited on
    // after a store is issued (the weight) also waits for that store to
    // reach memory.  The bf16 form stores the updated residual last, with
    // the output (1-2% faster).  The quantised forms store each slice in the
    // epilogue, once it has been read for the last time, when the launch is
    // one generation of blocks (p.res_last: the writes then come after the
    // row reduction, so after most of the launch's reads; 4-19% faster from
    // 12 MB of reads); in longer launches they store it here, which spreads
    // their writes between the generations.
    const bool res_late = EPI != NORM_EPI_BF16 && RES && p.res_last != 0;
    u32x4 *const late_ro = res_late ? ro : nullptr;
    // With few vectors per lane the FP8 form keeps h = f32(r) for the
    // epilogue (fewer instructions); otherwise the packed words are kept
    // (fewer registers, so more rows in flight) and widened again.
    constexpr bool KEEP = QUANT && VPT <= 2;
    // four independent binary64 chains (one per word of a vector), summed in
    // a fixed order at the end: a quarter of the dependent-FMA latency
    double acc4[4] = {0.0, 0.0, 0.0, 0.0};
    float hf[QUANT ? VPT : 1][8];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * WPR * 64;
        u32x4 r;
        if constexpr (RES) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r[e] = pack_bf16(bf_lo(xv[k][e]) + bf_lo(rv[k][e]), bf_hi(xv[k][e]) + bf_hi(rv[k][e]));
            if (EPI != NORM_EPI_BF16 && !res_late && v < nvec) st_stream(ro + v, r);
        } else {
            r = xv[k];
        }
        rv[k] = r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float h0 = bf_lo(r[e]), h1 = bf_hi(r[e]);
            if constexpr (KEEP) {
                hf[k][2 * e] = h0;
                hf[k][2 * e + 1] = h1;
            }
            acc4[e] = __builtin_fma((double)h0, (double)h0, acc4[e]);
            acc4[e] = __builtin_fma((double)h1, (double)h1, acc4[e]);
        }
    }
    double acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    AARMS_STAMP(1, (float)acc);
    hold_stores(t_start, p.hold_ticks, acc);
    if constexpr (W_LATE) {
        // keep the scheduler from hoisting these loads back to the top
        __builtin_amdgcn_sched_barrier(0);
        load_weight<WPR, VPT>(p, lane, nvec, wv);
    }
    acc = wave_sum(acc);
    AARMS_STAMP(2, (float)acc);
    if constexpr (WPR > 1) {
        if ((lane & 63) == 0) psum[lane >> 6] = acc;
        __syncthreads();
        AARMS_STAMP(3, (float)acc);
        acc = block_sum<WPR>(psum, lane & 63);
        if constexpr (EPI == NORM_EPI_FP8_DYNAMIC) AARMS_STAMP_DETAIL(10, (float)acc);
    }

    // ---- mean (rounded once to binary32), + eps, reciprocal square root;
    // the branches are uniform over the row (acc and var are the row's)
    float mean;
    if (acc <= __DBL_MAX__)
        mean = row_mean(acc, (double)p.hidden, p.inv_hidden);
    else
        mean = (float)(acc / (double)p.hidden);
    const float var = mean + p.eps;
    float rs;
    if (row_rsqrt_in_range(var))
        rs = row_rsqrt(var);
    else
        rs = (float)(1.0 / sqrt((double)var));
    if constexpr (EPI == NORM_EPI_FP8_DYNAMIC && WPR > 1) {
        AARMS_STAMP_DETAIL(11, rs);
        AARMS_STAMP_DETAIL(12, __uint_as_float(wv[0][0]));
    }

    if constexpr (EPI == NORM_EPI_BF16) {
        // ---- t = bf16(h * rs), y = bf16(w * t)
        u32x4 *o = (u32x4 *)((uint16_t *)p.out + base);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lane + k * WPR * 64;
            if (v >= nvec) continue;
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = norm_word(rv[k][e], wv[k][e], rs);
            st_stream(o + v, y);
        }
    } else if constexpr (EPI == NORM_EPI_MXFP4) {
        // ---- y as above; per 32-value block (the 4 slices of 4 adjacent
        // lanes) the E8M0 scale from the block amax, then E2M1 codes
        uint32_t *qo = (uint32_t *)((uint8_t *)p.out + (size_t)row * (size_t)(p.hidden / 2));
        uint8_t *so = (uint8_t *)p.scale_out + (size_t)row * (size_t)(p.hidden / 32);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lane + k * WPR * 64;
            uint32_t y[4];
            // NaN-propagating maxima: a block holding a NaN gets the NaN scale
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float p0, p1;
                y[e] = norm_word(rv[k][e], wv[k][e], rs, p0, p1);
                amax = __builtin_elementwise_maximum(
                    amax, __builtin_elementwise_maximum(__builtin_fabsf(p0), __builtin_fabsf(p1)));
            }
            if (late_ro && v < nvec) st_stream(late_ro + v, rv[k]);
            uint32_t mag = __float_as_uint(round_bf16(amax));
            // the block's 4 slices sit in lanes 4j..4j+3 (all inside or all
            // past the row end, as H is a multiple of 32)
            mag = max(mag, dpp_u32<DPP_XOR1>(mag));
            mag = max(mag, dpp_u32<DPP_XOR2>(mag));
            if (v >= nvec) continue;
            const uint32_t sb = mx_scale_byte(mag);
            const float inv = __uint_as_float((254u - (sb == 0xFFu ? 127u : sb)) << 23);
            const uint32_t q = (sb == 0xFFu) ? 0u : pack_e2m1x8(y, inv);
            st_stream(qo + v, q);
            if ((lane & 3) == 0) so[v >> 2] = (uint8_t)sb;
        }
    } else if constexpr (EPI == NORM_EPI_NVFP4) {
        // ---- y as above; per 16-value block (the slices of 2 adjacent lanes)
        // the E4M3 scale from the block amax under the tensor scale, then
        // E2M1 codes
        const Nvfp4Tensor nt = make_nvfp4_tensor(*p.scale_in, nv_inv[127]);
        uint32_t *qo = (uint32_t *)((uint8_t *)p.out + (size_t)row * (size_t)(p.hidden / 2));
        uint8_t *so = (uint8_t *)p.scale_out + (size_t)row * (size_t)(p.hidden / 16);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lane + k * WPR * 64;
            uint32_t y[4];
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float p0, p1;
                y[e] = norm_word(rv[k][e], wv[k][e], rs, p0, p1);
                amax = __builtin_elementwise_maximum(
                    amax, __builtin_elementwise_maximum(__builtin_fabsf(p0), __builtin_fabsf(p1)));
            }
            if (late_ro && v < nvec) st_stream(late_ro + v, rv[k]);
            uint32_t mag = __float_as_uint(round_bf16(amax));
            mag = max(mag, dpp_u32<DPP_XOR1>(mag));
            if (v >= nvec) continue;
            const uint32_t sb = nv_scale_byte(mag, nt);
            const uint32_t q = (sb == 0x7Fu) ? 0u : pack_nvfp4<4>(y, sb, nt, nv_inv[sb]);
            st_stream(qo + v, q);
            if ((lane & 1) == 0) so[v >> 1] = (uint8_t)sb;
        }
    } else if constexpr (EPI == NORM_EPI_FP8_GROUP) {
        // ---- y as above; per 128-value group (the slices of 16 adjacent
        // lanes, one DPP row) the scale s = amax / 448, then the E4M3 codes of
        // y / s.  Every lane takes part in the group maximum (slices past the
        // row end hold w = 0, so y = 0; H is a multiple of 128, so a group is
        // all inside or all past the row end).
        uint8_t *qo = (uint8_t *)p.out + base;
        float *so = p.scale_out + (size_t)row * (size_t)(p.hidden / FP8_GROUP);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lane + k * WPR * 64;
            float yf[8];
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float p0, p1;
                const uint32_t y = norm_word(rv[k][e], wv[k][e], rs, p0, p1);
                yf[2 * e] = bf_lo(y);
                yf[2 * e + 1] = bf_hi(y);
                amax = fmaxf(amax, fmaxf(__builtin_fabsf(p0), __builtin_fabsf(p1)));
            }
            if (late_ro && v < nvec) st_stream(late_ro + v, rv[k]);
            amax = group_max<16>(round_bf16(amax));
            if (v >= nvec) continue;
            const float s = amax / 448.0f;
            if ((lane & 15) == 0) so[v >> 4] = s;
            const E4m3Scale qs = make_e4m3_scale(s);
            float z[8];
            // |y| <= amax, so |y / s| <= 448 (1 + 2^-24): no input clamp
            if (e4m3_scale_is_fast(qs)) {
#pragma unroll
                for (int j = 0; j < 8; ++j) z[j] = e4m3_quotient<true, false>(yf[j], qs);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) z[j] = e4m3_quotient<false, false>(yf[j], qs);
            }
            u32x2 q;
            q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
            q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
            st_stream((u32x2 *)(qo + (size_t)v * 8), q);
        }
    } else if constexpr (EPI == NORM_EPI_FP8_STATIC) {
        // ---- y as above, q = e4m3(clamp(y / s)) with the given scale
        const E4m3Scale qs = make_e4m3_scale(*p.scale_in);
        uint8_t *qo = (uint8_t *)p.out + base;
        if (e4m3_scale_is_fast(qs))
            store_static_fp8<WPR, VPT, true>(rv, wv, rs, qs, qo, lane, nvec, late_ro);
        else
            store_static_fp8<WPR, VPT, false>(rv, wv, rs, qs, qo, lane, nvec, late_ro);
    } else {
        // ---- y as above, kept as binary32 values of bf16; row amax (from
        // the products, rounded once).  Slices past the row end hold w = 0,
        // so y = 0 there.
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float h0 = KEEP ? hf[k][2 * e] : bf_lo(rv[k][e]);
                const float h1 = KEEP ? hf[k][2 * e + 1] : bf_hi(rv[k][e]);
                const uint32_t t = pack_bf16(h0 * rs, h1 * rs);
                const float p0 = bf_lo(wv[k][e]) * bf_lo(t), p1 = bf_hi(wv[k][e]) * bf_hi(t);
                const uint32_t y = pack_bf16(p0, p1);
                hf[k][2 * e] = bf_lo(y);
                hf[k][2 * e + 1] = bf_hi(y);
                amax = fmaxf(amax, fmaxf(__builtin_fabsf(p0), __builtin_fabsf(p1)));
            }
            const int v = lane + k * WPR * 64;
            if (late_ro && v < nvec) st_stream(late_ro + v, rv[k]);
        }
        amax = round_bf16(amax);
        AARMS_STAMP(4, amax);
        amax = wave_max(amax);
        AARMS_STAMP(5, amax);
        if constexpr (WPR > 1) {
            if ((lane & 63) == 0) pmax[lane >> 6] = amax;
            __syncthreads();
            AARMS_STAMP(6, amax);
            amax = block_max<WPR>(pmax, lane & 63);
            AARMS_STAMP_DETAIL(13, amax);
        }
        // ---- per-token scale, then q = e4m3(clamp(y / s))
        const float s = amax / 448.0f;
        if (lane == 0) p.scale_out[row] = s;
        const E4m3Scale qs = make_e4m3_scale(s);
        if constexpr (WPR > 1) AARMS_STAMP_DETAIL(14, qs.inv);
        uint8_t *qo = (uint8_t *)p.out + base;
        if (e4m3_scale_is_fast(qs))
            quantize_row<WPR, VPT, true, false>(hf, qs, qo, lane, nvec);
        else
            quantize_row<WPR, VPT, false, false>(hf, qs, qo, lane, nvec);
    }

    // ---- the updated residual, bf16 form
    if constexpr (RES && EPI == NORM_EPI_BF16) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lane + k * WPR * 64;
            if (v < nvec) st_stream(ro + v, rv[k]);
        }
    }
    AARMS_STAMP(7, 0.0f);
#ifdef AARMS_PHASE_STAMPS
    if (p.stamps && (lane & 63) == 0) {
        uint64_t *s = p.stamps + ((size_t)row * WPR + (size_t)(lane >> 6)) * 16;
        s[8] = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID
        s[9] = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID
    }
#endif
}

// NVFP4: 1/S for each of the 127 finite block scales and 1/(6 g) in the
// slot of the NaN scale byte, one correctly rounded division per thread at
// the start of the block (before any early exit: every thread reaches the
// barrier), instead of one per block of 16 values on the row's critical path.
template <int EPI>
__device__ __forceinline__ void fill_nv_table(const NormParams &p, float *nv_inv)
{
    if constexpr (EPI == NORM_EPI_NVFP4) {
        const float g = *p.scale_in;
        if (threadIdx.x < 127u)
            nv_inv[threadIdx.x] = nv_block_inverse(threadIdx.x, nv_tensor_scale(g));
        else if (threadIdx.x == 127u)
            nv_inv[127] = nv_six_inverse(g);
        __syncthreads();
    }
}

// One row per block (WPR > 1) or per wave (WPR == 1, four rows per block);
// one block per row or row quartet.
template <int WPR, int VPT, int EPI, bool RES>
__global__ void __launch_bounds__(WPR == 1 ? 256 : WPR * 64)
norm_kernel(NormParams p)
{
    constexpr int ROW_THREADS = WPR * 64;
    constexpr int ROWS_PER_BLOCK = (WPR == 1) ? 4 : 1;
    __shared__ double psum[WPR];
    __shared__ float pmax[WPR];
    __shared__ float nv_inv[EPI == NORM_EPI_NVFP4 ? 128 : 1];
    fill_nv_table<EPI>(p, nv_inv);

    const int tid = threadIdx.x;
    const int lane = tid % ROW_THREADS;
    // the row is uniform over the wave (WPR == 1) or the block, and is made a
    // scalar so that row addresses are scalar bases plus one lane offset
    const int64_t row = linear_block() * ROWS_PER_BLOCK +
                        (WPR == 1 ? __builtin_amdgcn_readfirstlane(tid / ROW_THREADS) : 0);
    // WPR == 1: the test is per wave (no block barrier follows); WPR > 1:
    // one row per block, so the whole block leaves together.
    if (row >= p.tokens) return;
    const int nvec = p.hidden >> 3;
    const uint64_t t_start = p.hold_ticks ? __builtin_amdgcn_s_memrealtime() : 0;
    AARMS_STAMP(0, 0.0f);

    // all loads of the row slice in flight before any use
    u32x4 xv[VPT], rv[VPT], wv[VPT];
    load_row<WPR, VPT, RES>(p, row, lane, nvec, xv, rv);
    // wide rows with the residual load the weight after the first pass (its
    // registers are not live during the row loads); without the residual
    // there are registers to spare and the weight is loaded with the row
    constexpr bool W_LATE = WPR > 1 && RES;
    if constexpr (!W_LATE) load_weight<WPR, VPT>(p, lane, nvec, wv);
    finish_row<WPR, VPT, EPI, RES, W_LATE>(p, row, lane, nvec, xv, rv, wv, psum, pmax, nv_inv, t_start);
}

// Persistent and software-pipelined: a fixed grid of blocks walks the rows
// (row, row + G, row + 2G, ...); the weight is loaded once per block, and the
// next row's x and residual are loaded before the current row is processed,
// so their latency hides behind its reductions and stores.  The blocks in
// flight always cover a window of G consecutive rows.
template <int WPR, int VPT, int EPI, bool RES>
__global__ void __launch_bounds__(WPR == 1 ? 256 : WPR * 64)
norm_kernel_pipelined(NormParams p)
{
    constexpr int ROW_THREADS = WPR * 64;
    constexpr int ROWS_PER_BLOCK = (WPR == 1) ? 4 : 1;
    // the bf16 form has one barrier per row, so a fast wave could write the
    // next row's partial sums while a slow one still reads these: two sets
    __shared__ double psum[2][WPR];
    __shared__ float pmax[WPR];
    __shared__ float nv_inv[EPI == NORM_EPI_NVFP4 ? 128 : 1];
    fill_nv_table<EPI>(p, nv_inv);

    const int tid = threadIdx.x;
    const int lane = tid % ROW_THREADS;
    const int64_t step = (int64_t)gridDim.x * ROWS_PER_BLOCK;
    int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK +
                  (WPR == 1 ? __builtin_amdgcn_readfirstlane(tid / ROW_THREADS) : 0);
    // uniform per block for WPR > 1, per wave for WPR == 1
    if (row >= p.tokens) return;
    const int nvec = p.hidden >> 3;

    u32x4 wv[VPT];
    load_weight<WPR, VPT>(p, lane, nvec, wv);
    u32x4 xa[VPT], ra[VPT];
    load_row<WPR, VPT, RES>(p, row, lane, nvec, xa, ra);
    int par = 0;
    while (true) {
        const int64_t next = row + step;
        const bool more = next < p.tokens;
        u32x4 xb[VPT], rb[VPT];
        if (more) {
            load_row<WPR, VPT, RES>(p, next, lane, nvec, xb, rb);
        } else {
#pragma unroll
            for (int k = 0; k < VPT; ++k) xb[k] = rb[k] = (u32x4)0u;
        }
        finish_row<WPR, VPT, EPI, RES, false>(p, row, lane, nvec, xa, ra, wv, psum[par], pmax, nv_inv);
        if (!more) break;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            xa[k] = xb[k];
            ra[k] = rb[k];
        }
        row = next;
        par ^= 1;
    }
}

// ---------------------------------------------------------------- variants

static const NormVariant kNormVariants[] = {
    {1, 1, 0, "wave/row x1 vec"},   {1, 2, 0, "wave/row x2 vec"},   {1, 3, 0, "wave/row x3 vec"},
    {1, 4, 0, "wave/row x4 vec"},   {1, 6, 0, "wave/row x6 vec"},   {1, 8, 0, "wave/row x8 vec"},
    {2, 2, 0, "2 waves/row x2 vec"}, {2, 4, 0, "2 waves/row x4 vec"}, {2, 8, 0, "2 waves/row x8 vec"},
    {4, 1, 0, "4 waves/row x1 vec"}, {4, 2, 0, "4 waves/row x2 vec"}, {4, 4, 0, "4 waves/row x4 vec"},
    {4, 8, 0, "4 waves/row x8 vec"}, {8, 1, 0, "8 waves/row x1 vec"}, {8, 2, 0, "8 waves/row x2 vec"},
    {8, 4, 0, "8 waves/row x4 vec"}, {8, 8, 0, "8 waves/row x8 vec"}, {16, 1, 0, "16 waves/row x1 vec"},
    {16, 2, 0, "16 waves/row x2 vec"}, {16, 4, 0, "16 waves/row x4 vec"}, {16, 8, 0, "16 waves/row x8 vec"},
    // persistent, software-pipelined (blocks per CU)
    {1, 3, 4, "wave/row x3 vec, pipelined 4 blocks/CU"},
    {1, 3, 8, "wave/row x3 vec, pipelined 8 blocks/CU"},
    {1, 4, 4, "wave/row x4 vec, pipelined 4 blocks/CU"},
    {8, 4, 2, "8 waves/row x4 vec, pipelined 2 blocks/CU"},
    {16, 2, 1, "16 waves/row x2 vec, pipelined 1 block/CU"},
    {8, 2, 2, "8 waves/row x2 vec, pipelined 2 blocks/CU"},
    {4, 4, 4, "4 waves/row x4 vec, pipelined 4 blocks/CU"},
    {16, 4, 1, "16 waves/row x4 vec, pipelined 1 block/CU"},
    {16, 8, 1, "16 waves/row x8 vec, pipelined 1 block/CU"},
    // one wave holds the whole row (norm_resident.hip)
    {1, 32, NORM_RESIDENT_Y_IN_PLACE, "wave/row x32 vec, resident, 6-slice window"},
    {1, 32, NORM_RESIDENT, "wave/row x32 vec, resident, 10-slice window"},
};
constexpr int kNumNormVariants = sizeof(kNormVariants) / sizeof(kNormVariants[0]);
static_assert(kNumNormVariants <= 64, "the occupancy cache holds 64 variants per form");

int norm_variant_count() { return kNumNormVariants; }
const NormVariant *norm_variant(int id)
{
    return (id >= 0 && id < kNumNormVariants) ? &kNormVariants[id] : nullptr;
}

// Blocks of a kernel resident per CU at once (the HIP occupancy calculator),
// cached per (epilogue, residual, variant); 0 if the query fails.
constexpr int kOccupancySlots = 6 * 2 * 64;

static int resident_blocks_per_cu(const void *fn, int threads, int slot)
{
    static std::atomic<int> cache[kOccupancySlots];
    if (slot < 0 || slot >= kOccupancySlots) return 0;
    int n = cache[slot].load(std::memory_order_relaxed);
    if (n != 0) return n > 0 ? n : 0;
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, threads, 0) != hipSuccess || b <= 0) b = -1;
    cache[slot].store(b, std::memory_order_relaxed);
    return b > 0 ? b : 0;
}

template <int WPR, int VPT, int EPI, bool RES, bool PIPE>
static hipError_t launch_one(const NormParams &p, int blocks_per_cu, int num_cus, int slot,
                             hipStream_t stream)
{
    constexpr int threads = (WPR == 1) ? 256 : WPR * 64;
    constexpr int rows_per_block = (WPR == 1) ? 4 : 1;
    int64_t blocks = (p.tokens + rows_per_block - 1) / rows_per_block;
    if (PIPE) {
        const int64_t cap = (int64_t)num_cus * blocks_per_cu;
        if (blocks > cap) blocks = cap;
    }
    NormParams copy = p;
    void *args[] = {&copy};
    const void *fn = PIPE ? (const void *)&norm_kernel_pipelined<WPR, VPT, EPI, RES>
                          : (const void *)&norm_kernel<WPR, VPT, EPI, RES>;
    // the store hold and the late residual stores of the quantised forms
    // only order the reads and writes of one generation of blocks: a grid
    // that does not fit on the device at once runs without them
    if (copy.hold_ticks != 0 || copy.res_last != 0) {
        const int rb = PIPE ? 0 : resident_blocks_per_cu(fn, threads, slot);
        if (rb <= 0 || blocks > (int64_t)rb * num_cus) copy.hold_ticks = copy.res_last = 0;
        if (copy.hold_ticks > NORM_HOLD_MAX_TICKS) copy.hold_ticks = NORM_HOLD_MAX_TICKS;
    }
    return hipLaunchKernel(fn, linear_grid(blocks, threads), dim3(threads), args, 0, stream);
}

template <int EPI, bool RES>
static hipError_t dispatch(const NormParams &p, int variant, int num_cus, hipStream_t s)
{
    const NormVariant *v = norm_variant(variant);
    if (!v) return hipErrorInvalidValue;
    const int b = v->blocks_per_cu;
    if (b < 0) return launch_norm_resident(p, EPI, RES, b, s);
    const int slot = (EPI * 2 + (RES ? 1 : 0)) * 64 + variant;
#define AARMS_NORM_CASE(W, V)                                                              \
    if (v->waves_per_row == W && v->vecs_per_lane == V)                                    \
        return b ? launch_one<W, V, EPI, RES, true>(p, b, num_cus, slot, s)                 \
                 : launch_one<W, V, EPI, RES, false>(p, 0, num_cus, slot, s);
    AARMS_NORM_CASE(1, 1)
    AARMS_NORM_CASE(1, 2)
    AARMS_NORM_CASE(1, 3)
    AARMS_NORM_CASE(1, 4)
    AARMS_NORM_CASE(1, 6)
    AARMS_NORM_CASE(1, 8)
    AARMS_NORM_CASE(2, 2)
    AARMS_NORM_CASE(2, 4)
    AARMS_NORM_CASE(2, 8)
    AARMS_NORM_CASE(4, 1)
    AARMS_NORM_CASE(4, 2)
    AARMS_NORM_CASE(4, 4)
    AARMS_NORM_CASE(4, 8)
    AARMS_NORM_CASE(8, 1)
    AARMS_NORM_CASE(8, 2)
    AARMS_NORM_CASE(8, 4)
    AARMS_NORM_CASE(8, 8)
    AARMS_NORM_CASE(16, 1)
    AARMS_NORM_CASE(16, 2)
    AARMS_NORM_CASE(16, 4)
    AARMS_NORM_CASE(16, 8)
#undef AARMS_NORM_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_norm(const NormParams &p, int epi, bool residual, int variant, int num_cus,
                       hipStream_t stream)
{
    switch (epi) {
    case NORM_EPI_BF16:
        return residual ? dispatch<NORM_EPI_BF16, true>(p, variant, num_cus, stream)
                        : dispatch<NORM_EPI_BF16, false>(p, variant, num_cus, stream);
    case NORM_EPI_FP8_DYNAMIC:
        return residual ? dispatch<NORM_EPI_FP8_DYNAMIC, true>(p, variant, num_cus, stream)
                        : dispatch<NORM_EPI_FP8_DYNAMIC, false>(p, variant, num_cus, stream);
    case NORM_EPI_FP8_STATIC:
        return residual ? dispatch<NORM_EPI_FP8_STATIC, true>(p, variant, num_cus, stream)
                        : dispatch<NORM_EPI_FP8_STATIC, false>(p, variant, num_cus, stream);
    case NORM_EPI_MXFP4:
        return residual ? dispatch<NORM_EPI_MXFP4, true>(p, variant, num_cus, stream)
                        : dispatch<NORM_EPI_MXFP4, false>(p, variant, num_cus, stream);
    case NORM_EPI_NVFP4:
        return residual ? dispatch<NORM_EPI_NVFP4, true>(p, variant, num_cus, stream)
                        : dispatch<NORM_EPI_NVFP4, false>(p, variant, num_cus, stream);
    case NORM_EPI_FP8_GROUP:
        return residual ? dispatch<NORM_EPI_FP8_GROUP, true>(p, variant, num_cus, stream)
                        : dispatch<NORM_EPI_FP8_GROUP, false>(p, variant, num_cus, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace aarms
