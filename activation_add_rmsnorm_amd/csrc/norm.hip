// norm.hip -- fused residual add + RMSNorm for gfx950, with a bf16 epilogue
// or a dynamic per-token E4M3 epilogue.
//
// One pass over HBM: x and residual are read once with 16-byte streaming
// loads, the updated residual and the output are written once, and the row stays in
// registers between the reduction and the epilogue.  A row is handled by one
// wave (narrow rows, four rows per 256-thread block) or by a whole block of
// 2..16 waves (wide rows).  The sum of squares is accumulated per lane in
// binary64, reduced with a wave butterfly and, across waves, through LDS in
// a fixed order, so results are bitwise reproducible.
//
// The arithmetic follows the eight-operation RMSNorm with the residual add
// in front ("TensorRT-LLM: Compiling Inference Engines Ahead of Time",
// section "Fusing operations, measured"); the FP8 epilogue follows vLLM's
// RMSNorm + quant fusion ("Introduction to torch.compile and How It Works
// with vLLM", section 4).

#include "device.h"
#include "launch.h"

namespace aarms {

// q = e4m3(clamp(y / s)) for this lane's slices of the row, stored as 8-byte
// groups.
template <int WPR, int VPT, bool FAST>
__device__ __forceinline__ void quantize_row(const u32x4 (&yv)[VPT], const E4m3Scale &qs,
                                             uint8_t *qo, int lane, int nvec)
{
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * WPR * 64;
        if (v >= nvec) continue;
        float z[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[2 * e] = e4m3_quotient<FAST>(bf_lo(yv[k][e]), qs);
            z[2 * e + 1] = e4m3_quotient<FAST>(bf_hi(yv[k][e]), qs);
        }
        u32x2 q;
        q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
        q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
        st_stream((u32x2 *)(qo + (size_t)v * 8), q);
    }
}

template <int WPR, int VPT, bool QUANT>
__global__ void __launch_bounds__(WPR == 1 ? 256 : WPR * 64)
norm_kernel(NormParams p)
{
    constexpr int ROW_THREADS = WPR * 64;
    constexpr int ROWS_PER_BLOCK = (WPR == 1) ? 4 : 1;
    __shared__ double part_sum[WPR];
    __shared__ float part_max[WPR];

    const int tid = threadIdx.x;
    const int lane = tid % ROW_THREADS;
    const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + tid / ROW_THREADS;
    // WPR == 1: the test is per wave (no block barrier follows); WPR > 1:
    // one row per block, so the whole block leaves together.
    if (row >= p.tokens) return;

    const int H = p.hidden;
    const int nvec = H >> 3;
    const size_t base = (size_t)row * (size_t)H;
    const u32x4 *xr = (const u32x4 *)((const uint16_t *)p.x + base);
    const u32x4 *rr = (const u32x4 *)((const uint16_t *)p.residual + base);
    const u32x4 *wr = (const u32x4 *)p.weight;
    u32x4 *ro = (u32x4 *)((uint16_t *)p.residual_out + base);

    // ---- load the row slice (all loads in flight before any use)
    u32x4 xv[VPT], rv[VPT], wv[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * ROW_THREADS;
        const bool ok = v < nvec;
        xv[k] = ok ? ld_stream(xr + v) : (u32x4)0u;
        rv[k] = ok ? ld_stream(rr + v) : (u32x4)0u;
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * ROW_THREADS;
        wv[k] = (v < nvec) ? wr[v] : (u32x4)0u;
    }

    // ---- residual add (binary32, one rounding), store, sum of squares
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * ROW_THREADS;
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[e] = pack_bf16(bf_lo(xv[k][e]) + bf_lo(rv[k][e]), bf_hi(xv[k][e]) + bf_hi(rv[k][e]));
        rv[k] = r;
        if (v < nvec) st_stream(ro + v, r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double h0 = (double)bf_lo(r[e]);
            const double h1 = (double)bf_hi(r[e]);
            acc = __builtin_fma(h0, h0, acc);
            acc = __builtin_fma(h1, h1, acc);
        }
    }
    acc = wave_sum(acc);
    if constexpr (WPR > 1) {
        if ((lane & 63) == 0) part_sum[lane >> 6] = acc;
        __syncthreads();
        acc = part_sum[0];
#pragma unroll
        for (int i = 1; i < WPR; ++i) acc += part_sum[i];
    }

    // ---- mean (rounded once to binary32), + eps, reciprocal square root
    const float mean = (float)(acc / (double)H);
    const float var = mean + p.eps;
    const float rs = (float)(1.0 / sqrt((double)var));

    if constexpr (!QUANT) {
        // ---- t = bf16(h * rs), y = bf16(w * t)
        u32x4 *o = (u32x4 *)((uint16_t *)p.out + base);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lane + k * ROW_THREADS;
            if (v >= nvec) continue;
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t t = pack_bf16(bf_lo(rv[k][e]) * rs, bf_hi(rv[k][e]) * rs);
                y[e] = pack_bf16(bf_lo(wv[k][e]) * bf_lo(t), bf_hi(wv[k][e]) * bf_hi(t));
            }
            st_stream(o + v, y);
        }
    } else {
        // ---- y as above, kept in registers; row amax
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t t = pack_bf16(bf_lo(rv[k][e]) * rs, bf_hi(rv[k][e]) * rs);
                y[e] = pack_bf16(bf_lo(wv[k][e]) * bf_lo(t), bf_hi(wv[k][e]) * bf_hi(t));
                amax = fmaxf(amax, fmaxf(__builtin_fabsf(bf_lo(y[e])), __builtin_fabsf(bf_hi(y[e]))));
            }
            rv[k] = y;   // slices past the row end hold w = 0, so y = 0
        }
        amax = wave_max(amax);
        if constexpr (WPR > 1) {
            if ((lane & 63) == 0) part_max[lane >> 6] = amax;
            __syncthreads();
            amax = part_max[0];
#pragma unroll
            for (int i = 1; i < WPR; ++i) amax = fmaxf(amax, part_max[i]);
        }
        // ---- per-token scale, then q = e4m3(clamp(y / s))
        const float s = amax / 448.0f;
        if (lane == 0) p.scale_out[row] = s;
        const E4m3Scale qs = make_e4m3_scale(s);
        uint8_t *qo = (uint8_t *)p.out + base;
        if (e4m3_scale_is_fast(qs))
            quantize_row<WPR, VPT, true>(rv, qs, qo, lane, nvec);
        else
            quantize_row<WPR, VPT, false>(rv, qs, qo, lane, nvec);
    }
}

// ---------------------------------------------------------------- variants

static const NormVariant kNormVariants[] = {
    {1, 1, "wave/row x1 vec"},   {1, 2, "wave/row x2 vec"},   {1, 3, "wave/row x3 vec"},
    {1, 4, "wave/row x4 vec"},   {1, 6, "wave/row x6 vec"},   {1, 8, "wave/row x8 vec"},
    {2, 2, "2 waves/row x2 vec"}, {2, 4, "2 waves/row x4 vec"}, {2, 8, "2 waves/row x8 vec"},
    {4, 1, "4 waves/row x1 vec"}, {4, 2, "4 waves/row x2 vec"}, {4, 4, "4 waves/row x4 vec"},
    {4, 8, "4 waves/row x8 vec"}, {8, 1, "8 waves/row x1 vec"}, {8, 2, "8 waves/row x2 vec"},
    {8, 4, "8 waves/row x4 vec"}, {8, 8, "8 waves/row x8 vec"}, {16, 1, "16 waves/row x1 vec"},
    {16, 2, "16 waves/row x2 vec"}, {16, 4, "16 waves/row x4 vec"}, {16, 8, "16 waves/row x8 vec"},
};
constexpr int kNumNormVariants = sizeof(kNormVariants) / sizeof(kNormVariants[0]);

int norm_variant_count() { return kNumNormVariants; }
const NormVariant *norm_variant(int id)
{
    return (id >= 0 && id < kNumNormVariants) ? &kNormVariants[id] : nullptr;
}

template <int WPR, int VPT, bool Q>
static hipError_t launch_one(const NormParams &p, hipStream_t stream)
{
    constexpr int threads = (WPR == 1) ? 256 : WPR * 64;
    constexpr int rows_per_block = (WPR == 1) ? 4 : 1;
    const dim3 grid((unsigned)((p.tokens + rows_per_block - 1) / rows_per_block));
    NormParams copy = p;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)&norm_kernel<WPR, VPT, Q>, grid, dim3(threads), args, 0,
                           stream);
}

template <bool Q>
static hipError_t dispatch(const NormParams &p, int variant, hipStream_t s)
{
    switch (variant) {
    case 0: return launch_one<1, 1, Q>(p, s);
    case 1: return launch_one<1, 2, Q>(p, s);
    case 2: return launch_one<1, 3, Q>(p, s);
    case 3: return launch_one<1, 4, Q>(p, s);
    case 4: return launch_one<1, 6, Q>(p, s);
    case 5: return launch_one<1, 8, Q>(p, s);
    case 6: return launch_one<2, 2, Q>(p, s);
    case 7: return launch_one<2, 4, Q>(p, s);
    case 8: return launch_one<2, 8, Q>(p, s);
    case 9: return launch_one<4, 1, Q>(p, s);
    case 10: return launch_one<4, 2, Q>(p, s);
    case 11: return launch_one<4, 4, Q>(p, s);
    case 12: return launch_one<4, 8, Q>(p, s);
    case 13: return launch_one<8, 1, Q>(p, s);
    case 14: return launch_one<8, 2, Q>(p, s);
    case 15: return launch_one<8, 4, Q>(p, s);
    case 16: return launch_one<8, 8, Q>(p, s);
    case 17: return launch_one<16, 1, Q>(p, s);
    case 18: return launch_one<16, 2, Q>(p, s);
    case 19: return launch_one<16, 4, Q>(p, s);
    case 20: return launch_one<16, 8, Q>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_norm(const NormParams &p, bool quant, int variant, hipStream_t stream)
{
    return quant ? dispatch<true>(p, variant, stream) : dispatch<false>(p, variant, stream);
}

}  // namespace aarms
