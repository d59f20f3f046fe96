// swiglu.hip -- silu(gate) * up over a concatenated gate_up row, for gfx950,
// with a bf16 epilogue or a quantised one: E4M3 with a per-tensor, a
// per-token or a per-128-output scale, MXFP4 or NVFP4.
//
// A job is 8 adjacent outputs of one row, fed by one 16-byte load of gate and
// one of up from the same row of gate_up (gate first, up second:
// "TensorRT-LLM: Compiling Inference Engines Ahead of Time", section "Fusing
// operations, measured", the swiglu kernel), or 4 outputs fed by 8-byte
// loads (twice the lanes, half the dependent arithmetic per lane: for
// launch-bound decode batches).  The grid is (column chunk,
// row): a block of 256 lanes takes 256 * U consecutive jobs of one row, so
// the row is a per-block scalar, every load and store of a wave is one
// contiguous stretch, and blocks are dispatched in memory order (one block
// per chunk, no grid-stride loop: the blocks in flight then cover one
// contiguous window of HBM).  Nothing is kept between jobs.  A flat form of
// the grid takes blocks of 256 jobs over the rows laid end to end instead
// (see swiglu_block), so that no lane idles at a row's end.
//
// The per-token (dynamic) E4M3 form needs the row's amax before any code is
// written, so there a row belongs to one wave or one block (as in the norm),
// every job's y stays packed in registers through the amax reduction, and
// the scale s = amax / 448 is written per row.
//
// SiLU is rounded once to bf16 before the product, and that rounding must be
// the correctly rounded one: the fast hardware exp2/rcp form is used unless
// its result sits near a bf16 midpoint, in which case that lane recomputes
// the element exactly (see device.h).  The FP8 epilogue is vLLM's SiLU-and-
// mul + quant fusion ("Introduction to torch.compile and How It Works with
// vLLM", sections 3 and 4).

#include "device.h"
#include "launch.h"

namespace aarms {

template <int W>
struct Words;
template <>
struct Words<4> {
    typedef u32x4 T;   // 8 bf16
    typedef u32x2 Q;   // 8 E4M3 codes
};
template <>
struct Words<2> {
    typedef u32x2 T;   // 4 bf16
    typedef uint32_t Q;  // 4 E4M3 codes
};

// Running maxima of |y| over jobs, taken on the binary32 products a * u
// before their bf16 rounding (the caller rounds the result once, round_bf16):
// AMAX_DROP_NAN folds with fmaxf, which drops NaN (the per-token and
// per-group scale rules); AMAX_KEEP_NAN with the NaN-propagating maximum (the
// FP4 block rules, where a NaN marks the block).
enum JobAmax : int { AMAX_NONE = 0, AMAX_DROP_NAN = 1, AMAX_KEEP_NAN = 2 };

// 2W outputs of one job: a = bf16(silu(g)), y = bf16(a * u).  Returns the
// bf16 results as W packed words.  Each word of the gate is turned into its
// word of a at once (two SiLUs, one pack), so only the packed words stay
// live; a lane with a flagged element redoes its words in the rare branch.
// With AMAX, amax also takes the job's |a * u| (see JobAmax).
template <int W, int AMAX = AMAX_NONE>
__device__ __forceinline__ typename Words<W>::T swiglu_job(typename Words<W>::T gv, typename Words<W>::T uv,
                                                          float &amax)
{
    uint32_t a[W];
    // running extrema: smallest knife-edge key of the results, largest gate
    // bit pattern (above SILU_FAST_MIN_BITS means g < -16)
    uint32_t kmin = 0xFFFFFFFFu, gmax = 0u;
#pragma unroll
    for (int e = 0; e < W; ++e) {
        const uint32_t glo = gv[e] << 16, ghi = gv[e] & 0xFFFF0000u;
        const float s0 = silu_fast(__uint_as_float(glo)), s1 = silu_fast(__uint_as_float(ghi));
        kmin = min(kmin, min(silu_edge_key(s0), silu_edge_key(s1)));
        gmax = max(gmax, max(glo, ghi));
        a[e] = pack_bf16(s0, s1);
    }
    if (kmin <= SILU_EDGE_KEY_MAX || gmax > SILU_FAST_MIN_BITS) {
        // rare: recompute this lane's words, the flagged elements exactly.
        // The empty asm hides the gate word's earlier uses, so the fast values
        // are recomputed here instead of being kept live on the hot path.
#pragma unroll
        for (int e = 0; e < W; ++e) {
            uint32_t w = gv[e];
            asm volatile("" : "+v"(w));
            const uint32_t glo = w << 16, ghi = w & 0xFFFF0000u;
            float s0 = silu_fast(__uint_as_float(glo)), s1 = silu_fast(__uint_as_float(ghi));
            if (silu_edge_key(s0) <= SILU_EDGE_KEY_MAX || glo > SILU_FAST_MIN_BITS)
                s0 = silu_exact(__uint_as_float(glo));
            if (silu_edge_key(s1) <= SILU_EDGE_KEY_MAX || ghi > SILU_FAST_MIN_BITS)
                s1 = silu_exact(__uint_as_float(ghi));
            a[e] = pack_bf16(s0, s1);
        }
    }
    typename Words<W>::T y;
#pragma unroll
    for (int e = 0; e < W; ++e) {
        const float p0 = bf_lo(a[e]) * bf_lo(uv[e]), p1 = bf_hi(a[e]) * bf_hi(uv[e]);
        y[e] = pack_bf16(p0, p1);
        if constexpr (AMAX == AMAX_DROP_NAN)
            amax = fmaxf(amax, fmaxf(__builtin_fabsf(p0), __builtin_fabsf(p1)));
        else if constexpr (AMAX == AMAX_KEEP_NAN)
            amax = __builtin_elementwise_maximum(
                amax, __builtin_elementwise_maximum(__builtin_fabsf(p0), __builtin_fabsf(p1)));
    }
    return y;
}

template <int W>
__device__ __forceinline__ typename Words<W>::T swiglu_job(typename Words<W>::T gv, typename Words<W>::T uv)
{
    float unused = 0.0f;
    return swiglu_job<W, AMAX_NONE>(gv, uv, unused);
}

// MXFP4 block of 32 outputs = the jobs of 32 / (2W) adjacent lanes: the
// block amax of magnitude bits over those lanes (DPP), its E8M0 byte, then
// the E2M1 codes of this lane's 2W outputs (see device.h).
template <int W>
__device__ __forceinline__ uint32_t mx_block_max(uint32_t mag)
{
    mag = max(mag, dpp_u32<DPP_XOR1>(mag));
    mag = max(mag, dpp_u32<DPP_XOR2>(mag));
    if constexpr (W == 2) mag = max(mag, dpp_u32<DPP_HALF_MIRROR>(mag));
    return mag;
}

// MODE 0: bf16 output; 1: E4M3 output, fast quotient; 2: E4M3, IEEE
// division; 3: MXFP4 (codes to out, E8M0 block scales to scale_out); 4:
// NVFP4 (codes to out, E4M3 block scales to scale_out, tensor scale read
// from scale); 5: E4M3 with an fp32 scale per 128 outputs (scale_out).
// FLAT: the grid is one dimension of 256-job blocks over the rows laid end
// to end (U = 1, W = 4), so no lane idles at a row's end (a row of 1,120
// jobs fills 4.375 blocks of the row-chunked grid).  With at least 256 jobs
// per row a block spans at most two rows: the first is a per-block scalar
// (a division by the row length with the host's magic numbers), and a lane
// whose job lies past that row's end takes it from the next row.
template <int U, int W, int MODE, bool FLAT = false>
__device__ __forceinline__ void swiglu_block(const SwigluParams &p, const E4m3Scale &qs)
{
    typedef typename Words<W>::T V;
    const uint32_t njobs = p.vecs_per_row * (4 / W);
    // per job slot: its index in the row-major [T, njobs] job space (outputs
    // and block scales are indexed by it), whether it exists, and its gate
    // vector (the up vector is njobs further)
    uint64_t jout[U];
    bool ok[U];
    const V *gsrc[U];
    if constexpr (FLAT) {
        static_assert(U == 1 && W == 4, "flat grids take one 8-output job per lane");
        const uint32_t j0 = blockIdx.x * 256u;
        const uint32_t t1 = __umulhi(j0, p.div_magic);
        const uint32_t row0 = (t1 + ((j0 - t1) >> p.div_shift1)) >> p.div_shift2;
        const uint32_t c = j0 - row0 * njobs + threadIdx.x;
        const bool next = c >= njobs;
        // row (row0 + next), column c - (next ? njobs : 0): gate vector
        // 2 njobs (row0 + next) + c - (next ? njobs : 0)
        gsrc[0] = (const V *)p.gate_up + (uint64_t)row0 * 2u * njobs + (c + (next ? njobs : 0u));
        jout[0] = (uint64_t)j0 + threadIdx.x;
        ok[0] = (uint64_t)row0 + (next ? 1u : 0u) < (uint64_t)p.tokens;
    } else {
        const uint64_t row = (uint64_t)blockIdx.z * SWIGLU_ROWS_PER_Y + blockIdx.y;
        if (row >= (uint64_t)p.tokens) return;
        const uint32_t c0 = blockIdx.x * (256u * U) + threadIdx.x;
        const V *gate = (const V *)((const uint16_t *)p.gate_up + row * 2u * (uint64_t)p.inter);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = c0 + 256u * u;
            ok[u] = c < njobs;
            jout[u] = row * njobs + c;
            gsrc[u] = gate + c;
        }
    }
    V gv[U], uv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        gv[u] = ok[u] ? ld_stream(gsrc[u]) : (V)0u;
        uv[u] = ok[u] ? ld_stream(gsrc[u] + njobs) : (V)0u;
    }
    if constexpr (MODE == 3) {
        // every lane takes part in the block maxima (slots past the row end
        // hold zeros; N is a multiple of 32, so a block is all in or all out)
        constexpr uint32_t LANES = 16 / W;       // lanes per 32-output block
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float amax = 0.0f;
            const V y = swiglu_job<W, AMAX_KEEP_NAN>(gv[u], uv[u], amax);
            // magnitude bits of the job's largest |y| (a NaN or Inf gives bits
            // at or above 0x7F800000: the NaN scale)
            const uint32_t mag = mx_block_max<W>(__float_as_uint(round_bf16(amax)));
            if (!ok[u]) continue;
            const uint32_t sb = mx_scale_byte(mag);
            const float inv = __uint_as_float((254u - (sb == 0xFFu ? 127u : sb)) << 23);
            if constexpr (W == 4) {
                const uint32_t w4[4] = {y[0], y[1], y[2], y[3]};
                const uint32_t q = (sb == 0xFFu) ? 0u : pack_e2m1x8(w4, inv);
                st_stream((uint32_t *)p.out + jout[u], q);
            } else {
                uint32_t q = 0;
                if (sb != 0xFFu) {
                    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, bf_lo(y[0]) * inv, bf_hi(y[0]) * inv, 1.0f, 0);
                    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, bf_lo(y[1]) * inv, bf_hi(y[1]) * inv, 1.0f, 1);
                }
                st_stream((uint16_t *)p.out + jout[u], (uint16_t)q);
            }
            if (jout[u] % LANES == 0) ((uint8_t *)p.scale_out)[jout[u] / LANES] = (uint8_t)sb;
        }
        return;
    }
    if constexpr (MODE == 4) {
        // a 16-output block is the jobs of 2 adjacent lanes (4 for half jobs)
        constexpr uint32_t LANES = 8 / W;
        // 1/S for each of the 127 finite block scales, and 1/(6 g) in the
        // slot of the NaN scale byte (which never divides): one correctly
        // rounded division per thread while the loads are in flight, instead
        // of per job (the row test above is uniform per block, so every
        // thread reaches the barrier)
        const float g = *p.scale;
        __shared__ float nv_inv[128];
        if (threadIdx.x < 127u)
            nv_inv[threadIdx.x] = nv_block_inverse(threadIdx.x, nv_tensor_scale(g));
        else if (threadIdx.x == 127u)
            nv_inv[127] = nv_six_inverse(g);
        __syncthreads();
        const Nvfp4Tensor nt = make_nvfp4_tensor(g, nv_inv[127]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float amax = 0.0f;
            const V y = swiglu_job<W, AMAX_KEEP_NAN>(gv[u], uv[u], amax);
            uint32_t w[W];
#pragma unroll
            for (int e = 0; e < W; ++e) w[e] = y[e];
            uint32_t mag = __float_as_uint(round_bf16(amax));
            mag = max(mag, dpp_u32<DPP_XOR1>(mag));
            if constexpr (W == 2) mag = max(mag, dpp_u32<DPP_XOR2>(mag));
            if (!ok[u]) continue;
            const uint32_t sb = nv_scale_byte(mag, nt);
            const uint32_t q = (sb == 0x7Fu) ? 0u : pack_nvfp4<W>(w, sb, nt, nv_inv[sb]);
            if constexpr (W == 4)
                st_stream((uint32_t *)p.out + jout[u], q);
            else
                st_stream((uint16_t *)p.out + jout[u], (uint16_t)q);
            if (jout[u] % LANES == 0) ((uint8_t *)p.scale_out)[jout[u] / LANES] = (uint8_t)sb;
        }
        return;
    }
    if constexpr (MODE == 5) {
        // per 128 outputs (the jobs of 16 adjacent lanes, 32 for half jobs)
        // the scale s = amax / 448, then the E4M3 codes of y / s; every lane
        // takes part in the group maximum (slots past the row end hold zeros;
        // N is a multiple of 128, so a group is all in or all out)
        constexpr uint32_t LANES = FP8_GROUP / (2 * W);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float amax = 0.0f;
            const V y = swiglu_job<W, AMAX_DROP_NAN>(gv[u], uv[u], amax);
            float yf[2 * W];
#pragma unroll
            for (int e = 0; e < W; ++e) {
                yf[2 * e] = bf_lo(y[e]);
                yf[2 * e + 1] = bf_hi(y[e]);
            }
            amax = group_max<LANES>(round_bf16(amax));
            if (!ok[u]) continue;
            const float s = amax / 448.0f;
            // the scales are [T, N / 128] row-major: scale index = job index / LANES
            if (jout[u] % LANES == 0) p.scale_out[jout[u] / LANES] = s;
            const E4m3Scale gs = make_e4m3_scale(s);
            float z[2 * W];
            // |y| <= amax, so |y / s| <= 448 (1 + 2^-24): no input clamp
            if (e4m3_scale_is_fast(gs)) {
#pragma unroll
                for (int j = 0; j < 2 * W; ++j) z[j] = e4m3_quotient<true, false>(yf[j], gs);
            } else {
#pragma unroll
                for (int j = 0; j < 2 * W; ++j) z[j] = e4m3_quotient<false, false>(yf[j], gs);
            }
            typename Words<W>::Q q;
            if constexpr (W == 4) {
                q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
                q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
            } else {
                q = pack_e4m3x4(z[0], z[1], z[2], z[3]);
            }
            st_stream((typename Words<W>::Q *)p.out + jout[u], q);
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const V y = swiglu_job<W>(gv[u], uv[u]);
        if constexpr (MODE == 0) {
            st_stream((V *)p.out + jout[u], y);
        } else {
            float z[2 * W];
#pragma unroll
            for (int e = 0; e < W; ++e) {
                z[2 * e] = e4m3_quotient<MODE == 1>(bf_lo(y[e]), qs);
                z[2 * e + 1] = e4m3_quotient<MODE == 1>(bf_hi(y[e]), qs);
            }
            typename Words<W>::Q q;
            if constexpr (W == 4) {
                q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
                q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
            } else {
                q = pack_e4m3x4(z[0], z[1], z[2], z[3]);
            }
            st_stream((typename Words<W>::Q *)p.out + jout[u], q);
        }
    }
}

template <int U, int W, int EPI, bool FLAT = false>
__global__ void __launch_bounds__(256) swiglu_kernel(SwigluParams p)
{
    if constexpr (EPI == SWIGLU_EPI_FP8) {
        const E4m3Scale qs = make_e4m3_scale(*p.scale);
        if (e4m3_scale_is_fast(qs))
            swiglu_block<U, W, 1, FLAT>(p, qs);
        else
            swiglu_block<U, W, 2, FLAT>(p, qs);
    } else if constexpr (EPI == SWIGLU_EPI_MXFP4) {
        swiglu_block<U, W, 3, FLAT>(p, E4m3Scale{});
    } else if constexpr (EPI == SWIGLU_EPI_NVFP4) {
        swiglu_block<U, W, 4, FLAT>(p, E4m3Scale{});
    } else if constexpr (EPI == SWIGLU_EPI_FP8_GROUP) {
        swiglu_block<U, W, 5, FLAT>(p, E4m3Scale{});
    } else {
        swiglu_block<U, W, 0, FLAT>(p, E4m3Scale{});
    }
}

// Per-token E4M3: one row per wave (WPR == 1, four rows per 256-thread
// block) or per block of WPR waves, JPT jobs per lane.
template <int WPR, int JPT, bool FAST>
__device__ __forceinline__ void rowq_store(const u32x4 (&y)[JPT], const E4m3Scale &qs, u32x2 *qo,
                                           int lane, uint32_t njobs)
{
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
        const uint32_t v = lane + k * WPR * 64;
        if (v >= njobs) continue;
        float z[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // |y| <= amax, so |y / s| <= 448 (1 + 2^-24): no input clamp needed
            z[2 * e] = e4m3_quotient<FAST, false>(bf_lo(y[k][e]), qs);
            z[2 * e + 1] = e4m3_quotient<FAST, false>(bf_hi(y[k][e]), qs);
        }
        u32x2 q;
        q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
        q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
        st_stream(qo + v, q);
    }
}

template <int WPR, int JPT>
__global__ void __launch_bounds__(WPR == 1 ? 256 : WPR * 64) swiglu_rowq_kernel(SwigluParams p)
{
    constexpr int ROW_THREADS = WPR * 64;
    constexpr int ROWS_PER_BLOCK = (WPR == 1) ? 4 : 1;
    __shared__ float pmax[WPR];

    const int tid = threadIdx.x;
    const int lane = tid % ROW_THREADS;
    const int64_t row = linear_block() * ROWS_PER_BLOCK +
                        (WPR == 1 ? __builtin_amdgcn_readfirstlane(tid / ROW_THREADS) : 0);
    // uniform per wave (WPR == 1: no block barrier follows) or per block
    if (row >= p.tokens) return;
    const uint32_t njobs = p.vecs_per_row;
    const u32x4 *gate = (const u32x4 *)((const uint16_t *)p.gate_up + (uint64_t)row * 2u * (uint64_t)p.inter);
    const u32x4 *up = gate + njobs;

    u32x4 y[JPT], uv[JPT];
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
        const uint32_t v = lane + k * ROW_THREADS;
        const bool ok = v < njobs;
        y[k] = ok ? ld_stream(gate + v) : (u32x4)0u;
        uv[k] = ok ? ld_stream(up + v) : (u32x4)0u;
    }
    // y in place of the gate; slots past the row end hold gate = up = 0, so
    // y = 0 there and the amax is unaffected
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < JPT; ++k) y[k] = swiglu_job<4, AMAX_DROP_NAN>(y[k], uv[k], amax);
    amax = wave_max(round_bf16(amax));
    if constexpr (WPR > 1) {
        if ((lane & 63) == 0) pmax[lane >> 6] = amax;
        __syncthreads();
        amax = block_max<WPR>(pmax, lane & 63);
    }
    const float s = amax / 448.0f;
    if (lane == 0) p.scale_out[row] = s;
    const E4m3Scale qs = make_e4m3_scale(s);
    u32x2 *qo = (u32x2 *)p.out + (uint64_t)row * njobs;
    if (e4m3_scale_is_fast(qs))
        rowq_store<WPR, JPT, true>(y, qs, qo, lane, njobs);
    else
        rowq_store<WPR, JPT, false>(y, qs, qo, lane, njobs);
}

static const SwigluRowVariant kSwigluRowVariants[] = {
    {1, 1, "wave/row x1 job"},   {1, 2, "wave/row x2 jobs"},   {1, 4, "wave/row x4 jobs"},
    {4, 2, "4 waves/row x2 jobs"},  {4, 4, "4 waves/row x4 jobs"},
    {8, 2, "8 waves/row x2 jobs"},  {8, 3, "8 waves/row x3 jobs"},  {8, 4, "8 waves/row x4 jobs"},
    {16, 2, "16 waves/row x2 jobs"}, {16, 3, "16 waves/row x3 jobs"}, {16, 4, "16 waves/row x4 jobs"},
    {16, 8, "16 waves/row x8 jobs"},
};
constexpr int kNumSwigluRowVariants = sizeof(kSwigluRowVariants) / sizeof(kSwigluRowVariants[0]);

int swiglu_row_variant_count() { return kNumSwigluRowVariants; }
const SwigluRowVariant *swiglu_row_variant(int id)
{
    return (id >= 0 && id < kNumSwigluRowVariants) ? &kSwigluRowVariants[id] : nullptr;
}

template <int WPR, int JPT>
static hipError_t launch_rowq(const SwigluParams &p, hipStream_t stream)
{
    constexpr int threads = (WPR == 1) ? 256 : WPR * 64;
    constexpr int rows_per_block = (WPR == 1) ? 4 : 1;
    const int64_t blocks = (p.tokens + rows_per_block - 1) / rows_per_block;
    SwigluParams copy = p;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)&swiglu_rowq_kernel<WPR, JPT>, linear_grid(blocks, threads),
                           dim3(threads), args, 0, stream);
}

hipError_t launch_swiglu_rowq(const SwigluParams &p, int variant, hipStream_t s)
{
    const SwigluRowVariant *v = swiglu_row_variant(variant);
    if (!v) return hipErrorInvalidValue;
#define AARMS_ROWQ_CASE(W, J) \
    if (v->waves_per_row == W && v->jobs_per_lane == J) return launch_rowq<W, J>(p, s);
    AARMS_ROWQ_CASE(1, 1)
    AARMS_ROWQ_CASE(1, 2)
    AARMS_ROWQ_CASE(1, 4)
    AARMS_ROWQ_CASE(4, 2)
    AARMS_ROWQ_CASE(4, 4)
    AARMS_ROWQ_CASE(8, 2)
    AARMS_ROWQ_CASE(8, 3)
    AARMS_ROWQ_CASE(8, 4)
    AARMS_ROWQ_CASE(16, 2)
    AARMS_ROWQ_CASE(16, 3)
    AARMS_ROWQ_CASE(16, 4)
    AARMS_ROWQ_CASE(16, 8)
#undef AARMS_ROWQ_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- variants

static const SwigluVariant kSwigluVariants[] = {
    {1, 8, 0, "1 job/lane"},
    {2, 8, 0, "2 jobs/lane"},
    {4, 8, 0, "4 jobs/lane"},
    {1, 4, 0, "1 half job/lane"},
    {1, 8, 1, "1 job/lane, flat rows"},
};
constexpr int kNumSwigluVariants = sizeof(kSwigluVariants) / sizeof(kSwigluVariants[0]);

int swiglu_variant_count() { return kNumSwigluVariants; }
const SwigluVariant *swiglu_variant(int id)
{
    return (id >= 0 && id < kNumSwigluVariants) ? &kSwigluVariants[id] : nullptr;
}

template <int U, int W, int EPI>
static hipError_t launch_one(const SwigluParams &p, hipStream_t stream)
{
    const uint32_t per_block = 256u * U;
    const uint32_t njobs = p.vecs_per_row * (4 / W);
    const uint64_t T = (uint64_t)p.tokens;
    const dim3 grid((njobs + per_block - 1) / per_block,
                    (unsigned)(T < SWIGLU_ROWS_PER_Y ? T : SWIGLU_ROWS_PER_Y),
                    (unsigned)((T + SWIGLU_ROWS_PER_Y - 1) / SWIGLU_ROWS_PER_Y));
    SwigluParams copy = p;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)&swiglu_kernel<U, W, EPI>, grid, dim3(256), args, 0, stream);
}

// The flat grid (see swiglu_block): ceil(T * njobs / 256) blocks of 256
// jobs.  Rows under 256 jobs, or a launch of 2^32 jobs or more, take the
// row-chunked grid of one job per lane instead (same results).
template <int EPI>
static hipError_t launch_flat(const SwigluParams &p, hipStream_t stream)
{
    const uint32_t d = p.vecs_per_row;
    const uint64_t jobs = (uint64_t)p.tokens * d;
    if (d < 256u || jobs > 0xFFFFFF00ull) return launch_one<1, 4, EPI>(p, stream);
    SwigluParams copy = p;
    // floor(n / d) for every 32-bit n (Granlund and Montgomery's round-up
    // method): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1 < 2^32
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    copy.div_magic = (uint32_t)((((1ull << l) - d) << 32) / d + 1u);
    copy.div_shift1 = l < 1u ? l : 1u;
    copy.div_shift2 = l < 1u ? 0u : l - 1u;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)&swiglu_kernel<1, 4, EPI, true>, dim3((unsigned)((jobs + 255u) / 256u)),
                           dim3(256), args, 0, stream);
}

template <int Q>
static hipError_t dispatch(const SwigluParams &p, int variant, hipStream_t s)
{
    const SwigluVariant *v = swiglu_variant(variant);
    if (!v) return hipErrorInvalidValue;
    if (v->flat) return (v->jobs_per_lane == 1 && v->job_outputs == 8) ? launch_flat<Q>(p, s) : hipErrorInvalidValue;
    if (v->job_outputs == 8) {
        switch (v->jobs_per_lane) {
        case 1: return launch_one<1, 4, Q>(p, s);
        case 2: return launch_one<2, 4, Q>(p, s);
        case 4: return launch_one<4, 4, Q>(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (v->job_outputs == 4 && v->jobs_per_lane == 1) return launch_one<1, 2, Q>(p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_swiglu(const SwigluParams &p, int epi, int variant, hipStream_t stream)
{
    switch (epi) {
    case SWIGLU_EPI_BF16: return dispatch<SWIGLU_EPI_BF16>(p, variant, stream);
    case SWIGLU_EPI_FP8: return dispatch<SWIGLU_EPI_FP8>(p, variant, stream);
    case SWIGLU_EPI_MXFP4: return dispatch<SWIGLU_EPI_MXFP4>(p, variant, stream);
    case SWIGLU_EPI_NVFP4: return dispatch<SWIGLU_EPI_NVFP4>(p, variant, stream);
    case SWIGLU_EPI_FP8_GROUP: return dispatch<SWIGLU_EPI_FP8_GROUP>(p, variant, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace aarms
