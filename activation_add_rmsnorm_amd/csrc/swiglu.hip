// swiglu.hip -- silu(gate) * up over a concatenated gate_up row, with a bf16
// epilogue or a static per-tensor E4M3 epilogue, for gfx950.
//
// The output is a flat sequence of jobs; a job is 8 adjacent outputs of one
// row, fed by one 16-byte load of gate and one of up from the same row of
// gate_up (gate first, up second: "TensorRT-LLM: Compiling Inference Engines
// Ahead of Time", section "Fusing operations, measured", the swiglu kernel).
// Consecutive lanes take consecutive jobs, so every load and store of a wave
// is one contiguous stretch.  Nothing is kept between jobs: the kernel is a
// pure stream, bounded by HBM bandwidth and, for the FP8 form, by VALU work.
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

// 8 outputs of one job: a = bf16(silu(g)), y = bf16(a * u).  Returns the 8
// bf16 results as 4 packed words.
__device__ __forceinline__ u32x4 swiglu8(u32x4 gv, u32x4 uv)
{
    uint32_t gb[8];
    float g[8], s[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        gb[2 * e] = gv[e] << 16;
        gb[2 * e + 1] = gv[e] & 0xFFFF0000u;
        g[2 * e] = __uint_as_float(gb[2 * e]);
        g[2 * e + 1] = __uint_as_float(gb[2 * e + 1]);
    }
    // running extrema: smallest knife-edge key of the results, largest gate
    // bit pattern (above SILU_FAST_MIN_BITS means g < -16)
    uint32_t kmin = 0xFFFFFFFFu, gmax = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        s[j] = silu_fast(g[j]);
        kmin = min(kmin, silu_edge_key(s[j]));
        gmax = max(gmax, gb[j]);
    }
    if (kmin <= SILU_EDGE_KEY_MAX || gmax > SILU_FAST_MIN_BITS) {
        // recompute this lane's flagged elements exactly, one at a time
        uint32_t redo = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            redo |= (uint32_t)((silu_edge_key(s[j]) <= SILU_EDGE_KEY_MAX) |
                               (gb[j] > SILU_FAST_MIN_BITS)) << j;
        while (redo) {
            const int j = __builtin_ctz(redo);
            redo &= redo - 1u;
            float gj = g[0];
#pragma unroll
            for (int t = 1; t < 8; ++t) gj = (j == t) ? g[t] : gj;
            const float r = silu_exact(gj);
#pragma unroll
            for (int t = 0; t < 8; ++t) s[t] = (j == t) ? r : s[t];
        }
    }
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t a = pack_bf16(s[2 * e], s[2 * e + 1]);
        y[e] = pack_bf16(bf_lo(a) * bf_lo(uv[e]), bf_hi(a) * bf_hi(uv[e]));
    }
    return y;
}

// MODE 0: bf16 output; 1: E4M3 output, fast quotient; 2: E4M3, IEEE division.
template <int U, int MODE>
__device__ __forceinline__ void swiglu_loop(const SwigluParams &p, const E4m3Scale &qs)
{
    const uint16_t *gu = (const uint16_t *)p.gate_up;
    const uint64_t stride = (uint64_t)gridDim.x * 256u * U;
    for (uint64_t base = (uint64_t)blockIdx.x * 256u * U + threadIdx.x; base < p.jobs;
         base += stride) {
        u32x4 gv[U], uv[U];
        uint64_t job[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            job[u] = base + (uint64_t)u * 256u;
            const bool ok = job[u] < p.jobs;
            const uint64_t i = ok ? job[u] : 0;
            // row = i / (N/8): a binary64 estimate is the row or one below it
            uint64_t row = (uint64_t)((double)i * p.inv_vecs_per_row);
            if (i - row * p.vecs_per_row >= p.vecs_per_row) ++row;
            const uint16_t *g = gu + i * 8u + row * (uint64_t)p.inter;
            gv[u] = ok ? *(const u32x4 *)g : (u32x4)0u;
            uv[u] = ok ? *(const u32x4 *)(g + p.inter) : (u32x4)0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (job[u] >= p.jobs) continue;
            const u32x4 y = swiglu8(gv[u], uv[u]);
            if constexpr (MODE == 0) {
                *((u32x4 *)p.out + job[u]) = y;
            } else {
                float z[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[2 * e] = e4m3_quotient<MODE == 1>(bf_lo(y[e]), qs);
                    z[2 * e + 1] = e4m3_quotient<MODE == 1>(bf_hi(y[e]), qs);
                }
                u32x2 q;
                q[0] = pack_e4m3x4(z[0], z[1], z[2], z[3]);
                q[1] = pack_e4m3x4(z[4], z[5], z[6], z[7]);
                *((u32x2 *)p.out + job[u]) = q;
            }
        }
    }
}

template <int U, bool QUANT>
__global__ void __launch_bounds__(256) swiglu_kernel(SwigluParams p)
{
    if constexpr (QUANT) {
        const E4m3Scale qs = make_e4m3_scale(*p.scale);
        if (e4m3_scale_is_fast(qs))
            swiglu_loop<U, 1>(p, qs);
        else
            swiglu_loop<U, 2>(p, qs);
    } else {
        swiglu_loop<U, 0>(p, E4m3Scale{});
    }
}

// ---------------------------------------------------------------- variants

static const SwigluVariant kSwigluVariants[] = {
    {1, 0, "1 job/lane, one-shot grid"},
    {2, 0, "2 jobs/lane, one-shot grid"},
    {4, 0, "4 jobs/lane, one-shot grid"},
    {1, 8, "1 job/lane, 8 blocks/CU stride"},
    {2, 8, "2 jobs/lane, 8 blocks/CU stride"},
    {4, 8, "4 jobs/lane, 8 blocks/CU stride"},
    {2, 4, "2 jobs/lane, 4 blocks/CU stride"},
    {4, 4, "4 jobs/lane, 4 blocks/CU stride"},
};
constexpr int kNumSwigluVariants = sizeof(kSwigluVariants) / sizeof(kSwigluVariants[0]);

int swiglu_variant_count() { return kNumSwigluVariants; }
const SwigluVariant *swiglu_variant(int id)
{
    return (id >= 0 && id < kNumSwigluVariants) ? &kSwigluVariants[id] : nullptr;
}

template <int U, bool Q>
static hipError_t launch_one(const SwigluParams &p, int blocks_per_cu, int num_cus,
                             hipStream_t stream)
{
    const uint64_t per_block = 256u * (uint64_t)U;
    uint64_t blocks = (p.jobs + per_block - 1) / per_block;
    if (blocks_per_cu > 0) {
        const uint64_t cap = (uint64_t)num_cus * (uint64_t)blocks_per_cu;
        if (blocks > cap) blocks = cap;
    }
    SwigluParams copy = p;
    void *args[] = {&copy};
    return hipLaunchKernel((const void *)&swiglu_kernel<U, Q>, dim3((unsigned)blocks), dim3(256),
                           args, 0, stream);
}

template <bool Q>
static hipError_t dispatch(const SwigluParams &p, int variant, int num_cus, hipStream_t s)
{
    const SwigluVariant *v = swiglu_variant(variant);
    if (!v) return hipErrorInvalidValue;
    switch (v->jobs_per_lane) {
    case 1: return launch_one<1, Q>(p, v->blocks_per_cu, num_cus, s);
    case 2: return launch_one<2, Q>(p, v->blocks_per_cu, num_cus, s);
    case 4: return launch_one<4, Q>(p, v->blocks_per_cu, num_cus, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_swiglu(const SwigluParams &p, bool quant, int variant, int num_cus,
                         hipStream_t stream)
{
    return quant ? dispatch<true>(p, variant, num_cus, stream)
                 : dispatch<false>(p, variant, num_cus, stream);
}

}  // namespace aarms
