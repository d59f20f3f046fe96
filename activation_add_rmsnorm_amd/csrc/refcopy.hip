// refcopy.hip -- a plain streaming copy that moves the same bytes as one
// launch of a library kernel, for measurement only (libaarms_refcopy.so; the
// library itself does not use it).
//
// Two inputs of n 16-byte vectors are read and up to two outputs are written,
// out0_bytes and out1_bytes (0, 4, 8 or 16) per input vector, with the same
// streaming hints as the library kernels, one vector of each input per lane
// and the flattest possible grid.  Its time on the same buffers is a
// reference for a launch of that size and read/write mix: what the simplest
// stream reaches on the device.  It is not a bound (kernels that issue their
// accesses differently can beat it); the bound is the HBM peak.
//
//   fused_add_rmsnorm [T, H]:           in = x, residual; out0 = 16 (updated
//                                       residual), out1 = 16 (bf16 out)
//   fused_add_rmsnorm_quant_fp8 [T, H]: out0 = 16, out1 = 8 (E4M3 out)
//   swiglu [T, 2N] -> [T, N]:           in = the two halves of gate_up;
//                                       out0 = 16 (bf16) or 8 (E4M3)
//   fused_add_rmsnorm_quant_mxfp4:      out0 = 16, out1 = 4 (E2M1 pairs; the
//                                       E8M0 bytes, 1/32 of the data, left out)
//   swiglu_quant_mxfp4:                 out0 = 4
// (the weight and the scales, a few KB, are left out).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int O>
__device__ __forceinline__ void put(void *base, uint64_t i, u32x4 v)
{
    if constexpr (O == 16) __builtin_nontemporal_store(v, (u32x4 *)base + i);
    if constexpr (O == 8) __builtin_nontemporal_store((u32x2){v.x ^ v.z, v.y ^ v.w}, (u32x2 *)base + i);
    if constexpr (O == 4) __builtin_nontemporal_store(v.x ^ v.y ^ v.z ^ v.w, (uint32_t *)base + i);
}

template <int O0, int O1>
__global__ void __launch_bounds__(256)
stream_kernel(const u32x4 *__restrict__ in0, const u32x4 *__restrict__ in1, void *__restrict__ out0,
              void *__restrict__ out1, uint64_t n)
{
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    const u32x4 a = __builtin_nontemporal_load(in0 + i);
    const u32x4 b = __builtin_nontemporal_load(in1 + i);
    put<O0>(out0, i, a ^ b);
    put<O1>(out1, i, a + b);
}

template <int O0, int O1>
hipError_t launch(const void *in0, const void *in1, void *out0, void *out1, uint64_t n, hipStream_t s)
{
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL((stream_kernel<O0, O1>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const u32x4 *)in0, (const u32x4 *)in1, out0, out1, n);
    return hipGetLastError();
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Copy designs, for a sweep of how a plain stream of a given read/write mix
// is best issued on this device.  Per vector index i: KIND 0 reads in0[i]
// and in1[i] and writes one 16-byte vector (the SwiGLU mix), KIND 1 two (the
// bf16 norm mix), KIND 2 one 16-byte and one 8-byte vector (the E4M3 norm
// mix), KIND 6 one 8-byte vector (the E4M3 SwiGLU mix); KIND 3 only reads
// in0[i] and in1[i] (its store is guarded by a test no data passes in
// practice, so the loads are not dead), KIND 4 only writes out0[i], KIND 5
// reads in0[i] and writes out0[i].  U vectors per lane; NT = streaming
// hints; the grid is either one-shot (one block per 256 U vectors) or
// smaller, with a grid-stride loop.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void st(T *p, T v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <int KIND, int U, bool NT>
__global__ void __launch_bounds__(256)
copy_design_kernel(const u32x4 *__restrict__ in0, const u32x4 *__restrict__ in1, u32x4 *__restrict__ out0,
                   void *__restrict__ out1, uint64_t n)
{
    const uint64_t stride = (uint64_t)gridDim.x * 256u * U;
    for (uint64_t base = (uint64_t)blockIdx.x * 256u * U + threadIdx.x; base < n; base += stride) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * 256u;
            a[u] = b[u] = (u32x4)0u;
            if (i < n) {
                if constexpr (KIND != 4) a[u] = ld<NT>(in0 + i);
                if constexpr (KIND != 4 && KIND != 5) b[u] = ld<NT>(in1 + i);
            }
        }
        if constexpr (KIND == 3) {
            u32x4 acc = (u32x4)0u;
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= a[u] + b[u];
            if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0x85EBCA6Bu && acc.w == 0xC2B2AE35u &&
                base < n)
                st<NT>(out0 + base, acc);
            continue;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * 256u;
            if (i >= n) continue;
            if constexpr (KIND == 4) {
                st<NT>(out0 + i, (u32x4)(uint32_t)i);
            } else if constexpr (KIND == 6) {
                st<NT>((u32x2 *)out0 + i, (u32x2){a[u].x ^ b[u].z, a[u].y ^ b[u].w});
            } else {
                st<NT>(out0 + i, a[u] ^ b[u]);
                if constexpr (KIND == 1) st<NT>((u32x4 *)out1 + i, a[u] + b[u]);
                if constexpr (KIND == 2) st<NT>((u32x2 *)out1 + i, (u32x2){a[u].x ^ b[u].z, a[u].y ^ b[u].w});
            }
        }
    }
}

template <int KIND, int U, bool NT>
hipError_t launch_design(const void *in0, const void *in1, void *out0, void *out1, uint64_t n, uint64_t grid,
                         hipStream_t s)
{
    hipLaunchKernelGGL((copy_design_kernel<KIND, U, NT>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const u32x4 *)in0, (const u32x4 *)in1, (u32x4 *)out0, out1, n);
    return hipGetLastError();
}

template <int KIND, bool NT>
hipError_t design_u(int u, const void *in0, const void *in1, void *out0, void *out1, uint64_t n, uint64_t grid,
                    hipStream_t s)
{
    if (u == 1) return launch_design<KIND, 1, NT>(in0, in1, out0, out1, n, grid, s);
    if (u == 2) return launch_design<KIND, 2, NT>(in0, in1, out0, out1, n, grid, s);
    return launch_design<KIND, 4, NT>(in0, in1, out0, out1, n, grid, s);
}

// A copy in the one-wave-per-row layout of the norm's store hold: rows of
// V * 64 16-byte vectors, four rows (waves) per 256-thread block, every lane
// loading its V vectors of each input, then waiting until hold_ticks of the
// 100 MHz real-time clock have passed since the wave started (bounded; 0: no
// wait), then writing out0 = a ^ b and out1 = a + b.  All of a launch's rows
// are resident at once for the sizes it is used at.
template <int V>
__global__ void __launch_bounds__(256) held_copy_kernel(const u32x4 *__restrict__ in0, const u32x4 *__restrict__ in1,
                                                        u32x4 *__restrict__ out0, u32x4 *__restrict__ out1,
                                                        uint64_t rows, uint32_t hold_ticks)
{
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t row = (uint64_t)blockIdx.x * 4u + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint64_t base = row * (uint64_t)(V * 64) + (threadIdx.x & 63u);
    u32x4 a[V], b[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        a[v] = __builtin_nontemporal_load(in0 + base + v * 64);
        b[v] = __builtin_nontemporal_load(in1 + base + v * 64);
    }
    if (hold_ticks) {
        asm volatile("" : : "v"(a[0]), "v"(b[V - 1]));
        while (true) {
            const uint64_t now = __builtin_amdgcn_s_memrealtime();
            if (now < t0 || now - t0 >= hold_ticks) break;
            __builtin_amdgcn_s_sleep(2);
        }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
        __builtin_nontemporal_store(a[v] ^ b[v], out0 + base + v * 64);
        __builtin_nontemporal_store(a[v] + b[v], out1 + base + v * 64);
    }
}

}  // namespace

// Returns 0 on success, -1 for bad arguments (nothing launched), or the HIP
// error code of the launch.  n is at most (2^31 - 1) * 256 vectors; out0_bytes is
// 4, 8 or 16, out1_bytes 0, 4, 8 or 16; inputs and 16-byte outputs 16-byte
// aligned, 8- and 4-byte outputs aligned to their size.  Buffers are the
// caller's.
extern "C" __attribute__((visibility("default"))) int aarms_reference_copy(void *out0, int out0_bytes, void *out1, int out1_bytes,
                                    const void *in0, const void *in1, int64_t n, hipStream_t stream)
{
    if (n < 0 || (uint64_t)n > (uint64_t)INT32_MAX * 256u) return -1;
    if (n == 0) return 0;
    if (!in0 || !in1 || !out0 || (out1_bytes && !out1)) return -1;
    if (!aligned(in0, 16) || !aligned(in1, 16) || out0_bytes <= 0 || !aligned(out0, (uintptr_t)out0_bytes))
        return -1;
    if (out1_bytes && !aligned(out1, (uintptr_t)out1_bytes)) return -1;
    const uint64_t m = (uint64_t)n;
    hipError_t e;
    if (out0_bytes == 16 && out1_bytes == 16) e = launch<16, 16>(in0, in1, out0, out1, m, stream);
    else if (out0_bytes == 16 && out1_bytes == 8) e = launch<16, 8>(in0, in1, out0, out1, m, stream);
    else if (out0_bytes == 16 && out1_bytes == 4) e = launch<16, 4>(in0, in1, out0, out1, m, stream);
    else if (out0_bytes == 16 && out1_bytes == 0) e = launch<16, 0>(in0, in1, out0, out1, m, stream);
    else if (out0_bytes == 8 && out1_bytes == 0) e = launch<8, 0>(in0, in1, out0, out1, m, stream);
    else if (out0_bytes == 4 && out1_bytes == 0) e = launch<4, 0>(in0, in1, out0, out1, m, stream);
    else return -1;
    return (int)e;
}

// One launch of a copy design (see copy_design_kernel): kind 0 to 6;
// vecs_per_lane 1, 2 or 4; nt 0 or 1; grid_blocks 0 for the one-shot grid,
// else that many 256-lane blocks looping over the data.  n 16-byte vectors
// per input; out0 holds n 16-byte vectors (n 8-byte ones for kind 6), out1
// n 16-byte (kind 1) or 8-byte (kind 2) vectors and is ignored otherwise;
// in1 is ignored by kinds 4 and 5, in0 by kind 4 (they may then be null).
// Returns 0, -1 for bad arguments (nothing launched), or the HIP error.
extern "C" __attribute__((visibility("default"))) int aarms_copy_design(int kind, int vecs_per_lane, int nt,
                                                                       int64_t grid_blocks, void *out0, void *out1,
                                                                       const void *in0, const void *in1, int64_t n,
                                                                       hipStream_t stream)
{
    if (kind < 0 || kind > 6 || (vecs_per_lane != 1 && vecs_per_lane != 2 && vecs_per_lane != 4) || n < 0 ||
        grid_blocks < 0)
        return -1;
    if (n == 0) return 0;
    const bool reads0 = kind != 4, reads1 = kind != 4 && kind != 5, has_out1 = kind == 1 || kind == 2;
    if ((reads0 && (!in0 || !aligned(in0, 16))) || (reads1 && (!in1 || !aligned(in1, 16))) || !out0 ||
        !aligned(out0, kind == 6 ? 8 : 16) || (has_out1 && (!out1 || !aligned(out1, kind == 1 ? 16 : 8))))
        return -1;
    const uint64_t m = (uint64_t)n;
    const uint64_t per_block = 256u * (uint64_t)vecs_per_lane;
    uint64_t grid = (m + per_block - 1) / per_block;
    if (grid_blocks > 0 && (uint64_t)grid_blocks < grid) grid = (uint64_t)grid_blocks;
    if (grid > (uint64_t)INT32_MAX) return -1;
#define AARMS_DESIGN_KIND(K)                                                                     \
    if (kind == K)                                                                               \
        return (int)(nt ? design_u<K, true>(vecs_per_lane, in0, in1, out0, out1, m, grid, stream) \
                        : design_u<K, false>(vecs_per_lane, in0, in1, out0, out1, m, grid, stream));
    AARMS_DESIGN_KIND(0)
    AARMS_DESIGN_KIND(1)
    AARMS_DESIGN_KIND(2)
    AARMS_DESIGN_KIND(3)
    AARMS_DESIGN_KIND(4)
    AARMS_DESIGN_KIND(5)
    AARMS_DESIGN_KIND(6)
#undef AARMS_DESIGN_KIND
    return -1;
}

// The held copy (held_copy_kernel): rows of row_vecs 16-byte vectors (64,
// 128, 192 or 256) in each of in0, in1, out0 and out1 (16-byte aligned),
// hold_ticks at most 4,000 (40 us).  Returns 0, -1 for bad arguments
// (nothing launched), or the HIP error.
extern "C" __attribute__((visibility("default"))) int aarms_copy_held(int64_t rows, int row_vecs, int hold_ticks,
                                                                     void *out0, void *out1, const void *in0,
                                                                     const void *in1, hipStream_t stream)
{
    if (rows < 0 || rows > (int64_t)INT32_MAX * 4 || hold_ticks < 0 || hold_ticks > 4000) return -1;
    if (row_vecs != 64 && row_vecs != 128 && row_vecs != 192 && row_vecs != 256) return -1;
    if (rows == 0) return 0;
    if (!in0 || !in1 || !out0 || !out1 || !aligned(in0, 16) || !aligned(in1, 16) || !aligned(out0, 16) ||
        !aligned(out1, 16))
        return -1;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const u32x4 *a = (const u32x4 *)in0, *b = (const u32x4 *)in1;
    u32x4 *o0 = (u32x4 *)out0, *o1 = (u32x4 *)out1;
    const uint64_t r = (uint64_t)rows;
    const uint32_t h = (uint32_t)hold_ticks;
    switch (row_vecs / 64) {
    case 1: hipLaunchKernelGGL(held_copy_kernel<1>, grid, block, 0, stream, a, b, o0, o1, r, h); break;
    case 2: hipLaunchKernelGGL(held_copy_kernel<2>, grid, block, 0, stream, a, b, o0, o1, r, h); break;
    case 3: hipLaunchKernelGGL(held_copy_kernel<3>, grid, block, 0, stream, a, b, o0, o1, r, h); break;
    default: hipLaunchKernelGGL(held_copy_kernel<4>, grid, block, 0, stream, a, b, o0, o1, r, h); break;
    }
    return (int)hipGetLastError();
}
