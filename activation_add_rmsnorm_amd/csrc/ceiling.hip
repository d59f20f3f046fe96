// ceiling.hip -- a plain streaming kernel that moves the same bytes as one
// launch of a library kernel, for measurement only (libaarms_ceiling.so; the
// library itself does not use it).
//
// Two inputs of n 16-byte vectors are read and up to two outputs are written,
// out0_bytes and out1_bytes (0, 4, 8 or 16) per input vector, with the same
// streaming hints as the library kernels, one vector of each input per lane
// and the flattest possible grid.  Its time on the same buffers is the
// bandwidth a launch of that size and read/write mix can reach on the device,
// which separates a kernel's own losses from the fixed cost of a launch and
// from the read/write turnaround of HBM.
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

}  // namespace

// Returns 0 on success, -1 for bad arguments (nothing launched), or the HIP
// error code of the launch.  n is at most (2^31 - 1) * 256 vectors; out0_bytes is
// 4, 8 or 16, out1_bytes 0, 4, 8 or 16; inputs and 16-byte outputs 16-byte
// aligned, 8- and 4-byte outputs aligned to their size.  Buffers are the
// caller's.
extern "C" __attribute__((visibility("default"))) int aarms_stream_ceiling(void *out0, int out0_bytes, void *out1, int out1_bytes,
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
