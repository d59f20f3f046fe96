// launch.h -- internal interface between the C ABI (capi.cpp) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace aarms {

// A dispatch counts its work-items per grid dimension in 32 bits.  The
// kernels of one block per row (or row quartet) are launched on a 1-D grid
// while it fits; past that, on rows of 2^LINEAR_GRID_SHIFT blocks (grid y =
// the number of such rows), and they number their blocks (blockIdx.y <<
// LINEAR_GRID_SHIFT) + blockIdx.x -- blockIdx.x itself on a 1-D grid.  With
// at most 1,024 threads a block, 2^21 blocks are 2^31 work-items.
constexpr int LINEAR_GRID_SHIFT = 21;

inline dim3 linear_grid(int64_t blocks, int threads)
{
    if ((uint64_t)blocks * (uint64_t)threads <= 0xFFFFFFFFull) return dim3((unsigned)blocks);
    const int64_t x = (int64_t)1 << LINEAR_GRID_SHIFT;
    return dim3((unsigned)x, (unsigned)((blocks + x - 1) / x));
}

// Norm epilogues.
enum NormEpilogue : int {
    NORM_EPI_BF16 = 0,        // bf16 out
    NORM_EPI_FP8_DYNAMIC = 1, // E4M3 out, per-token scale written to scale_out
    NORM_EPI_FP8_STATIC = 2,  // E4M3 out, per-tensor scale read from scale_in
    NORM_EPI_MXFP4 = 3,       // MXFP4 out: E2M1 codes, E8M0 scale per 32 values to scale_out
    NORM_EPI_NVFP4 = 4,       // NVFP4 out: E2M1 codes, E4M3 scale per 16 values to scale_out,
                              // fp32 tensor scale from scale_in
    NORM_EPI_FP8_GROUP = 5,   // E4M3 out, fp32 scale per 128 values to scale_out [T, H/128]
};

// Values per scale of the per-group (block) E4M3 forms: the slices of 16
// adjacent lanes (one DPP row).
constexpr int FP8_GROUP = 128;

struct NormParams {
    void *out;               // bf16 [T,H], or fp8 [T,H] when quantising
    void *residual_out;      // bf16 [T,H] (with the residual add), else null
    const void *x;           // bf16 [T,H]
    const void *residual;    // bf16 [T,H] (with the residual add), else null
    const void *weight;      // bf16 [H]
    float *scale_out;        // fp32 [T], dynamic FP8 only; uint8 [T, H/32] for MXFP4
    const float *scale_in;   // fp32 [1], static FP8 only
    int64_t tokens;
    int32_t hidden;
    float eps;
    double inv_hidden;       // binary64(1 / hidden), correctly rounded
    // Store hold of the one-shot kernel, in ticks of the 100 MHz real-time
    // clock: a row's stores wait until this long after its wave started (0:
    // none).  At most NORM_HOLD_MAX_TICKS.
    uint32_t hold_ticks;
    // Quantised forms with the residual add: store the updated residual after
    // the output rather than right after the add (1), if the launch turns out
    // to be one generation of blocks (the launcher clears it otherwise).
    uint32_t res_last;
#ifdef AARMS_PHASE_STAMPS
    // Measurement build only (libaarms_stamps.so): per wave of each row,
    // 16 slots of real-time-clock stamps at the phases of norm_kernel;
    // stamp_detail: also the sub-steps of the chain after the first barrier.
    uint64_t *stamps;
    uint32_t stamp_detail;
#endif
};

constexpr uint32_t NORM_HOLD_MAX_TICKS = 2000;   // 20 us

// SwiGLU epilogues (the per-token FP8 form has its own row kernel).
enum SwigluEpilogue : int {
    SWIGLU_EPI_BF16 = 0,
    SWIGLU_EPI_FP8 = 1,       // static per-tensor E4M3, scale read from scale
    SWIGLU_EPI_MXFP4 = 2,     // E2M1 codes, E8M0 scale per 32 outputs to scale_out
    SWIGLU_EPI_NVFP4 = 3,     // E2M1 codes, E4M3 scale per 16 outputs to scale_out, tensor
                              // scale from scale
    SWIGLU_EPI_FP8_GROUP = 4, // E4M3 codes, fp32 scale per 128 outputs to scale_out [T, N/128]
};

struct SwigluParams {
    void *out;               // bf16 [T,N], or fp8 [T,N] when quantising
    const void *gate_up;     // bf16 [T,2N]
    const float *scale;      // fp32 [1], static FP8 only
    float *scale_out;        // fp32 [T], per-token FP8; uint8 [T, N/32] for MXFP4
    int64_t tokens;          // T
    int64_t inter;           // N
    uint32_t vecs_per_row;   // N / 8: one job = 8 adjacent outputs of a row
    // Flat grid only: floor(n / jobs per row) for 32-bit n as
    // (t + ((n - t) >> div_shift1)) >> div_shift2 with t = mulhi(n, div_magic)
    uint32_t div_magic, div_shift1, div_shift2;
};

// Rows per launch along grid y; more rows go to grid z.
constexpr uint32_t SWIGLU_ROWS_PER_Y = 65535;

// Norm variants: (waves per row, 16-byte vectors per lane).  A row of H
// elements needs waves * 64 * vectors * 8 >= H.
struct NormVariant {
    int waves_per_row;
    int vecs_per_lane;
    int blocks_per_cu;       // 0: one block per row (or row quartet); > 0: a persistent,
                             // software-pipelined grid of this many blocks per CU; < 0: a
                             // resident-row kernel (norm_resident.hip), NORM_RESIDENT_*
    const char *name;
};

// Resident-row kernels: one wave holds a row of up to 16,384 values in its
// registers (rows a multiple of 512 wide).  NORM_RESIDENT_Y_IN_PLACE: a
// 6-slice load window, and the per-token E4M3 form overwrites h with y in its
// amax pass; NORM_RESIDENT: a 10-slice window.
constexpr int NORM_RESIDENT_Y_IN_PLACE = -1;
constexpr int NORM_RESIDENT = -2;
constexpr int NORM_RESIDENT_MAX_HIDDEN = 16384;
constexpr int NORM_RESIDENT_WIDTH_MULTIPLE = 512;

struct SwigluVariant {
    int jobs_per_lane;       // a block of 256 lanes covers 256 * jobs_per_lane jobs of one row
    int job_outputs;         // outputs per job: 8 (16-byte loads) or 4 (8-byte loads)
    int flat;                // 1: blocks of 256 jobs over the rows laid end to end (one 8-output
                             // job per lane; rows of at least 256 jobs, under 2^32 jobs per launch)
    const char *name;
};

// Per-token FP8 SwiGLU variants: (waves per row, 8-output jobs per lane).
// A row of N outputs needs waves * 64 * jobs * 8 >= N.
struct SwigluRowVariant {
    int waves_per_row;
    int jobs_per_lane;
    const char *name;
};

int norm_variant_count();
const NormVariant *norm_variant(int id);
int swiglu_variant_count();
const SwigluVariant *swiglu_variant(int id);

hipError_t launch_norm(const NormParams &p, int epi, bool residual, int variant, int num_cus,
                       hipStream_t stream);
hipError_t launch_norm_resident(const NormParams &p, int epi, bool residual, int kind, hipStream_t stream);
int swiglu_row_variant_count();
const SwigluRowVariant *swiglu_row_variant(int id);
hipError_t launch_swiglu(const SwigluParams &p, int epi, int variant, hipStream_t stream);
hipError_t launch_swiglu_rowq(const SwigluParams &p, int variant, hipStream_t stream);

}  // namespace aarms
