// capi.cpp -- the extern "C" entry points of libaarms.so (include/aarms.h):
// argument validation, variant choice and kernel launch.  Validation runs
// entirely on the host before any HIP call, so every error path can be
// exercised without a GPU.

#include "aarms.h"
#include "launch.h"

#include <atomic>
#include <cmath>
#include <cstdint>

using namespace aarms;

#ifdef AARMS_PHASE_STAMPS
// Measurement build only (libaarms_stamps.so): where the one-shot norm kernel
// writes its phase stamps (16 uint64 per wave of each row; null: none).
static uint64_t *g_phase_stamps = nullptr;
static uint32_t g_stamp_detail = 0;
extern "C" __attribute__((visibility("default"))) void aarms_set_phase_stamps(void *stamps)
{
    g_phase_stamps = (uint64_t *)stamps;
}
// detail != 0: also stamp the sub-steps after the first barrier (more stores
// and waits in the stamped kernel, so a separate pass)
extern "C" __attribute__((visibility("default"))) void aarms_set_phase_stamp_detail(int detail)
{
    g_stamp_detail = detail ? 1u : 0u;
}
#endif

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void *p, uint64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }
bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Row-width checks shared by all ops.
static_assert(FP8_GROUP == AARMS_FP8_GROUP, "the kernels' group is the header's");

int check_width(int64_t tokens, int64_t width, int64_t max_width)
{
    if (tokens < 0 || width <= 0 || width % 8 != 0) return AARMS_ERR_BAD_SHAPE;
    if (max_width > 0 && width > max_width) return AARMS_ERR_UNSUPPORTED_SHAPE;
    if (tokens > 0 && width > AARMS_MAX_ELEMENTS / tokens) return AARMS_ERR_UNSUPPORTED_SHAPE;
    if (tokens > AARMS_MAX_TOKENS) return AARMS_ERR_UNSUPPORTED_SHAPE;
    return AARMS_OK;
}

int check_eps(float eps)
{
    return (std::isfinite(eps) && eps >= 0.0f) ? AARMS_OK : AARMS_ERR_BAD_EPS;
}

// An output must not overlap any other argument, except when it is exactly
// the named in-place partner.
struct Arg {
    Range r;
    const void *ptr;
};

int check_outputs(const Arg *outs, const int *partner, int n_out, const Arg *ins, int n_in)
{
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_out; ++j)
            if (i != j && overlap(outs[i].r, outs[j].r)) return AARMS_ERR_ALIAS;
        for (int j = 0; j < n_in; ++j) {
            if (!overlap(outs[i].r, ins[j].r)) continue;
            const bool in_place = partner[i] == j && outs[i].ptr == ins[j].ptr &&
                                  outs[i].r.hi == ins[j].r.hi;
            if (!in_place) return AARMS_ERR_ALIAS;
        }
    }
    return AARMS_OK;
}

// Compute units of the current device, cached per device (the grid of the
// persistent variants is sized from it).
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int norm_capacity(const NormVariant *v) { return v->waves_per_row * 64 * v->vecs_per_lane * 8; }

// Whether variant v runs rows of `hidden` values: wide enough, and for the
// resident-row kernels a width that is a multiple of 512 (whole 64-slice
// chunks of the row, which the weight's LDS transfer moves per wave).
bool norm_fits(const NormVariant *v, int64_t hidden)
{
    if (!v || hidden <= 0 || norm_capacity(v) < hidden) return false;
    return v->blocks_per_cu >= 0 || hidden % NORM_RESIDENT_WIDTH_MULTIPLE == 0;
}

// One-shot variant with `waves` waves per row that fits the row with the
// fewest vectors per lane, if that is at most max_vecs; else -1.
static int norm_fit(int waves, int64_t hidden, int max_vecs)
{
    int best = -1;
    for (int i = 0; i < norm_variant_count(); ++i) {
        const NormVariant *v = norm_variant(i);
        if (v->blocks_per_cu != 0 || v->waves_per_row != waves || norm_capacity(v) < hidden) continue;
        if (v->vecs_per_lane > max_vecs) continue;
        if (best < 0 || v->vecs_per_lane < norm_variant(best)->vecs_per_lane) best = i;
    }
    return best;
}

// The variant with exactly these parameters, or -1.
static int norm_find(int waves, int vecs, int blocks_per_cu)
{
    for (int i = 0; i < norm_variant_count(); ++i) {
        const NormVariant *v = norm_variant(i);
        if (v->waves_per_row == waves && v->vecs_per_lane == vecs && v->blocks_per_cu == blocks_per_cu) return i;
    }
    return -1;
}

// Below this many rows a narrow-row launch is latency-bound (a few waves per
// CU at most) and splitting each row over four waves shortens every row's
// dependent chain of loads and reductions; from here on one wave per row
// wins (measured on MI355X, 256 CUs, rows of 1,536).
constexpr int64_t kNarrowMultiWaveTokens = 1024;
// With the residual add, four waves per row stay ahead longer: one wave per
// row holds at most two rows per SIMD there.  Timed by graph replay, four
// waves of one vector beat one wave per row for bf16 by 2-5% at 1,024-1,280
// tokens of 1,024, by 5-21% at 1,024-2,047 tokens of 1,536 and by 4-15% at
// 1,024-1,792 tokens of 2,048 (one wave per row ahead again from 1,536
// tokens of 1,024); for the per-tensor E4M3, MXFP4, NVFP4 and per-group
// E4M3 forms by 4-32% at 1,024-1,536 tokens of 1,536 and 2,048, and at
// 1,792 tokens of 2,048 (2-11%).  On rows of 1,537-2,048 (four vectors per
// lane in one wave) one wave per row is ahead again at 2,047 tokens (up to
// 10%), on rows of 1,025-1,536 from 2,048.  Per-token E4M3 (two row
// reductions) was not consistently faster either way, and on rows of 1,024
// the quantised forms were within a few percent: those keep
// kNarrowMultiWaveTokens.
constexpr int64_t kNarrowMultiWaveTokensAdd = 2048, kNarrowMultiWaveTokensAdd2048 = 1800,
                  kNarrowMultiWaveTokensAdd1024 = 1536;

// Per-token E4M3 with the residual add reduces each row twice (sum of
// squares, then amax), so the cost of a cross-wave barrier weighs more: for
// rows wider than 8,192 in batches up to 1,024 tokens, 8 waves of 4 vectors
// per lane beat 16 waves of 2 (1.5-7% at 1 to 1,024 tokens of 12,288 and
// 16,384; from 2,048 tokens 16 x 2 is as fast or faster).  The block-scaled
// forms, with one reduction, keep 16 x 2.
constexpr int64_t kDynamicFp8FewWavesTokens = 1024;
constexpr int64_t kWideOneVecTokensBf16 = 512, kWideOneVecTokensFp8 = 64;
constexpr int64_t kNoAddOneWaveMaxTokensBf16 = 3072, kNoAddOneWaveMaxTokensFp8 = 4096;

// bf16 with the residual add on rows of 4,097-8,192: from 1,024 to 1,536
// tokens a one-shot grid of 8-wave blocks runs about 1-1.5 generations
// and leaves a partial one.  Fewer waves per row (fewer, longer-lived
// blocks) fit such a batch into one generation: timed by graph replay on
// three boxes at 5,120, 6,144 and 8,192 wide, 4 waves of 4 vectors were the
// fastest or within 3% at 1,024-1,280 tokens (up to 14% ahead of 8 x 2, and
// of the persistent, software-pipelined 8 x 2 variant chosen here before)
// and 2 waves of 8 the fastest at 1,536 (6-17% ahead).  Below 1,024 tokens
// the general rule's 8 x 2 is as fast or faster (6% at 768 x 5,120).
constexpr int64_t kWideFewWavesMinTokens = 1024, kWideFourWavesMaxTokens = 1280, kWideFewWavesMaxTokens = 1536;

// bf16 with the residual add on rows of 2,049-4,096 (4 waves of 2 vectors
// by default): batches of 2,049-2,560 tokens spill the 4-wave blocks into a
// thin second generation, and 2 waves of 4 vectors keep them in one: 3-9%
// faster at 2,049 tokens and 18-25% at 2,304-2,560 of 2,560-4,096 (graph
// replay, two boxes; from 3,072 tokens mixed).  Per-token E4M3 was within
// 3.6% either way there and keeps 4 x 2.
constexpr int64_t kMidTwoWavesMinTokens = 2049, kMidTwoWavesMaxTokens = 2560;

// Store hold of the one-shot kernel (norm.hip, hold_stores): each row's
// stores wait until about the time the launch's reads take after its wave
// started, so that HBM serves the reads of a launch whose blocks are all
// resident before its writes.  Measured on MI355X for the bf16 output with
// one wave per row: with the residual add 12-21% faster at 4,096-8,192
// rows of 896-2,048 (22-50 MB of reads), with the best hold
// near reads / 7-8 TB/s and falling off on both sides (a hold too short
// gains little, one too long adds its excess).  With the residual add,
// reads / 7.8 TB/s measured 1.3% and 1.5% faster than 7.4 TB/s at
// [4096, 1536] and [4096, 2048] and 0.3% slower at [8192, 1536]; without
// it no single rate wins (7.0 TB/s: 0.5% and 1.8% faster at 4,096 rows,
// 1.8% slower at [8192, 1536]), so that form keeps 7.4.  Without the residual add
// (rmsnorm) the gain starts at about 12 MB of reads (4-18% at 12.6-18.9 MB,
// 4,096-8,192 rows of 896-2,048).  No gain below 4,096 rows, below those
// read sizes (16.8 MB with the add at [4096, 1024]; 7-8 MB without) or
// with several waves per row.  The launcher drops the hold when the grid
// does not fit on the device at once.
constexpr int64_t kHoldMinTokens = 4096;
constexpr double kHoldMinReadBytesAdd = 20e6, kHoldMinReadBytesNoAdd = 12e6;
// read bytes served per 10 ns tick of the hold: 7.8 and 7.4 TB/s
constexpr double kHoldReadBytesPerTickAdd = 78000.0, kHoldReadBytesPerTickNoAdd = 74000.0;

// The quantised forms with the residual add store the updated residual in
// the epilogue (after the row reduction) rather than right after the add in
// launches of one generation of blocks from this many bytes of reads:
// measured 3-16% faster at [256, 16384], [512, 16384] and [1024, 4096] in
// every quantised form and 2-15% at [4096, 1536] (1% slower for per-token
// E4M3 there); neutral to 3% slower at 8 MB and below.  Keeping the residual
// live for the choice costs multi-generation launches 0-2.5% (0.6% faster
// for the Llama-405B per-token E4M3 norm).
constexpr double kResLastMinReadBytes = 12e6;

uint32_t norm_res_last(int64_t tokens, int64_t hidden, int epi, bool res)
{
    if (!res || epi == NORM_EPI_BF16) return 0;
    return (double)tokens * (double)hidden * 4.0 >= kResLastMinReadBytes ? 1u : 0u;
}

uint32_t norm_hold_ticks(int64_t tokens, int64_t hidden, int epi, bool res, const NormVariant *v)
{
    if (epi != NORM_EPI_BF16 || v->waves_per_row != 1 || v->blocks_per_cu != 0 || tokens < kHoldMinTokens)
        return 0;
    const double reads = (double)tokens * (double)hidden * (res ? 4.0 : 2.0);
    if (reads < (res ? kHoldMinReadBytesAdd : kHoldMinReadBytesNoAdd)) return 0;
    const double ticks = reads / (res ? kHoldReadBytesPerTickAdd : kHoldReadBytesPerTickNoAdd);
    return ticks > (double)NORM_HOLD_MAX_TICKS ? 0u : (uint32_t)(ticks + 0.5);
}

// epi: the output format (NORM_EPI_*); residual: with the add in front.
int pick_norm(int64_t tokens, int64_t hidden, int epi, bool residual)
{
    if (hidden <= 0 || hidden > AARMS_MAX_HIDDEN) return -1;
    // Resident rows (one wave holds the row, the batch one generation of
    // four-row blocks) on rows of 12,289-16,384 (multiples of 512) in batches
    // that fill 0.8-1 or 1.75-2 blocks per CU.  Measured on MI355X (256 CUs)
    // against the split rows, 16,384 wide: per-token E4M3 with the residual
    // add 3-11% faster at 832-1,024 tokens and 1.5-9% at 1,792-2,048; bf16
    // with the add 13-20% and 7-8.5%; per-tensor E4M3 with the add 15-17% and
    // 5-10%; bf16 without it 4-11% and 5-8%.  Between the bands the CUs that
    // hold two blocks set the pace and the split rows win (1,536 tokens: up
    // to 4% slower resident); NVFP4, MXFP4, per-group E4M3 and the quantised
    // forms without the add were as fast or faster split (their epilogues
    // need more instructions per byte than two waves per SIMD can hide).  In
    // the first band every form takes the 6-slice window; in the second the
    // forms with the add take 10 slices.
    // With the residual add the resident rows also pay on narrower rows
    // (graph replay, 832-2,048 tokens): on rows of 10,240-12,288 in both
    // bands, bf16 3-8%, per-token E4M3 2-13% and per-tensor E4M3 7-24%
    // faster than the split rows; on rows of 6,144-9,728 bf16 only, in the
    // second band (5-14%; in the first band and for the E4M3 forms the split
    // rows were as fast or faster).  On these rows the 6-slice window was
    // the faster or within 1.3% in both bands.
    const bool res_wide = hidden > 12288 && hidden <= NORM_RESIDENT_MAX_HIDDEN;
    const bool res_mid = residual && hidden >= 10240 && hidden <= 12288;
    const bool res_mid_bf16 = residual && epi == NORM_EPI_BF16 && hidden >= 6144 && hidden < 10240;
    if ((res_wide || res_mid || res_mid_bf16) && hidden % NORM_RESIDENT_WIDTH_MULTIPLE == 0 &&
        (epi == NORM_EPI_BF16 || (residual && (epi == NORM_EPI_FP8_DYNAMIC || epi == NORM_EPI_FP8_STATIC)))) {
        const int64_t blocks = (tokens + 3) / 4, cus = device_cus();
        const bool one = blocks * 5 >= cus * 4 && blocks <= cus;
        const bool two = blocks * 4 >= cus * 7 && blocks <= 2 * cus;
        if (res_mid_bf16 ? two : (one || two)) {
            const int i = norm_find(1, 32, (res_wide && two && residual) ? NORM_RESIDENT : NORM_RESIDENT_Y_IN_PLACE);
            if (i >= 0) return i;
        }
    }
    if (epi == NORM_EPI_BF16 && residual && hidden > 4096 && hidden <= 8192 &&
        tokens >= kWideFewWavesMinTokens && tokens <= kWideFewWavesMaxTokens) {
        const int i = tokens <= kWideFourWavesMaxTokens ? norm_find(4, 4, 0) : norm_find(2, 8, 0);
        if (i >= 0) return i;
    }
    // The same rows at 1.75-2 four-row blocks per CU (1,792-2,048 tokens on
    // 256 CUs): one wave per row makes the batch a single generation of two
    // waves per SIMD, as the resident rows do for wider rows.  Graph replay
    // on three boxes at 2,048 tokens of 2,560-4,096: 4-13% faster than 4 x 2
    // in bf16 and per-token E4M3 (0-5% at 1,792).
    if (residual && (epi == NORM_EPI_BF16 || epi == NORM_EPI_FP8_DYNAMIC) && hidden > 2048 && hidden <= 4096) {
        const int64_t blocks = (tokens + 3) / 4, cus = device_cus();
        if (blocks * 4 >= cus * 7 && blocks <= 2 * cus) {
            const int i = norm_fit(1, hidden, 8);
            if (i >= 0) return i;
        }
    }
    // Past that band, on rows of 2,049-3,072: one wave per row again.  At
    // 2,561-3,072 tokens (one generation of three waves per SIMD) 8 vectors
    // per lane, 1-15% faster than 4 x 2 by graph replay (6 vectors lost 4% at
    // 2,600 x 3,072); at four waves per SIMD (4,096 tokens on 256 CUs, where
    // the store hold applies) the fewest vectors that fit, whose registers
    // let the whole batch be resident: 11-20% faster (8 vectors do not fit).
    if (residual && epi == NORM_EPI_BF16 && hidden > 2048 && hidden <= 3072) {
        int i = -1;
        if (tokens > kMidTwoWavesMaxTokens && tokens <= 3072)
            i = norm_find(1, 8, 0);
        else if (tokens >= kHoldMinTokens && tokens <= 16 * device_cus())
            i = norm_fit(1, hidden, 8);
        if (i >= 0) return i;
    }
    if (residual && epi == NORM_EPI_BF16 && hidden > 2048 && hidden <= 4096 &&
        tokens >= kMidTwoWavesMinTokens && tokens <= kMidTwoWavesMaxTokens) {
        const int i = norm_find(2, 4, 0);
        if (i >= 0) return i;
    }
    // The same band without the residual add, on rows of 8,193-16,384 (8
    // waves of 4 vectors): the pipelined 8 x 4 grid measured 5-25% faster
    // from 512 to 2,048 tokens at 16,384 wide (bf16 only: the per-token E4M3
    // form is slower pipelined); the resident rows above take the batches
    // they fit better.
    if (epi == NORM_EPI_BF16 && !residual && hidden > 8192 && hidden <= 16384 && tokens >= 512 &&
        tokens <= 2048) {
        const int i = norm_find(8, 4, 2);
        if (i >= 0) return i;
    }
    // Without the residual, rows of 2,049-4,096 in batches under 1,024
    // tokens: 4 waves of 2 vectors per lane beat 2 waves of 4 by 9-18% (the
    // shorter per-lane chain matters while the launch is latency-bound);
    // from 1,024 tokens 2 x 4 is as fast or faster.
    // Without the residual add, rows of 2,049-4,096 once a batch fills the
    // device: one wave per row (6 or 8 vectors) keeps 1,792-3,072 tokens in
    // one generation of up to three waves per SIMD, and a batch of four per
    // SIMD (4,096 tokens on 256 CUs) both fits one generation and takes the
    // store hold.  Graph replay on two boxes: bf16 level at 1,792 tokens,
    // 6-23% faster than 2 x 4 at 2,048-3,072 and 15-28% at 4,096 (between
    // 3,072 and 4,096, without the hold, 1-9% slower: not taken); per-token
    // E4M3 on rows up to 3,072 wide 1-13% faster at 1,792-4,096 tokens
    // (mixed from 6,144, and at 3,584-4,096 wide).
    if (!residual && hidden > 2048 && tokens >= 1792) {
        const int64_t cus = device_cus();
        const bool bf16_band = epi == NORM_EPI_BF16 && hidden <= 4096 &&
                               (tokens <= kNoAddOneWaveMaxTokensBf16 ||
                                (tokens >= kHoldMinTokens && tokens <= 16 * cus));
        const bool fp8_band = epi == NORM_EPI_FP8_DYNAMIC && hidden <= 3072 && tokens <= kNoAddOneWaveMaxTokensFp8;
        if (bf16_band || fp8_band) {
            const int i = norm_fit(1, hidden, 8);
            if (i >= 0) return i;
        }
    }
    if (!residual && hidden > 2048 && hidden <= 4096 && tokens < kNarrowMultiWaveTokens) {
        const int i = norm_fit(4, hidden, 2);
        if (i >= 0) return i;
    }
    // Small batches with the residual add on rows of 2,049-8,192: one vector
    // per lane over twice the waves (8 up to 4,096 wide, else 16) shortens
    // every row's chain while the launch is latency-bound.  Graph replay:
    // bf16 5-10% faster at 1-64 tokens and 2.4-3.9% at 512 (level at 512 x
    // 8,192); per-token E4M3 3.5-5.4% at 1-64 tokens of 3,072-4,096 (level
    // at 512, and at any batch from 5,120 wide, where its two row
    // reductions favour fewer waves).
    if (residual && hidden > 2048 && hidden <= 8192 &&
        ((epi == NORM_EPI_BF16 && tokens <= kWideOneVecTokensBf16) ||
         (epi == NORM_EPI_FP8_DYNAMIC && hidden <= 4096 && tokens <= kWideOneVecTokensFp8))) {
        const int i = norm_find(hidden <= 4096 ? 8 : 16, 1, 0);
        if (i >= 0) return i;
    }
    if (epi == NORM_EPI_FP8_DYNAMIC && residual && hidden > 8192 && tokens <= kDynamicFp8FewWavesTokens) {
        const int i = norm_fit(8, hidden, 4);
        if (i >= 0) return i;
    }
    // Narrow rows (up to 4 vectors per lane, 2,048 wide): one wave per row
    // with as few vectors per lane as fit (four waves per row for small
    // batches).  Wider rows: the fewest waves per row that fit with at most
    // 2 vectors per lane (the row's loads spread over many short slices, few
    // registers per wave), else 4, else 8; at 4,096 wide four waves of 2
    // vectors beat one wave of 8 (146 registers) by 4-18% from 1,024 tokens
    // up, every epilogue.  Without the residual a slice holds half the data,
    // and 4 vectors per lane (half the waves per row, twice the rows in
    // flight) come first.
    if (hidden <= 2048) {
        int64_t multi = kNarrowMultiWaveTokens;
        if (residual && epi != NORM_EPI_FP8_DYNAMIC && hidden > 1024)
            multi = hidden > 1536 ? kNarrowMultiWaveTokensAdd2048 : kNarrowMultiWaveTokensAdd;
        else if (residual && epi == NORM_EPI_BF16)
            multi = kNarrowMultiWaveTokensAdd1024;
        const int i = norm_fit(tokens < multi ? 4 : 1, hidden, 4);
        if (i >= 0) return i;
    }
    for (int max_vecs : {residual ? 2 : 4, 4, 8})
        for (int w : {2, 4, 8, 16}) {
            const int i = norm_fit(w, hidden, max_vecs);
            if (i >= 0) return i;
        }
    return -1;
}

// Launch-bound below about two million outputs (a decode batch): half jobs
// (4 outputs per lane) halve every lane's dependent chain of loads and SiLU
// arithmetic.  Measured on MI355X over T x 8,960 and T x 28,672.
constexpr int64_t kSwigluHalfJobOutputs = (int64_t)1 << 21;
constexpr int64_t kSwigluFp8TwoJobOutputs = (int64_t)1 << 22;
constexpr int64_t kSwigluNvfp4TwoJobOutputs = (int64_t)1 << 25;
// the flat grid indexes jobs with 32 bits (larger launches take the row-chunked grid)
constexpr int64_t kSwigluFlatMaxJobs = 0xFFFFFF00ll;

static int swiglu_find(int jobs_per_lane, int job_outputs, int flat = 0)
{
    for (int i = 0; i < swiglu_variant_count(); ++i) {
        const SwigluVariant *v = swiglu_variant(i);
        if (v->jobs_per_lane == jobs_per_lane && v->job_outputs == job_outputs && v->flat == flat) return i;
    }
    return -1;
}

int pick_swiglu(int64_t tokens, int64_t inter, int epi)
{
    if (tokens < 0 || inter <= 0) return -1;
    // tokens * inter against the thresholds, without forming the product
    if (tokens <= kSwigluHalfJobOutputs / inter) return swiglu_find(1, 4);
    const int64_t njobs = inter / 8;
    const bool flat_fits = njobs > 256 && tokens <= kSwigluFlatMaxJobs / njobs;
    // Rows of 257-511 jobs (N = 2,056-4,088) in every output format: the
    // flat grid (blocks of 256 jobs over the rows laid end to end) measured
    // 1-6% faster than the row-chunked one at N = 3,584 (4,096 and 8,192
    // tokens) in the bf16, MXFP4, NVFP4 and per-group forms.
    if (flat_fits && njobs < 512) return swiglu_find(1, 8, 1);
    // bf16, MXFP4 and per-group E4M3 output: one job per lane on the
    // row-chunked grid (the most blocks, each short-lived, so the blocks in
    // flight stay on one contiguous stretch of memory; per-group E4M3 with
    // two jobs per lane on whole 512-job rows measured 1-2% slower from 8,192
    // tokens of 28,672).  Per-tensor E4M3 output, from about four million
    // outputs: the flat grid, one job per lane and no lane idle at a row's
    // end.  Against two jobs per lane (which gives the longer per-job
    // arithmetic two loads in flight) it measured 2-17% faster from 512
    // tokens on rows that are not whole 512-job blocks (N = 2,560-14,336,
    // where two jobs leave up to 27% of the last block's lanes idle), and
    // on whole 512-job rows (N = 28,672) tied or won at 8,192 tokens on
    // three boxes (up to 4.1%) and at 16,384 (5%), within 1.4% either way at
    // 4,096; on rows of exactly 256 jobs two jobs per lane are faster.
    // NVFP4 output (the most arithmetic per output): two jobs per lane from
    // about 32 million outputs on rows of whole 512-job blocks.
    if (epi == SWIGLU_EPI_FP8 && tokens > kSwigluFp8TwoJobOutputs / inter)
        return flat_fits ? swiglu_find(1, 8, 1) : swiglu_find(2, 8);
    if (epi == SWIGLU_EPI_NVFP4 && tokens > kSwigluNvfp4TwoJobOutputs / inter && (inter / 8) % 512 == 0)
        return swiglu_find(2, 8);
    // The row-chunked grid numbers a row's blocks consecutively, and blocks
    // are dealt to the 8 XCDs in turn.  A row whose jobs end in a partial
    // block and that spans an even number of blocks puts every (light)
    // partial block on the same half of the XCDs or fewer, which then idle
    // while the others finish: the flat grid measured 3-9% faster at
    // 4,096-8,192 tokens of 7,168, 11,008 and 18,944 (4, 6 and 10 blocks per
    // row) in bf16, and level (+-2%) where the count is odd (5,632, 8,960,
    // 9,728, 13,824) or the row is whole blocks.  Per-tensor E4M3 from two
    // million outputs (where half jobs stop): the flat grid, 1.4-5.3% faster
    // at 2.8-3.7 million outputs.
    const int64_t row_blocks = (njobs + 255) / 256;
    if (flat_fits && ((njobs % 256 != 0 && row_blocks % 2 == 0) || epi == SWIGLU_EPI_FP8))
        return swiglu_find(1, 8, 1);
    return swiglu_find(1, 8);
}

int rowq_capacity(const SwigluRowVariant *v) { return v->waves_per_row * 64 * v->jobs_per_lane * 8; }

// Per-token FP8 SwiGLU: the fewest waves per row (one, else 4, 8, 16) that
// hold the row with at most 4 jobs per lane, the fewest jobs for that count;
// else the widest variant.
// A row on one wave takes up to 4 jobs per lane; a row over several waves
// takes at most 3 jobs per lane before it takes 4 (twice the waves with half
// the jobs measured 2-25% faster at 5,632 and 14,336 wide up to 2,048 tokens,
// and never slower by more than 0.3%), then 8.
int pick_swiglu_rowq(int64_t tokens, int64_t inter)
{
    if (tokens < 0 || inter <= 0 || inter > AARMS_MAX_INTER_PER_TOKEN) return -1;
    for (int i = 0; i < swiglu_row_variant_count(); ++i) {
        const SwigluRowVariant *v = swiglu_row_variant(i);
        if (v->waves_per_row == 1 && v->jobs_per_lane <= 4 && rowq_capacity(v) >= inter) return i;
    }
    for (int max_jobs : {3, 4, 8})
        for (int w : {4, 8, 16}) {
            int best = -1;
            for (int i = 0; i < swiglu_row_variant_count(); ++i) {
                const SwigluRowVariant *v = swiglu_row_variant(i);
                if (v->waves_per_row != w || v->jobs_per_lane > max_jobs || rowq_capacity(v) < inter) continue;
                if (best < 0 || v->jobs_per_lane < swiglu_row_variant(best)->jobs_per_lane) best = i;
            }
            if (best >= 0) return best;
        }
    return -1;
}

int launch_status(hipError_t e) { return e == hipSuccess ? AARMS_OK : AARMS_ERR_HIP; }

// All norm forms: epi = NORM_EPI_*, res = with the residual add in front
// (residual and residual_out), scale_out for the dynamic E4M3 form, scale_in
// for the static one.
int norm_common(void *out, float *scale_out, const float *scale_in, void *residual_out,
                const void *x, const void *residual, const void *weight, int64_t tokens,
                int64_t hidden, float eps, int epi, bool res, int variant, hipStream_t stream)
{
    const bool stat = epi == NORM_EPI_FP8_STATIC, grp = epi == NORM_EPI_FP8_GROUP;
    const bool dyn = epi == NORM_EPI_FP8_DYNAMIC || grp;    // scales written to scale_out (fp32)
    const bool mx = epi == NORM_EPI_MXFP4, nv = epi == NORM_EPI_NVFP4;
    const bool fp4 = mx || nv;
    int st = check_width(tokens, hidden, AARMS_MAX_HIDDEN);
    if (st) return st;
    if ((mx && hidden % 32 != 0) || (nv && hidden % 16 != 0) || (grp && hidden % FP8_GROUP != 0))
        return AARMS_ERR_BAD_SHAPE;
    if ((st = check_eps(eps))) return st;
    if (variant < -1 || variant >= norm_variant_count()) return AARMS_ERR_BAD_VARIANT;
    if (tokens == 0) return AARMS_OK;
    if (!out || !x || !weight || (res && (!residual_out || !residual)) || ((dyn || fp4) && !scale_out) ||
        ((stat || nv) && !scale_in))
        return AARMS_ERR_NULL_POINTER;
    if (!aligned(out, 16) || !aligned(x, 16) || !aligned(weight, 16) ||
        (res && (!aligned(residual_out, 16) || !aligned(residual, 16))) ||
        (dyn && !aligned(scale_out, 4)) || ((stat || nv) && !aligned(scale_in, 4)))
        return AARMS_ERR_MISALIGNED;
    const uint64_t elems = (uint64_t)tokens * (uint64_t)hidden;
    // inputs: x, weight, then residual and scale_in when present
    Arg ins[4];
    int n_in = 0;
    ins[n_in++] = {span(x, 2 * elems), x};
    ins[n_in++] = {span(weight, 2 * (uint64_t)hidden), weight};
    const int res_idx = res ? n_in : -1;
    if (res) ins[n_in++] = {span(residual, 2 * elems), residual};
    if (stat || nv) ins[n_in++] = {span(scale_in, 4), scale_in};
    // outputs: out (may be x itself in the bf16 form), residual_out (may be
    // the residual itself), scale_out
    Arg outs[3];
    int partner[3];
    int n_out = 0;
    partner[n_out] = (epi == NORM_EPI_BF16) ? 0 : -1;
    outs[n_out++] = {span(out, epi == NORM_EPI_BF16 ? 2 * elems : fp4 ? elems / 2 : elems), out};
    if (res) {
        partner[n_out] = res_idx;
        outs[n_out++] = {span(residual_out, 2 * elems), residual_out};
    }
    if (dyn || fp4) {
        partner[n_out] = -1;
        outs[n_out++] = {span(scale_out, mx ? elems / 32 : nv ? elems / 16
                                         : grp ? 4 * (elems / FP8_GROUP) : 4 * (uint64_t)tokens),
                         scale_out};
    }
    if ((st = check_outputs(outs, partner, n_out, ins, n_in))) return st;
    if (variant == -1) variant = pick_norm(tokens, hidden, epi, res);
    const NormVariant *v = norm_variant(variant);
    if (!norm_fits(v, hidden)) return AARMS_ERR_BAD_VARIANT;
    NormParams p{};
    p.out = out;
    p.residual_out = res ? residual_out : nullptr;
    p.x = x;
    p.residual = res ? residual : nullptr;
    p.weight = weight;
    p.scale_out = (dyn || fp4) ? scale_out : nullptr;
    p.scale_in = (stat || nv) ? scale_in : nullptr;
    p.tokens = tokens;
    p.hidden = (int32_t)hidden;
    p.eps = eps;
    p.inv_hidden = 1.0 / (double)hidden;
    p.hold_ticks = norm_hold_ticks(tokens, hidden, epi, res, v);
    p.res_last = norm_res_last(tokens, hidden, epi, res);
#ifdef AARMS_PHASE_STAMPS
    p.stamps = g_phase_stamps;
    p.stamp_detail = g_stamp_detail;
#endif
    return launch_status(launch_norm(p, epi, res, variant, device_cus(), stream));
}

// swiglu, its static E4M3 form (scale), its FP4 forms (codes, byte scales
// to scale_out) and its per-group E4M3 form (codes, fp32 scales to
// scale_out).
int swiglu_common(void *out, const void *gate_up, const float *scale, uint8_t *scale_out,
                  int64_t tokens, int64_t inter, int epi, int variant, hipStream_t stream)
{
    const bool fp8 = epi == SWIGLU_EPI_FP8, mx = epi == SWIGLU_EPI_MXFP4, nv = epi == SWIGLU_EPI_NVFP4;
    const bool grp = epi == SWIGLU_EPI_FP8_GROUP;
    const bool with_scale = fp8 || nv, fp4 = mx || nv, with_sout = fp4 || grp;
    int st = check_width(tokens, inter, 0);
    if (st) return st;
    if ((mx && inter % 32 != 0) || (nv && inter % 16 != 0) || (grp && inter % FP8_GROUP != 0))
        return AARMS_ERR_BAD_SHAPE;
    if (inter > AARMS_MAX_INTER) return AARMS_ERR_UNSUPPORTED_SHAPE;
    if (tokens > 0 && 2 * inter > AARMS_MAX_ELEMENTS / tokens) return AARMS_ERR_UNSUPPORTED_SHAPE;
    if (variant < -1 || variant >= swiglu_variant_count()) return AARMS_ERR_BAD_VARIANT;
    if (tokens == 0) return AARMS_OK;
    if (!out || !gate_up || (with_scale && !scale) || (with_sout && !scale_out)) return AARMS_ERR_NULL_POINTER;
    if (!aligned(out, 16) || !aligned(gate_up, 16) || (with_scale && !aligned(scale, 4)) ||
        (grp && !aligned(scale_out, 4)))
        return AARMS_ERR_MISALIGNED;
    const uint64_t elems = (uint64_t)tokens * (uint64_t)inter;
    Arg outs[2];
    int n_out = 0;
    outs[n_out++] = {span(out, (fp8 || grp) ? elems : fp4 ? elems / 2 : 2 * elems), out};
    if (with_sout)
        outs[n_out++] = {span(scale_out, mx ? elems / 32 : nv ? elems / 16 : 4 * (elems / FP8_GROUP)),
                         scale_out};
    const Arg ins[2] = {{span(gate_up, 4 * elems), gate_up}, {span(scale, with_scale ? 4 : 0), scale}};
    const int partner[2] = {-1, -1};
    if ((st = check_outputs(outs, partner, n_out, ins, with_scale ? 2 : 1))) return st;
    if (variant == -1) variant = pick_swiglu(tokens, inter, epi);
    SwigluParams p{};
    p.out = out;
    p.gate_up = gate_up;
    p.scale = with_scale ? scale : nullptr;
    p.scale_out = with_sout ? (float *)scale_out : nullptr;
    p.tokens = tokens;
    p.inter = inter;
    p.vecs_per_row = (uint32_t)(inter / 8);
    return launch_status(launch_swiglu(p, epi, variant, stream));
}

int swiglu_rowq_common(void *out, float *scale_out, const void *gate_up, int64_t tokens,
                       int64_t inter, int variant, hipStream_t stream)
{
    int st = check_width(tokens, inter, AARMS_MAX_INTER_PER_TOKEN);
    if (st) return st;
    if (tokens > 0 && 2 * inter > AARMS_MAX_ELEMENTS / tokens) return AARMS_ERR_UNSUPPORTED_SHAPE;
    if (variant < -1 || variant >= swiglu_row_variant_count()) return AARMS_ERR_BAD_VARIANT;
    if (tokens == 0) return AARMS_OK;
    if (!out || !scale_out || !gate_up) return AARMS_ERR_NULL_POINTER;
    if (!aligned(out, 16) || !aligned(gate_up, 16) || !aligned(scale_out, 4)) return AARMS_ERR_MISALIGNED;
    const uint64_t elems = (uint64_t)tokens * (uint64_t)inter;
    const Arg outs[2] = {{span(out, elems), out}, {span(scale_out, 4 * (uint64_t)tokens), scale_out}};
    const Arg ins[1] = {{span(gate_up, 4 * elems), gate_up}};
    const int partner[2] = {-1, -1};
    if ((st = check_outputs(outs, partner, 2, ins, 1))) return st;
    if (variant == -1) variant = pick_swiglu_rowq(tokens, inter);
    const SwigluRowVariant *v = swiglu_row_variant(variant);
    if (!v || rowq_capacity(v) < inter) return AARMS_ERR_BAD_VARIANT;
    SwigluParams p{};
    p.out = out;
    p.gate_up = gate_up;
    p.scale = nullptr;
    p.scale_out = scale_out;
    p.tokens = tokens;
    p.inter = inter;
    p.vecs_per_row = (uint32_t)(inter / 8);
    return launch_status(launch_swiglu_rowq(p, variant, stream));
}

}  // namespace

extern "C" {

int fused_add_rmsnorm(void *out, void *residual_out, const void *x, const void *residual,
                      const void *weight, int64_t num_tokens, int64_t hidden, float eps,
                      hipStream_t stream)
{
    return norm_common(out, nullptr, nullptr, residual_out, x, residual, weight, num_tokens, hidden,
                       eps, NORM_EPI_BF16, true, -1, stream);
}

int fused_add_rmsnorm_ex(void *out, void *residual_out, const void *x, const void *residual,
                         const void *weight, int64_t num_tokens, int64_t hidden, float eps,
                         int variant, hipStream_t stream)
{
    return norm_common(out, nullptr, nullptr, residual_out, x, residual, weight, num_tokens, hidden,
                       eps, NORM_EPI_BF16, true, variant, stream);
}

int fused_add_rmsnorm_quant_fp8(void *out_fp8, float *scale_out, void *residual_out,
                                const void *x, const void *residual, const void *weight,
                                int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, residual_out, x, residual, weight, num_tokens,
                       hidden, eps, NORM_EPI_FP8_DYNAMIC, true, -1, stream);
}

int fused_add_rmsnorm_quant_fp8_ex(void *out_fp8, float *scale_out, void *residual_out,
                                   const void *x, const void *residual, const void *weight,
                                   int64_t num_tokens, int64_t hidden, float eps, int variant,
                                   hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, residual_out, x, residual, weight, num_tokens,
                       hidden, eps, NORM_EPI_FP8_DYNAMIC, true, variant, stream);
}

int fused_add_rmsnorm_quant_fp8_static(void *out_fp8, void *residual_out, const void *x,
                                       const void *residual, const void *weight, const float *scale,
                                       int64_t num_tokens, int64_t hidden, float eps,
                                       hipStream_t stream)
{
    return norm_common(out_fp8, nullptr, scale, residual_out, x, residual, weight, num_tokens,
                       hidden, eps, NORM_EPI_FP8_STATIC, true, -1, stream);
}

int fused_add_rmsnorm_quant_fp8_static_ex(void *out_fp8, void *residual_out, const void *x,
                                          const void *residual, const void *weight,
                                          const float *scale, int64_t num_tokens, int64_t hidden,
                                          float eps, int variant, hipStream_t stream)
{
    return norm_common(out_fp8, nullptr, scale, residual_out, x, residual, weight, num_tokens,
                       hidden, eps, NORM_EPI_FP8_STATIC, true, variant, stream);
}

int rmsnorm(void *out, const void *x, const void *weight, int64_t num_tokens, int64_t hidden,
            float eps, hipStream_t stream)
{
    return norm_common(out, nullptr, nullptr, nullptr, x, nullptr, weight, num_tokens, hidden, eps,
                       NORM_EPI_BF16, false, -1, stream);
}

int rmsnorm_ex(void *out, const void *x, const void *weight, int64_t num_tokens, int64_t hidden,
               float eps, int variant, hipStream_t stream)
{
    return norm_common(out, nullptr, nullptr, nullptr, x, nullptr, weight, num_tokens, hidden, eps,
                       NORM_EPI_BF16, false, variant, stream);
}

int rmsnorm_quant_fp8(void *out_fp8, float *scale_out, const void *x, const void *weight,
                      int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, nullptr, x, nullptr, weight, num_tokens, hidden,
                       eps, NORM_EPI_FP8_DYNAMIC, false, -1, stream);
}

int rmsnorm_quant_fp8_ex(void *out_fp8, float *scale_out, const void *x, const void *weight,
                         int64_t num_tokens, int64_t hidden, float eps, int variant,
                         hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, nullptr, x, nullptr, weight, num_tokens, hidden,
                       eps, NORM_EPI_FP8_DYNAMIC, false, variant, stream);
}

int rmsnorm_quant_fp8_static(void *out_fp8, const void *x, const void *weight, const float *scale,
                             int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream)
{
    return norm_common(out_fp8, nullptr, scale, nullptr, x, nullptr, weight, num_tokens, hidden,
                       eps, NORM_EPI_FP8_STATIC, false, -1, stream);
}

int rmsnorm_quant_fp8_static_ex(void *out_fp8, const void *x, const void *weight,
                                const float *scale, int64_t num_tokens, int64_t hidden, float eps,
                                int variant, hipStream_t stream)
{
    return norm_common(out_fp8, nullptr, scale, nullptr, x, nullptr, weight, num_tokens, hidden,
                       eps, NORM_EPI_FP8_STATIC, false, variant, stream);
}

int swiglu(void *out, const void *gate_up, int64_t num_tokens, int64_t inter, hipStream_t stream)
{
    return swiglu_common(out, gate_up, nullptr, nullptr, num_tokens, inter, SWIGLU_EPI_BF16, -1, stream);
}

int swiglu_ex(void *out, const void *gate_up, int64_t num_tokens, int64_t inter, int variant,
              hipStream_t stream)
{
    return swiglu_common(out, gate_up, nullptr, nullptr, num_tokens, inter, SWIGLU_EPI_BF16, variant,
                         stream);
}

int swiglu_quant_fp8(void *out_fp8, const void *gate_up, const float *scale, int64_t num_tokens,
                     int64_t inter, hipStream_t stream)
{
    return swiglu_common(out_fp8, gate_up, scale, nullptr, num_tokens, inter, SWIGLU_EPI_FP8, -1, stream);
}

int swiglu_quant_fp8_ex(void *out_fp8, const void *gate_up, const float *scale,
                        int64_t num_tokens, int64_t inter, int variant, hipStream_t stream)
{
    return swiglu_common(out_fp8, gate_up, scale, nullptr, num_tokens, inter, SWIGLU_EPI_FP8, variant,
                         stream);
}

int fused_add_rmsnorm_quant_mxfp4(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                  const void *x, const void *residual, const void *weight,
                                  int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, nullptr, residual_out, x, residual, weight,
                       num_tokens, hidden, eps, NORM_EPI_MXFP4, true, -1, stream);
}

int fused_add_rmsnorm_quant_mxfp4_ex(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                     const void *x, const void *residual, const void *weight,
                                     int64_t num_tokens, int64_t hidden, float eps, int variant,
                                     hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, nullptr, residual_out, x, residual, weight,
                       num_tokens, hidden, eps, NORM_EPI_MXFP4, true, variant, stream);
}

int rmsnorm_quant_mxfp4(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                        int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, nullptr, nullptr, x, nullptr, weight, num_tokens,
                       hidden, eps, NORM_EPI_MXFP4, false, -1, stream);
}

int rmsnorm_quant_mxfp4_ex(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                           int64_t num_tokens, int64_t hidden, float eps, int variant,
                           hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, nullptr, nullptr, x, nullptr, weight, num_tokens,
                       hidden, eps, NORM_EPI_MXFP4, false, variant, stream);
}

int swiglu_quant_mxfp4(void *out_fp4, uint8_t *scale_out, const void *gate_up, int64_t num_tokens,
                       int64_t inter, hipStream_t stream)
{
    return swiglu_common(out_fp4, gate_up, nullptr, scale_out, num_tokens, inter, SWIGLU_EPI_MXFP4, -1,
                         stream);
}

int swiglu_quant_mxfp4_ex(void *out_fp4, uint8_t *scale_out, const void *gate_up, int64_t num_tokens,
                          int64_t inter, int variant, hipStream_t stream)
{
    return swiglu_common(out_fp4, gate_up, nullptr, scale_out, num_tokens, inter, SWIGLU_EPI_MXFP4,
                         variant, stream);
}

int swiglu_quant_nvfp4(void *out_fp4, uint8_t *scale_out, const void *gate_up,
                       const float *tensor_scale, int64_t num_tokens, int64_t inter, hipStream_t stream)
{
    return swiglu_common(out_fp4, gate_up, tensor_scale, scale_out, num_tokens, inter, SWIGLU_EPI_NVFP4,
                         -1, stream);
}

int swiglu_quant_nvfp4_ex(void *out_fp4, uint8_t *scale_out, const void *gate_up,
                          const float *tensor_scale, int64_t num_tokens, int64_t inter, int variant,
                          hipStream_t stream)
{
    return swiglu_common(out_fp4, gate_up, tensor_scale, scale_out, num_tokens, inter, SWIGLU_EPI_NVFP4,
                         variant, stream);
}

int fused_add_rmsnorm_quant_nvfp4(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                  const void *x, const void *residual, const void *weight,
                                  const float *tensor_scale, int64_t num_tokens, int64_t hidden,
                                  float eps, hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, tensor_scale, residual_out, x, residual, weight,
                       num_tokens, hidden, eps, NORM_EPI_NVFP4, true, -1, stream);
}

int fused_add_rmsnorm_quant_nvfp4_ex(void *out_fp4, uint8_t *scale_out, void *residual_out,
                                     const void *x, const void *residual, const void *weight,
                                     const float *tensor_scale, int64_t num_tokens, int64_t hidden,
                                     float eps, int variant, hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, tensor_scale, residual_out, x, residual, weight,
                       num_tokens, hidden, eps, NORM_EPI_NVFP4, true, variant, stream);
}

int rmsnorm_quant_nvfp4(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                        const float *tensor_scale, int64_t num_tokens, int64_t hidden, float eps,
                        hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, tensor_scale, nullptr, x, nullptr, weight,
                       num_tokens, hidden, eps, NORM_EPI_NVFP4, false, -1, stream);
}

int rmsnorm_quant_nvfp4_ex(void *out_fp4, uint8_t *scale_out, const void *x, const void *weight,
                           const float *tensor_scale, int64_t num_tokens, int64_t hidden, float eps,
                           int variant, hipStream_t stream)
{
    return norm_common(out_fp4, (float *)scale_out, tensor_scale, nullptr, x, nullptr, weight,
                       num_tokens, hidden, eps, NORM_EPI_NVFP4, false, variant, stream);
}

int swiglu_quant_fp8_dynamic(void *out_fp8, float *scale_out, const void *gate_up,
                             int64_t num_tokens, int64_t inter, hipStream_t stream)
{
    return swiglu_rowq_common(out_fp8, scale_out, gate_up, num_tokens, inter, -1, stream);
}

int swiglu_quant_fp8_dynamic_ex(void *out_fp8, float *scale_out, const void *gate_up,
                                int64_t num_tokens, int64_t inter, int variant, hipStream_t stream)
{
    return swiglu_rowq_common(out_fp8, scale_out, gate_up, num_tokens, inter, variant, stream);
}

const char *aarms_status_string(int status)
{
    switch (status) {
    case AARMS_OK: return "ok";
    case AARMS_ERR_NULL_POINTER: return "a required pointer is NULL";
    case AARMS_ERR_BAD_SHAPE: return "bad shape: negative size, zero width or width not a multiple of 8";
    case AARMS_ERR_UNSUPPORTED_SHAPE: return "unsupported shape: width or element count beyond the limits";
    case AARMS_ERR_MISALIGNED: return "misaligned pointer: tensors need 16 bytes, scales 4";
    case AARMS_ERR_ALIAS: return "an output overlaps another argument";
    case AARMS_ERR_BAD_EPS: return "eps must be finite and >= 0";
    case AARMS_ERR_HIP: return "the HIP runtime refused the launch";
    case AARMS_ERR_BAD_VARIANT: return "unknown kernel variant, or too narrow for the row";
    default: return "unknown status";
    }
}

int aarms_variant_count(int op)
{
    return (op == 0 || op == 3) ? norm_variant_count()
         : op == 1 ? swiglu_variant_count()
         : op == 2 ? swiglu_row_variant_count() : 0;
}

const char *aarms_variant_name(int op, int variant)
{
    if (op == 0 || op == 3) {
        const NormVariant *v = norm_variant(variant);
        return v ? v->name : nullptr;
    }
    if (op == 1) {
        const SwigluVariant *v = swiglu_variant(variant);
        return v ? v->name : nullptr;
    }
    if (op == 2) {
        const SwigluRowVariant *v = swiglu_row_variant(variant);
        return v ? v->name : nullptr;
    }
    return nullptr;
}

int fused_add_rmsnorm_quant_fp8_group(void *out_fp8, float *scale_out, void *residual_out,
                                      const void *x, const void *residual, const void *weight,
                                      int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, residual_out, x, residual, weight, num_tokens,
                       hidden, eps, NORM_EPI_FP8_GROUP, true, -1, stream);
}

int fused_add_rmsnorm_quant_fp8_group_ex(void *out_fp8, float *scale_out, void *residual_out,
                                         const void *x, const void *residual, const void *weight,
                                         int64_t num_tokens, int64_t hidden, float eps, int variant,
                                         hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, residual_out, x, residual, weight, num_tokens,
                       hidden, eps, NORM_EPI_FP8_GROUP, true, variant, stream);
}

int rmsnorm_quant_fp8_group(void *out_fp8, float *scale_out, const void *x, const void *weight,
                            int64_t num_tokens, int64_t hidden, float eps, hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, nullptr, x, nullptr, weight, num_tokens, hidden, eps,
                       NORM_EPI_FP8_GROUP, false, -1, stream);
}

int rmsnorm_quant_fp8_group_ex(void *out_fp8, float *scale_out, const void *x, const void *weight,
                               int64_t num_tokens, int64_t hidden, float eps, int variant,
                               hipStream_t stream)
{
    return norm_common(out_fp8, scale_out, nullptr, nullptr, x, nullptr, weight, num_tokens, hidden, eps,
                       NORM_EPI_FP8_GROUP, false, variant, stream);
}

int swiglu_quant_fp8_group(void *out_fp8, float *scale_out, const void *gate_up, int64_t num_tokens,
                           int64_t inter, hipStream_t stream)
{
    return swiglu_common(out_fp8, gate_up, nullptr, (uint8_t *)scale_out, num_tokens, inter,
                         SWIGLU_EPI_FP8_GROUP, -1, stream);
}

int swiglu_quant_fp8_group_ex(void *out_fp8, float *scale_out, const void *gate_up, int64_t num_tokens,
                              int64_t inter, int variant, hipStream_t stream)
{
    return swiglu_common(out_fp8, gate_up, nullptr, (uint8_t *)scale_out, num_tokens, inter,
                         SWIGLU_EPI_FP8_GROUP, variant, stream);
}

int aarms_variant_fits(int op, int variant, int64_t width)
{
    if (op == 0 || op == 3) return norm_fits(norm_variant(variant), width) ? 1 : 0;
    if (op == 1) return swiglu_variant(variant) && width > 0 && width % 8 == 0 ? 1 : 0;
    if (op == 2) {
        const SwigluRowVariant *v = swiglu_row_variant(variant);
        return v && width > 0 && width % 8 == 0 && rowq_capacity(v) >= width ? 1 : 0;
    }
    return 0;
}

int aarms_pick_variant(int op, int64_t num_tokens, int64_t width, int quant)
{
    if (op == 0 || op == 3) {
        // quant: the output format (0 bf16, 1 E4M3 per token, 2 E4M3 per
        // tensor, 3 MXFP4, 4 NVFP4, 5 E4M3 per 128-value group)
        if (quant < NORM_EPI_BF16 || quant > NORM_EPI_FP8_GROUP) return -1;
        if (num_tokens < 0 || width % 8 != 0) return -1;
        return pick_norm(num_tokens, width, quant, op == 0);
    }
    if (op == 1) {
        // quant: the output format (0 bf16, 1 E4M3, 2 MXFP4, 3 NVFP4, 4 E4M3
        // with a scale per 128 outputs)
        if (width <= 0 || width % 8 != 0 || quant < 0 || quant > 4) return -1;
        return pick_swiglu(num_tokens, width, quant);
    }
    if (op == 2) return (width > 0 && width % 8 == 0) ? pick_swiglu_rowq(num_tokens, width) : -1;
    return -1;
}

}  // extern "C"
