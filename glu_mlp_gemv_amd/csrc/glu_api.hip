// C ABI of the dual-weight GLU projection: argument validation, the choice of
// kernel by M (DeepSpeed PR #8602, comment "Plan B: Dual-Weight GEMV": the
// DualWeightGluGEMV forward sends a 1-D hidden to the custom kernel and a
// batch elsewhere; the later dispatcher routes by batch size), and launch.
// Validation happens before any HIP call; nothing is allocated or cached.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

#include "../../include/glu_gemv.h"
#include "../../include/glu_gemv_tuning.h"
#include "glu_backward.h"
#include "glu_ceiling.h"
#include "glu_grouped.h"
#include "glu_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = 0x7fffffff;    // N and K index rows and columns in 32 bits
// the VALU and MFMA kernels address a group's weight rows and the hidden
// rows of one launch with 32-bit byte offsets: 32 rows * K * 2 bytes < 2^32
constexpr int64_t kMaxFastK = (int64_t)1 << 25;
constexpr int64_t kMaxValuK = 8192;        // VALU: at most 16 chunks per lane per row
constexpr int64_t kValuMaxDefaultK = 4096;  // longer rows stream faster through the MFMA kernel
constexpr int kCUs = 256;                  // MI355X compute units
constexpr int kValuDefaultWaves = 4;       // waves per workgroup
constexpr int kValuWavesPerCU = 3;         // persistent waves per CU the grid aims for
constexpr int kMfmaDefaultWaves = 4;
constexpr int kMfmaWavesPerCU = 4;
constexpr int kGrouped8MinM = 8;  // grouped MFMA: 8-row groups by default above this many rows of hidden
constexpr int64_t kGemmSlice = 65536;        // rows of hidden per GEMM launch
constexpr int64_t kGemmMaxN = 1 << 30;       // GEMM tile row indices stay in 32 bits
constexpr int kMfmaSlice = 32;
constexpr int kGroupedSlices64U = 8;  // the grouped slice kernel's stage (64-element segments) at 33..64 rows

bool mul_overflows(int64_t a, int64_t b, int64_t limit)
{
    return a != 0 && b > limit / a;
}

struct Launch {
    int kernel = GLU_KERNEL_NONE;
    int m_per_launch = 0;
    int launches = 0;
    glu::ValuConfig valu{};
    glu::MfmaConfig mfma{};
    glu::GemmConfig gemm{};
    int gemm_grid = 0;
    int generic_grid = 0;
    int accum_depth = 0;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Persistent grid: about `target` waves in total, each owning the same number of
// work units to within one.
int64_t balanced_waves(int64_t units, int64_t target)
{
    if (units < 1) return 0;
    const int64_t per = ceil_div(units, target < 1 ? 1 : target);
    return ceil_div(units, per);
}

// Workgroups for the grouped 8-row layout: `groups` groups of 8 weight rows, at most `slots` waves
// resident, `waves` per workgroup.  One CU's share of the bandwidth saturates near
// kMfmaWavesPerCU waves of this kernel, so a CU takes about max(its groups / kMfmaWavesPerCU, the
// groups of its busiest wave) group-times.  For p = 1..4 more than the fewest groups per wave that
// fit the slots, spread evenly, the plan takes the p with the fewest such steps (ties: more waves).
// Measured at K = 2560 with 12 and 16 rows of hidden: two 9216-row projections run in 19.7 and
// 20.6 us on 192 workgroups against 25.0 and 26.3 on the 288 of an even spread over all 2048 slots.
int64_t grouped8_grid(int64_t groups, int64_t slots, int64_t waves)
{
    const int64_t p0 = ceil_div(groups, slots < 1 ? 1 : slots);
    int64_t best = 1, best_steps = INT64_MAX;
    for (int64_t p = p0; p < p0 + 4; ++p) {
        const int64_t blocks = ceil_div(ceil_div(groups, p), waves);
        const int64_t waves_per_cu = ceil_div(blocks * waves, kCUs);
        const int64_t steps = p * ceil_div(waves_per_cu, kMfmaWavesPerCU);
        if (steps < best_steps) {
            best_steps = steps;
            best = blocks;
        }
    }
    return best;
}

glu_status plan_valu(int64_t M, int64_t N, int64_t K, const glu_tuning* t, Launch* L)
{
    if (M > glu::kValuMaxM || K > kMaxValuK) return GLU_ERR_UNSUPPORTED;
    glu::ValuConfig c{};
    const int64_t nchunks = K / 8;
    const int64_t cpl = ceil_div(nchunks, glu::kWave);
    c.NB = cpl <= 8 ? 1 : 2;
    c.U = (int)ceil_div(cpl, c.NB);
    c.ragged = (int64_t)c.NB * c.U * glu::kWave != nchunks;
    c.R = (t && t->rows_per_wave) ? t->rows_per_wave : 1;
    const int waves = (t && t->waves_per_block) ? t->waves_per_block : kValuDefaultWaves;
    if (waves < 1 || waves * glu::kWave > glu::kValuMaxThreads) return GLU_ERR_UNSUPPORTED;
    c.block = waves * glu::kWave;
    // rows of hidden per launch: all of them, unless staging in LDS needs slices
    int64_t m_pl = M;
    if (glu::valu_hidden_in_lds((int)M, c.U, c.NB)) {
        const int64_t m_fit = glu::kLdsBudget / (2 * K);
        m_pl = M < m_fit ? M : m_fit;
    }
    const int64_t groups = ceil_div(N, c.R);
    int64_t grid;
    if (t && t->grid > 0) {
        grid = t->grid;
    } else {
        grid = ceil_div(balanced_waves(groups, (int64_t)kCUs * kValuWavesPerCU), waves);
    }
    c.grid = (int)(grid < 1 ? 1 : grid);
    c.M = (int)m_pl;
    // M = 1: the dot products on the matrix cores by default (the 32-layer K=2560 N=9216 stack in
    // interleaved warm graphs: 15.56 against 15.65 us per call with fp32 FMAs on the vector ALU)
    const int dot = t ? t->gemv_dot : 0;
    if (dot < 0 || dot > 2 || (dot == 2 && M != 1)) return GLU_ERR_UNSUPPORTED;
    if (dot == 2 && c.block > glu::kMfmaMaxThreads) return GLU_ERR_UNSUPPORTED;
    c.diag = M == 1 && dot != 1 && c.block <= glu::kMfmaMaxThreads;
    if (!glu::valu_supported(c)) return GLU_ERR_UNSUPPORTED;
    glu::ValuConfig last = c;  // the last slice may be narrower: it must be instantiated too
    last.M = (int)(M - (ceil_div(M, m_pl) - 1) * m_pl);
    if (!glu::valu_supported(last)) return GLU_ERR_UNSUPPORTED;
    L->kernel = GLU_KERNEL_VALU;
    L->valu = c;
    L->m_per_launch = (int)m_pl;
    L->launches = (int)ceil_div(M, m_pl);
    // FMA: a lane's 8 products per chunk in order, then the butterfly.  Matrix cores: per row one
    // MFMA per 512-element piece, each adding a 32-product block (a tree of depth 5) to the
    // accumulator, counted at twice the fp32 unit roundoff (the core's internal rounding is not
    // specified), then the butterfly over the 16 diagonal entries
    L->accum_depth = c.diag ? 2 * (c.U * c.NB + 5) + glu::kWaveSumDepth : 8 * c.U * c.NB + glu::kWaveSumDepth;
    return GLU_OK;
}

// Segments per stage: the largest of 5, 4, 2 that divides the segment count (no
// ragged tail) and keeps the stage's registers in budget as hidden tiles grow.
int default_segments(int64_t nsegs, int mt4, int hidden)
{
    const int cap = hidden == glu::kHiddenL2 ? 2 : (hidden == glu::kHiddenSlices ? 4 : (mt4 <= 2 ? 5 : (mt4 <= 4 ? 4 : 2)));
    for (int u : {5, 4, 2}) {
        if (u <= cap && nsegs % u == 0) return u;
    }
    return cap < 4 ? cap : 4;
}

glu_status plan_mfma_shape(int64_t M, int64_t N, int64_t K, const glu_tuning* t, Launch* L)
{
    glu::MfmaConfig c{};
    // the slice-major 8-row kernel with stages of 4 segments takes up to 64 rows of hidden per launch
    const bool pass64 = t && t->rows_per_wave == 8 && t->mfma_order == 2 && t->mfma_segments == 4;
    const int64_t m_cap = pass64 ? 2 * kMfmaSlice : kMfmaSlice;
    const int64_t m_pl = M < m_cap ? M : m_cap;
    if (pass64 && m_pl <= kMfmaSlice) return GLU_ERR_UNSUPPORTED;  // 4-segment stages serve 33..64 rows
    c.MT4 = (int)((m_pl + 3) / 4);
    const int64_t nchunks = K / 8;
    const int64_t nsegs = ceil_div(nchunks, 16);
    const int waves = (t && t->waves_per_block) ? t->waves_per_block : kMfmaDefaultWaves;
    const int seg_req = t ? t->mfma_segments : 0;
    const int rows_req = t ? t->rows_per_wave : 0;
    const int order_req = t ? t->mfma_order : 0;
    if (t && t->mfma_hidden) {
        c.hidden = t->mfma_hidden - 1;
    } else if (rows_req == 8) {
        c.hidden = glu::kHiddenSlices;  // the only place 8 rows per wave are built for
    } else if (glu::mfma_hidden_lds_bytes((int)m_pl, K) <= (size_t)glu::kLdsBudget) {
        c.hidden = glu::kHiddenLds;
    } else if (waves * glu::kWave == glu::kMfmaMaxThreads && (seg_req == 0 || seg_req == 2 || seg_req == 4)) {
        c.hidden = glu::kHiddenSlices;
    } else {
        c.hidden = glu::kHiddenL2;
    }
    // 8 weight rows per wave halve the MFMAs, operand reads and hidden-slice
    // traffic per weight byte, which pays once the slices carry more than 16
    // rows of hidden; up to 16 rows 4 rows per wave stream the weights faster
    // (K=5120 N=17408: 62.7 against 64.9 us at M = 16, 71.8 against 81.6 at 32)
    const bool seg8 = seg_req == 0 || seg_req == 4 || seg_req == 8;  // stage sizes built for 8 rows
    const int rows_dflt = (c.hidden == glu::kHiddenSlices && m_pl > 16 && seg8) ? 8 : 4;
    c.rows = rows_req ? rows_req : rows_dflt;
    if (c.rows != 4 && !(c.rows == 8 && c.hidden == glu::kHiddenSlices)) return GLU_ERR_UNSUPPORTED;
    // segments of 128 K-elements at 4 rows per wave, of 64 at 8
    const int64_t seg_chunks = c.rows == 8 ? 8 : 16;
    const int64_t nseg = ceil_div(nchunks, seg_chunks);
    if (c.rows == 8) {
        c.U = seg_req ? seg_req : 8;
    } else {
        c.U = seg_req ? seg_req : default_segments(nsegs, c.MT4, c.hidden);
    }
    if (c.U < 1) return GLU_ERR_UNSUPPORTED;
    if (c.hidden == glu::kHiddenSlices) {
        int dflt = c.rows == 8 ? glu::mfma8_slice_depth(c.U) : glu::mfma_slice_depth(c.U);
        if (c.rows == 8 && c.U == 8 && m_pl <= 16) dflt = 2;  // fewer MFMAs per stage: room for a deeper pipeline
        if (c.rows == 8 && order_req == 2) dflt = 1;  // the slice-major kernel keeps one stage in flight
        c.depth = (t && t->mfma_depth) ? t->mfma_depth : dflt;
    } else if (t && t->mfma_depth) {
        return GLU_ERR_UNSUPPORTED;  // only the lockstep kernels take a depth
    }
    c.nsg = (int)ceil_div(nseg, c.U);
    c.ragged = (int64_t)c.nsg * c.U * seg_chunks != nchunks;
    if (waves < 1 || waves * glu::kWave > glu::kMfmaMaxThreads) return GLU_ERR_UNSUPPORTED;
    c.block = waves * glu::kWave;
    const int64_t groups = ceil_div(N, c.rows);
    int64_t grid;
    if (t && t->grid > 0) {
        grid = t->grid;
    } else if (c.hidden == glu::kHiddenSlices) {
        // workgroups take blocks of `waves` adjacent groups
        grid = balanced_waves(ceil_div(groups, waves), (int64_t)kCUs * kMfmaWavesPerCU / waves);
    } else {
        grid = ceil_div(balanced_waves(groups, (int64_t)kCUs * kMfmaWavesPerCU), waves);
    }
    c.grid = (int)(grid < 1 ? 1 : grid);
    // 8 rows per wave: the order of the K walk (block by block, or K once for up to
    // kPassBlocks blocks of a workgroup, each hidden slice loaded once for all of them)
    if (order_req < 0 || order_req > 2 || (order_req && c.rows != 8)) return GLU_ERR_UNSUPPORTED;
    c.order = glu::kOrderBlocks;
    if (c.rows == 8) {
        const bool pass_fits = ((c.U == 8 && m_pl > 8 && m_pl <= kMfmaSlice) || (c.U == 4 && m_pl > kMfmaSlice)) &&
                               c.depth == 1 && (int64_t)c.grid * glu::kPassBlocks >= glu::mfma8_blocks(N);
        if (order_req == 2 && !pass_fits) return GLU_ERR_UNSUPPORTED;
        c.order = order_req == 2 ? glu::kOrderSlices : glu::kOrderBlocks;
    }
    if (c.hidden == glu::kHiddenSlices && c.block != glu::kMfmaMaxThreads) return GLU_ERR_UNSUPPORTED;
    if (!glu::mfma_supported(c)) return GLU_ERR_UNSUPPORTED;
    L->kernel = GLU_KERNEL_MFMA;
    L->mfma = c;
    L->m_per_launch = (int)m_pl;
    L->launches = (int)ceil_div(M, m_pl);
    // per output lane: one MFMA per segment, each adding a 32-product block
    // (a summation tree of depth 5) to the accumulator, then the block sums
    // (two quad additions at 4 rows, one pair addition at 8); the matrix
    // core's internal rounding is not specified, so every step is counted at
    // twice the fp32 unit roundoff (a truncating adder)
    L->accum_depth = (int)(2 * (nseg + 5 + 2));
    return GLU_OK;
}

// Above 8 rows of hidden, when hidden does not fit in LDS, the default is 8 weight rows per wave
// with the K walk done once for up to 3 blocks of a workgroup (each K-slice of hidden loaded and
// published once for all of them).  K=5120 N=17408, interleaved warm graphs: M = 16 60.5 us
// against 62.3 for 4 rows per wave; M = 24 62.7 against 68.7 and M = 32 64.9 against 71.7 for the
// block-by-block walk (M = 1 at that shape: 53.3).  Above 32 rows the same kernel takes launches of
// 64 rows with stages of 4 segments: M = 64 74.4 us against 128.6 for two launches of 32 rows and
// 111.2 for the tiled GEMM, which the default path takes above 64 rows.  Overrides of the rows, the
// order, the stage size, the depth or where hidden lives plan exactly what they ask for.
glu_status plan_mfma(int64_t M, int64_t N, int64_t K, const glu_tuning* t, Launch* L)
{
    const int64_t m_pl = M < kMfmaSlice ? M : kMfmaSlice;
    const int waves = (t && t->waves_per_block) ? t->waves_per_block : kMfmaDefaultWaves;
    const bool free_shape = !t || (!t->rows_per_wave && !t->mfma_order && !t->mfma_segments && !t->mfma_depth &&
                                   !t->mfma_hidden);
    if (free_shape && waves * glu::kWave == glu::kMfmaMaxThreads &&
        (M > kMfmaSlice || (m_pl > 8 && glu::mfma_hidden_lds_bytes((int)m_pl, K) > (size_t)glu::kLdsBudget))) {
        glu_tuning t8 = t ? *t : glu_tuning{};
        t8.rows_per_wave = 8;
        t8.mfma_order = 2;
        if (M > kMfmaSlice) t8.mfma_segments = 4;  // launches of 64 rows
        if (plan_mfma_shape(M, N, K, &t8, L) == GLU_OK) return GLU_OK;
    }
    return plan_mfma_shape(M, N, K, t, L);
}

// Tiled GEMM: 64 weight rows per tile; 64 hidden rows up to M = 256, else 128.
// Smaller tiles let 2-3 workgroups share a CU, and that occupancy hides more
// load latency than the larger tiles' operand reuse saves (measured at K=5120
// N=17408 and K=2560 N=9216, M = 64..1024).
glu_status plan_gemm(int64_t M, int64_t N, int64_t K, const glu_tuning* t, Launch* L)
{
    if (N > kGemmMaxN) return GLU_ERR_UNSUPPORTED;
    if (t && (t->rows_per_wave || t->waves_per_block || t->grid || t->mfma_segments || t->mfma_hidden)) {
        return GLU_ERR_UNSUPPORTED;
    }
    glu::GemmConfig c{};
    c.depth = (t && t->mfma_depth) ? t->mfma_depth : 2;  // two stages of loads in flight: 2-12 % faster
    c.bm = (t && t->gemm_tile_m) ? t->gemm_tile_m : (M <= 256 ? 64 : 128);
    c.bn = (t && t->gemm_tile_n) ? t->gemm_tile_n : 64;
    c.ktail = K % 64 != 0;
    int64_t m_pl = M < kGemmSlice ? M : kGemmSlice;
    if (!glu::gemm_supported(c)) return GLU_ERR_UNSUPPORTED;
    // the grid of one launch stays below 2^30 workgroups
    const int64_t nbn = ceil_div(N, c.bn);
    const int64_t max_m = (((int64_t)1 << 30) / nbn) * c.bm;
    if (m_pl > max_m) m_pl = max_m;
    L->kernel = GLU_KERNEL_GEMM;
    L->gemm = c;
    L->m_per_launch = (int)m_pl;
    L->launches = (int)ceil_div(M, m_pl);
    L->gemm_grid = (int)glu::gemm_grid(c, m_pl, N);
    L->accum_depth = (int)(2 * (ceil_div(K, 32) + 6));
    return GLU_OK;
}

glu_status plan_launch_any(int64_t M, int64_t N, int64_t K, bool aligned16, const glu_tuning* t, Launch* L)
{
    if (M < 0 || N < 0 || K < 0 || N > kMaxDim || K > kMaxDim) return GLU_ERR_BAD_SHAPE;
    const int64_t lim = INT64_MAX / 2;  // element counts must also fit as byte counts
    if (mul_overflows(M, K, lim) || mul_overflows(N, K, lim) || mul_overflows(M, N, lim)) {
        return GLU_ERR_BAD_SHAPE;
    }
    *L = Launch{};
    if (M == 0 || N == 0) return GLU_OK;
    if (K == 0) {
        L->kernel = GLU_KERNEL_ZERO;
        L->m_per_launch = (int)(M > kMaxDim ? kMaxDim : M);
        L->launches = 1;
        return GLU_OK;
    }
    const int forced = t ? t->kernel : 0;
    if (t && t->xcd_bands) return GLU_ERR_UNSUPPORTED;  // only the streaming-read yardstick takes it
    const bool fast = aligned16 && (K % 8 == 0) && K <= kMaxFastK;
    if (forced != 0 && forced != GLU_KERNEL_GENERIC && !fast) return GLU_ERR_UNSUPPORTED;
    const bool gemm_fields = t && (t->gemm_tile_n || t->gemm_tile_m);
    if (gemm_fields && forced != 0 && forced != GLU_KERNEL_GEMM) return GLU_ERR_UNSUPPORTED;
    if (forced == GLU_KERNEL_VALU) return plan_valu(M, N, K, t, L);
    if (forced == GLU_KERNEL_MFMA) return plan_mfma(M, N, K, t, L);
    if (forced == GLU_KERNEL_GEMM) return plan_gemm(M, N, K, t, L);
    if (forced == 0 && fast) {
        if (gemm_fields || (M > 2 * kMfmaSlice && N <= kGemmMaxN)) return plan_gemm(M, N, K, t, L);
        if (M == 1 && K <= kValuMaxDefaultK) return plan_valu(M, N, K, t, L);
        return plan_mfma(M, N, K, t, L);
    }
    if (gemm_fields) return GLU_ERR_UNSUPPORTED;
    if (forced != 0 && forced != GLU_KERNEL_GENERIC) return GLU_ERR_UNSUPPORTED;
    L->kernel = GLU_KERNEL_GENERIC;
    L->m_per_launch = (int)(M < 8 ? M : 8);
    L->launches = (int)ceil_div(M, L->m_per_launch);
    L->generic_grid = (int)ceil_div(N, 4);
    L->accum_depth = (int)ceil_div(K, glu::kWave) + glu::kWaveSumDepth;
    return GLU_OK;
}

// Streaming-read ceiling: the VALU GEMV's launch shape for two matrices of `rows`
// rows of row_bytes bytes (a row of K bf16 weights is 2K bytes).
struct CeilingLaunch {
    int U = 0, R = 0, grid = 0, block = 0;
    bool xcd_bands = false;
};

glu_status plan_ceiling(int64_t rows, int64_t row_bytes, const glu_tuning* t, CeilingLaunch* c)
{
    if (rows < 0 || row_bytes < 0 || rows > kMaxDim) return GLU_ERR_BAD_SHAPE;
    if (mul_overflows(rows, row_bytes, INT64_MAX / 2)) return GLU_ERR_BAD_SHAPE;
    if (t && (t->kernel || t->mfma_segments || t->mfma_hidden || t->mfma_depth || t->gemm_tile_n ||
              t->gemm_tile_m || t->mfma_order || t->gemv_dot)) {
        return GLU_ERR_UNSUPPORTED;
    }
    *c = CeilingLaunch{};
    if (rows == 0) return GLU_OK;
    if (row_bytes == 0 || row_bytes % 1024 != 0) return GLU_ERR_UNSUPPORTED;
    c->U = (int)(row_bytes / 1024 < 9 ? row_bytes / 1024 : 0);
    c->R = (t && t->rows_per_wave) ? t->rows_per_wave : 1;
    if (!glu::read_ceiling_supported(c->U, c->R)) return GLU_ERR_UNSUPPORTED;
    const int waves = (t && t->waves_per_block) ? t->waves_per_block : kValuDefaultWaves;
    if (waves < 1 || waves * glu::kWave > glu::kValuMaxThreads) return GLU_ERR_UNSUPPORTED;
    c->block = waves * glu::kWave;
    const int64_t groups = ceil_div(rows, c->R);
    const int64_t grid = (t && t->grid > 0) ? t->grid
                                            : ceil_div(balanced_waves(groups, (int64_t)kCUs * kValuWavesPerCU), waves);
    c->grid = (int)(grid < 1 ? 1 : grid);
    c->xcd_bands = t && t->xcd_bands;
    if (c->xcd_bands && c->grid % glu::kXcds != 0) return GLU_ERR_UNSUPPORTED;
    return GLU_OK;
}

glu_status plan_launch(int64_t M, int64_t N, int64_t K, bool aligned16, const glu_tuning* t, Launch* L)
{
    const glu_status st = plan_launch_any(M, N, K, aligned16, t, L);
    // the K-walk order is a field of the 8-row MFMA kernel only, the dot products' unit of the VALU GEMV
    if (st == GLU_OK && t && t->mfma_order && L->kernel != GLU_KERNEL_NONE &&
        !(L->kernel == GLU_KERNEL_MFMA && L->mfma.rows == 8)) {
        return GLU_ERR_UNSUPPORTED;
    }
    if (st == GLU_OK && t && t->gemv_dot && L->kernel != GLU_KERNEL_NONE && L->kernel != GLU_KERNEL_VALU) {
        return GLU_ERR_UNSUPPORTED;
    }
    return st;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes)
{
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

glu_status fail_launch(hipError_t e)
{
    g_last_hip_error = (int)e;
    return GLU_ERR_LAUNCH;
}

// Elements spanned by `rows` rows of `len` elements at stride `ld`, or -1 if
// that does not fit in int64 as a byte count.
int64_t extent(int64_t rows, int64_t ld, int64_t len)
{
    const int64_t lim = INT64_MAX / 2;
    if (rows <= 0 || len <= 0) return 0;
    if (mul_overflows(rows - 1, ld, lim) || (rows - 1) * ld > lim - len) return -1;
    return (rows - 1) * ld + len;
}

glu_status run(const uint16_t* hidden, int64_t ldh, const uint16_t* gate_w, int64_t ldg, const uint16_t* up_w,
               int64_t ldu, uint16_t* out, int64_t ldo, int64_t M, int64_t N, int64_t K, void* stream,
               const glu_tuning* t)
{
    if (M < 0 || N < 0 || K < 0) return GLU_ERR_BAD_SHAPE;
    Launch L;
    // shape errors first, independent of the pointers
    glu_status st = plan_launch(M, N, K, true, nullptr, &L);
    if (st != GLU_OK) return st;
    if (M == 0 || N == 0) return GLU_OK;
    // strides: every row must fit in front of the next; inputs only matter when K > 0
    if (ldo < N || (K > 0 && (ldh < K || ldg < K || ldu < K))) return GLU_ERR_BAD_STRIDE;
    const int64_t out_len = extent(M, ldo, N);
    const int64_t h_len = K > 0 ? extent(M, ldh, K) : 0;
    const int64_t g_len = K > 0 ? extent(N, ldg, K) : 0;
    const int64_t u_len = K > 0 ? extent(N, ldu, K) : 0;
    if (out_len < 0 || h_len < 0 || g_len < 0 || u_len < 0) return GLU_ERR_BAD_STRIDE;
    if (!out || (K > 0 && (!hidden || !gate_w || !up_w))) return GLU_ERR_NULL_POINTER;
    const uintptr_t odd = ((uintptr_t)out | (uintptr_t)hidden | (uintptr_t)gate_w | (uintptr_t)up_w) & 1u;
    if (odd) return GLU_ERR_MISALIGNED;
    if (K > 0 && (overlaps(out, out_len * 2, hidden, h_len * 2) || overlaps(out, out_len * 2, gate_w, g_len * 2) ||
                  overlaps(out, out_len * 2, up_w, u_len * 2))) {
        return GLU_ERR_ALIASING;
    }
    // the fast kernels read 16-byte chunks of every row: pointers and row
    // strides must keep rows 16-byte aligned, and strides fit their 32-bit offsets
    const bool aligned16 = (((uintptr_t)hidden | (uintptr_t)gate_w | (uintptr_t)up_w) & 15u) == 0 &&
                           ((ldh | ldg | ldu) & 7) == 0 && ldh <= kMaxFastK && ldg <= kMaxFastK && ldu <= kMaxFastK;
    st = plan_launch(M, N, K, aligned16, t, &L);
    if (st != GLU_OK) return st;

    const glu::RowStrides ld{ldh, ldg, ldu, ldo};
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    switch (L.kernel) {
    case GLU_KERNEL_ZERO:
        e = glu::zero_launch(out, M, N, ldo, s);
        break;
    case GLU_KERNEL_GENERIC:
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += L.m_per_launch) {
            const int mc = (int)(M - m0 < L.m_per_launch ? M - m0 : L.m_per_launch);
            e = glu::generic_launch(mc, hidden + m0 * ldh, gate_w, up_w, out + m0 * ldo, N, K, ld, s);
        }
        break;
    case GLU_KERNEL_VALU:
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += L.m_per_launch) {
            glu::ValuConfig c = L.valu;
            c.M = (int)(M - m0 < L.m_per_launch ? M - m0 : L.m_per_launch);
            e = glu::valu_launch(c, hidden + m0 * ldh, gate_w, up_w, out + m0 * ldo, N, K, ld, s);
        }
        break;
    case GLU_KERNEL_MFMA:
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += L.m_per_launch) {
            const int mc = (int)(M - m0 < L.m_per_launch ? M - m0 : L.m_per_launch);
            e = glu::mfma_launch(L.mfma, mc, hidden + m0 * ldh, gate_w, up_w, out + m0 * ldo, N, K, ld, s);
        }
        break;
    case GLU_KERNEL_GEMM:
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += L.m_per_launch) {
            const int mc = (int)(M - m0 < L.m_per_launch ? M - m0 : L.m_per_launch);
            e = glu::gemm_launch(L.gemm, mc, hidden + m0 * ldh, gate_w, up_w, out + m0 * ldo, (int)N, (int)K, ld, s);
        }
        break;
    default:
        return GLU_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? GLU_OK : fail_launch(e);
}

// ---- grouped GEMV ------------------------------------------------------------

// Grouped GEMV launch.  `fast`: the layout meets the fast kernels' conditions;
// `mult4` / `mult8`: every projection's row count is a multiple of 4 / 8.  M >= 2
// (or a forced MFMA) with fast and mult4 takes the block-diagonal MFMA kernel,
// M <= 32 per launch, in groups of 8 weight rows above 8 rows of hidden when
// mult8 holds and hidden fits in LDS; else the VALU kernel (at most 16 chunks
// per lane per row, K <= 8192, M <= 8 per launch); else the generic kernel.
glu_status plan_grouped(int64_t M, int64_t K, int64_t rows, bool fast, bool mult4, bool mult8, const glu_tuning* t,
                        Launch* L)
{
    if (M < 0 || K < 0 || rows < 0 || M > kMaxDim || K > kMaxDim || rows > kMaxDim) return GLU_ERR_BAD_SHAPE;
    const int64_t lim = INT64_MAX / 2;
    if (mul_overflows(M, K, lim) || mul_overflows(rows, K, lim) || mul_overflows(M, rows, lim)) {
        return GLU_ERR_BAD_SHAPE;
    }
    *L = Launch{};
    if (M == 0 || rows == 0) return GLU_OK;
    if (K == 0) {
        L->kernel = GLU_KERNEL_ZERO;
        L->m_per_launch = (int)(M > kMaxDim ? kMaxDim : M);
        L->launches = 1;
        return GLU_OK;
    }
    const int forced = t ? t->kernel : 0;
    if (t && (t->gemm_tile_n || t->gemm_tile_m || t->xcd_bands || t->mfma_order || t->gemv_dot)) {
        return GLU_ERR_UNSUPPORTED;
    }
    const bool mfma_fields = t && (t->mfma_segments || t->mfma_hidden || t->mfma_depth);
    const bool mfma = fast && mult4 && (forced == GLU_KERNEL_MFMA || (forced == 0 && (M >= 2 || mfma_fields)));
    if (forced == GLU_KERNEL_MFMA && !mfma) return GLU_ERR_UNSUPPORTED;
    if (mfma_fields && !mfma) return GLU_ERR_UNSUPPORTED;
    if (mfma) {
        if (t && (t->mfma_depth || (t->rows_per_wave && t->rows_per_wave != 4 && t->rows_per_wave != 8))) {
            return GLU_ERR_UNSUPPORTED;
        }
        if (rows % 4 != 0) return GLU_ERR_UNSUPPORTED;  // whole 4-row groups only
        glu::MfmaConfig c{};
        const int64_t m_pl = M < kMfmaSlice ? M : kMfmaSlice;
        c.rows = 4;
        c.MT4 = (int)((m_pl + 3) / 4);
        const int64_t nchunks = K / 8;
        const int64_t nsegs = ceil_div(nchunks, 16);
        // 8 weight rows per group (the 8-row layout) above 8 rows of hidden held in LDS: half the
        // MFMAs and LDS operand reads per weight byte (K=2560, a 63 MB quad: 18.3 -> 16.8 us at
        // M = 16, 31.1 -> 21.6 at M = 32)
        const bool can8 = mult8 && m_pl > 8 && nchunks % 16 == 0 && (!t || !t->mfma_hidden || t->mfma_hidden == 1) &&
                          glu::mfma_hidden_lds_bytes((int)m_pl, K) <= (size_t)glu::kLdsMax;
        const int rows_req = t ? t->rows_per_wave : 0;
        // 8-row layout with K-slices of hidden streamed under the weights (mfma_hidden = 3, and the
        // default above 8 rows of hidden when every projection's N is a multiple of 8): a workgroup of
        // 4 waves walks K once for up to 3 blocks of 4 groups.  Against hidden staged whole into LDS
        // first (K=2560): a QKV-like triple (31.5 MB) at M = 16 / 32 9.7 / 10.7 us against 11.0 / 15.0,
        // a GDN-input-like quad (63.2 MB) 14.5 / 16.4 against 17.0 / 21.6
        const bool slices_default = mult8 && m_pl > kGrouped8MinM &&
                                    (!t || (!t->mfma_hidden && (!t->mfma_segments || t->mfma_segments == 4) &&
                                            !t->rows_per_wave && !t->waves_per_block && !t->grid));
        if (slices_default || (t && t->mfma_hidden == 3)) {
            const int seg_req = t ? t->mfma_segments : 0;
            if (!mult8 || (t && ((rows_req && rows_req != 8) || (seg_req && seg_req != 8 && seg_req != 4) ||
                                 (t->waves_per_block && t->waves_per_block != 4)))) {
                return GLU_ERR_UNSUPPORTED;
            }
            // up to 64 rows of hidden per launch (the weights read once where launches of 32 rows
            // read them twice); stages of 4 segments only above 32 rows
            const int64_t m_s = M < 2 * kMfmaSlice ? M : 2 * kMfmaSlice;
            const int useg = seg_req ? seg_req : (m_s > kMfmaSlice ? kGroupedSlices64U : 8);
            if (useg == 4 && m_s <= kMfmaSlice) return GLU_ERR_UNSUPPORTED;
            const int64_t nsegs8 = ceil_div(nchunks, 8);
            c.rows = 8;
            c.MT4 = (int)(m_s <= 8 ? 2 : (m_s + 7) / 8);
            c.hidden = glu::kHiddenSlices;
            c.U = useg;
            c.nsg = (int)ceil_div(nsegs8, c.U);
            c.ragged = (int64_t)c.nsg * c.U * 8 != nchunks;
            c.block = glu::kMfmaMaxThreads;
            const int64_t blocks = ceil_div(rows / 8, 4);
            // about one workgroup per CU: the fewest blocks per workgroup that keep the grid within the
            // CUs (QKV-like 192 blocks: one each; GDN-like 386: two each, measured best of 1, 2, 3)
            const int64_t jb = std::min<int64_t>(ceil_div(blocks, kCUs), glu::kPassBlocks);
            const int64_t grid = (t && t->grid > 0) ? t->grid : ceil_div(blocks, jb);
            if (grid < ceil_div(blocks, glu::kPassBlocks) || grid > blocks) return GLU_ERR_UNSUPPORTED;
            c.grid = (int)grid;
            if (!glu::grouped_mfma_supported(c)) return GLU_ERR_UNSUPPORTED;
            L->kernel = GLU_KERNEL_MFMA;
            L->mfma = c;
            L->m_per_launch = (int)m_s;
            L->launches = (int)ceil_div(M, m_s);
            L->accum_depth = (int)(2 * (nsegs8 + 5 + 2));
            return GLU_OK;
        }
        if (rows_req == 8 && !can8) return GLU_ERR_UNSUPPORTED;
        if (can8 && (rows_req == 8 || (rows_req == 0 && m_pl > kGrouped8MinM))) {
            const int64_t nsegs8 = nchunks / 8;
            c.rows = 8;
            c.MT4 = (int)((m_pl + 7) / 8);
            c.hidden = glu::kHiddenLds;
            c.U = (t && t->mfma_segments) ? t->mfma_segments : (nsegs8 % 8 == 0 || nsegs8 % 5 != 0 ? 8 : 5);
            if (c.U < 1) return GLU_ERR_UNSUPPORTED;
            c.nsg = (int)ceil_div(nsegs8, c.U);
            c.ragged = (int64_t)c.nsg * c.U * 8 != nchunks;
            const int waves = (t && t->waves_per_block) ? t->waves_per_block : kMfmaDefaultWaves;
            if (waves < 1 || waves * glu::kWave > glu::kMfmaMaxThreads) return GLU_ERR_UNSUPPORTED;
            c.block = waves * glu::kWave;
            const bool two_fit = 2 * glu::mfma_hidden_lds_bytes((int)m_pl, K) <= (size_t)glu::kLdsMax;
            const int64_t per_cu = two_fit ? 2 * kMfmaWavesPerCU : kMfmaWavesPerCU;
            const int64_t grid = (t && t->grid > 0) ? t->grid : grouped8_grid(rows / 8, (int64_t)kCUs * per_cu, waves);
            c.grid = (int)(grid < 1 ? 1 : grid);
            if (!glu::grouped_mfma_supported(c)) return GLU_ERR_UNSUPPORTED;
            L->kernel = GLU_KERNEL_MFMA;
            L->mfma = c;
            L->m_per_launch = (int)m_pl;
            L->launches = (int)ceil_div(M, m_pl);
            L->accum_depth = (int)(2 * (nsegs8 + 5 + 2));
            return GLU_OK;
        }
        if (t && t->mfma_hidden) {
            c.hidden = t->mfma_hidden - 1;
        } else {
            c.hidden = glu::mfma_hidden_lds_bytes((int)m_pl, K) <= (size_t)glu::kLdsMax ? glu::kHiddenLds
                                                                                       : glu::kHiddenL2;
        }
        if (c.hidden == glu::kHiddenLds && glu::mfma_hidden_lds_bytes((int)m_pl, K) > (size_t)glu::kLdsMax) {
            return GLU_ERR_UNSUPPORTED;
        }
        // one weight stream leaves registers for 5 segments in flight per stage at every MT4 when hidden
        // sits in LDS (with MT4 x 2 hidden registers per segment, 2 when it comes from L2)
        const int dflt_u = c.hidden == glu::kHiddenL2 ? 2 : (nsegs % 5 == 0 ? 5 : 4);
        c.U = (t && t->mfma_segments) ? t->mfma_segments : dflt_u;
        if (c.U < 1) return GLU_ERR_UNSUPPORTED;
        c.nsg = (int)ceil_div(nsegs, c.U);
        c.ragged = (int64_t)c.nsg * c.U * 16 != nchunks;
        const int waves = (t && t->waves_per_block) ? t->waves_per_block : kMfmaDefaultWaves;
        if (waves < 1 || waves * glu::kWave > glu::kMfmaMaxThreads) return GLU_ERR_UNSUPPORTED;
        c.block = waves * glu::kWave;
        // 8 waves per CU where two workgroups' hidden fits one CU's LDS, else 4
        const bool two_fit = c.hidden != glu::kHiddenLds ||
                             2 * glu::mfma_hidden_lds_bytes((int)m_pl, K) <= (size_t)glu::kLdsMax;
        const int64_t per_cu = two_fit ? 2 * kMfmaWavesPerCU : kMfmaWavesPerCU;
        const int64_t grid = (t && t->grid > 0) ? t->grid
                                                : ceil_div(balanced_waves(rows / 4, (int64_t)kCUs * per_cu), waves);
        c.grid = (int)(grid < 1 ? 1 : grid);
        if (!glu::grouped_mfma_supported(c)) return GLU_ERR_UNSUPPORTED;
        L->kernel = GLU_KERNEL_MFMA;
        L->mfma = c;
        L->m_per_launch = (int)m_pl;
        L->launches = (int)ceil_div(M, m_pl);
        L->accum_depth = (int)(2 * (nsegs + 5 + 2));
        return GLU_OK;
    }
    if (forced != 0 && forced != GLU_KERNEL_VALU && forced != GLU_KERNEL_GENERIC) return GLU_ERR_UNSUPPORTED;
    const bool valu = fast && K <= kMaxValuK;
    if (forced == GLU_KERNEL_VALU && !valu) return GLU_ERR_UNSUPPORTED;
    if (valu && forced != GLU_KERNEL_GENERIC) {
        glu::ValuConfig c{};
        const int64_t nchunks = K / 8;
        const int64_t cpl = ceil_div(nchunks, glu::kWave);
        c.NB = cpl <= 8 ? 1 : 2;
        c.U = (int)ceil_div(cpl, c.NB);
        c.ragged = (int64_t)c.NB * c.U * glu::kWave != nchunks;
        int64_t m_pl = M < glu::kValuMaxM ? M : glu::kValuMaxM;
        if (glu::valu_hidden_in_lds((int)m_pl, c.U, c.NB)) {
            const int64_t m_fit = glu::kLdsBudget / (2 * K);
            m_pl = m_pl < m_fit ? m_pl : m_fit;
        }
        c.M = (int)m_pl;
        c.R = (t && t->rows_per_wave) ? t->rows_per_wave : (m_pl <= 4 ? 2 : 1);
        const int waves = (t && t->waves_per_block) ? t->waves_per_block : kValuDefaultWaves;
        if (waves < 1 || waves * glu::kWave > glu::kValuMaxThreads) return GLU_ERR_UNSUPPORTED;
        c.block = waves * glu::kWave;
        const int64_t groups = ceil_div(rows, c.R);
        const int64_t grid = (t && t->grid > 0) ? t->grid
                                                : ceil_div(balanced_waves(groups, (int64_t)kCUs * kValuWavesPerCU), waves);
        c.grid = (int)(grid < 1 ? 1 : grid);
        if (!glu::grouped_supported(c)) return GLU_ERR_UNSUPPORTED;
        glu::ValuConfig last = c;  // the last slice may be narrower: it must be instantiated too
        last.M = (int)(M - (ceil_div(M, m_pl) - 1) * m_pl);
        if (!glu::grouped_supported(last)) return GLU_ERR_UNSUPPORTED;
        L->kernel = GLU_KERNEL_VALU;
        L->valu = c;
        L->m_per_launch = (int)m_pl;
        L->launches = (int)ceil_div(M, m_pl);
        L->accum_depth = 8 * c.U * c.NB + glu::kWaveSumDepth;
        return GLU_OK;
    }
    if (t && (t->rows_per_wave || t->waves_per_block || t->grid)) return GLU_ERR_UNSUPPORTED;
    L->kernel = GLU_KERNEL_GENERIC;
    L->m_per_launch = (int)(M < 8 ? M : 8);
    L->launches = (int)ceil_div(M, L->m_per_launch);
    L->generic_grid = (int)ceil_div(rows, glu::kGroupedGenericWaves);
    L->accum_depth = (int)ceil_div(K, glu::kWave) + glu::kWaveSumDepth;
    return GLU_OK;
}

glu_status run_grouped(const uint16_t* hidden, int64_t ldh, const glu_projection* proj, int n, int64_t M,
                       int64_t K, void* stream, const glu_tuning* t)
{
    if (n < 1 || n > glu::kGroupMax) return GLU_ERR_BAD_SHAPE;
    if (!proj) return GLU_ERR_NULL_POINTER;
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim) return GLU_ERR_BAD_SHAPE;
    int64_t rows = 0;
    for (int i = 0; i < n; ++i) {
        if (proj[i].N < 0 || proj[i].N > kMaxDim) return GLU_ERR_BAD_SHAPE;
        rows += proj[i].N;
    }
    Launch L;
    glu_status st = plan_grouped(M, K, rows, false, false, false, nullptr, &L);  // shape errors first
    if (st != GLU_OK) return st;
    if (M == 0 || rows == 0) return GLU_OK;
    // strides and extents
    if (K > 0 && ldh < K) return GLU_ERR_BAD_STRIDE;
    int64_t h_len = K > 0 ? extent(M, ldh, K) : 0;
    if (h_len < 0) return GLU_ERR_BAD_STRIDE;
    int64_t w_len[glu::kGroupMax] = {}, o_len[glu::kGroupMax] = {};
    for (int i = 0; i < n; ++i) {
        const glu_projection& p = proj[i];
        if (p.N == 0) continue;
        if (p.ldo < p.N || (K > 0 && p.ldw < K)) return GLU_ERR_BAD_STRIDE;
        o_len[i] = extent(M, p.ldo, p.N);
        w_len[i] = K > 0 ? extent(p.N, p.ldw, K) : 0;
        if (o_len[i] < 0 || w_len[i] < 0) return GLU_ERR_BAD_STRIDE;
    }
    // pointers
    if (K > 0 && !hidden) return GLU_ERR_NULL_POINTER;
    uintptr_t odd = (uintptr_t)hidden, a16 = (uintptr_t)hidden;
    for (int i = 0; i < n; ++i) {
        const glu_projection& p = proj[i];
        if (p.N == 0) continue;
        if (!p.out || (K > 0 && !p.weight)) return GLU_ERR_NULL_POINTER;
        odd |= (uintptr_t)p.out | (uintptr_t)p.weight;
        a16 |= (uintptr_t)p.weight;
    }
    if (odd & 1u) return GLU_ERR_MISALIGNED;
    for (int i = 0; i < n; ++i) {
        const glu_projection& p = proj[i];
        if (p.N == 0) continue;
        if (K > 0 && overlaps(p.out, o_len[i] * 2, hidden, h_len * 2)) return GLU_ERR_ALIASING;
        for (int j = 0; j < n; ++j) {
            if (proj[j].N == 0) continue;
            if (K > 0 && overlaps(p.out, o_len[i] * 2, proj[j].weight, w_len[j] * 2)) return GLU_ERR_ALIASING;
            if (j != i && overlaps(p.out, o_len[i] * 2, proj[j].out, o_len[j] * 2)) return GLU_ERR_ALIASING;
        }
    }
    bool fast = (a16 & 15u) == 0 && K % 8 == 0 && (ldh & 7) == 0 && ldh <= kMaxFastK;
    bool mult4 = true, mult8 = true;
    glu::GroupDesc d{};
    for (int i = 0; i < n; ++i) {
        const glu_projection& p = proj[i];
        if (p.N == 0) continue;
        fast = fast && (p.ldw & 7) == 0 && p.ldw <= kMaxFastK;
        mult4 = mult4 && p.N % 4 == 0;
        mult8 = mult8 && p.N % 8 == 0;
        d.w[d.n] = p.weight;
        d.out[d.n] = p.out;
        d.ldw[d.n] = p.ldw;
        d.ldo[d.n] = p.ldo;
        d.row0[d.n] = d.rows;
        d.rows += (int)p.N;
        ++d.n;
    }
    d.row0[d.n] = d.rows;
    st = plan_grouped(M, K, rows, fast, mult4, mult8, t, &L);
    if (st != GLU_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    switch (L.kernel) {
    case GLU_KERNEL_ZERO:
        for (int i = 0; i < d.n && e == hipSuccess; ++i) {
            e = glu::zero_launch(d.out[i], M, d.row0[i + 1] - d.row0[i], d.ldo[i], s);
        }
        break;
    case GLU_KERNEL_VALU:
    case GLU_KERNEL_GENERIC:
    case GLU_KERNEL_MFMA:
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += L.m_per_launch) {
            const int mc = (int)(M - m0 < L.m_per_launch ? M - m0 : L.m_per_launch);
            glu::GroupDesc dm = d;
            for (int i = 0; i < d.n; ++i) dm.out[i] = d.out[i] + m0 * d.ldo[i];
            if (L.kernel == GLU_KERNEL_MFMA) {
                e = glu::grouped_mfma_launch(L.mfma, mc, hidden + m0 * ldh, ldh, K, dm, s);
            } else if (L.kernel == GLU_KERNEL_VALU) {
                glu::ValuConfig c = L.valu;
                c.M = mc;
                e = glu::grouped_launch(c, hidden + m0 * ldh, ldh, K, dm, s);
            } else {
                e = glu::grouped_generic_launch(mc, hidden + m0 * ldh, ldh, K, dm, s);
            }
        }
        break;
    default:
        return GLU_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? GLU_OK : fail_launch(e);
}

// ---- backward ------------------------------------------------------------------

glu_status plan_backward(int64_t M, int64_t N, int64_t K, glu::BwdPlan* bp)
{
    Launch L;
    const glu_status st = plan_launch(M, N, K, true, nullptr, &L);  // shape errors
    if (st != GLU_OK) return st;
    if (M > glu::kBwdMaxM) return GLU_ERR_UNSUPPORTED;
    *bp = glu::bwd_plan(M, N, K);
    bp->gu_fused = glu::kGuGrouped;
    bp->gu_cfg = glu::MfmaConfig{};
    // where the forward runs one MFMA launch for (M, N, K), that kernel forms dg and du in its epilogue
    // (the same G and U; one launch fewer): the slice-major 8-row kernel for 8 < M <= 64, the 4-row
    // kernel with hidden in LDS up to 16 rows
    const glu::MfmaConfig& c = L.mfma;
    const bool one_mfma = L.kernel == GLU_KERNEL_MFMA && L.launches == 1 && c.block >= glu::kWave &&
                          c.block <= glu::kMfmaMaxThreads;
    if (one_mfma && bp->path == glu::kPathMfma && !bp->gu_gemm && c.rows == 8 && c.order == glu::kOrderSlices &&
        c.hidden == glu::kHiddenSlices && c.depth == 1 && c.block == glu::kMfmaMaxThreads) {
        bp->gu_fused = glu::kGuFusedPass;
    } else if (one_mfma && (bp->path == glu::kPathChunks || (bp->path == glu::kPathMfma && !bp->gu_gemm)) &&
               glu::mfma_act_supported(c, (int)M)) {
        bp->gu_fused = glu::kGuFusedMfma4;
    }
    if (bp->gu_fused != glu::kGuGrouped) {
        bp->gu_cfg = c;
        bp->accum_depth = std::max(bp->accum_depth, L.accum_depth);
    }
    return GLU_OK;
}

glu_status run_backward(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* dout,
                        uint16_t* dh, uint16_t* dwg, uint16_t* dwu, int64_t M, int64_t N, int64_t K, void* ws,
                        int64_t ws_bytes, void* stream, bool validate_only = false)
{
    glu::BwdPlan bp;
    glu_status st = plan_backward(M, N, K, &bp);
    if (st != GLU_OK) return st;
    const int64_t hk = M * K, nk = N * K, mn = M * N;
    if ((hk > 0 && (!hidden || !dh)) || (nk > 0 && (!gate_w || !up_w || !dwg || !dwu)) || (mn > 0 && !dout)) {
        return GLU_ERR_NULL_POINTER;
    }
    const uintptr_t odd = ((uintptr_t)hidden | (uintptr_t)gate_w | (uintptr_t)up_w | (uintptr_t)dout |
                           (uintptr_t)dh | (uintptr_t)dwg | (uintptr_t)dwu) & 1u;
    if (odd) return GLU_ERR_MISALIGNED;
    // outputs (and the workspace) overlap no input and no other output
    const bool run_all = M > 0 && N > 0 && K > 0;
    const void* ins[4] = {hidden, gate_w, up_w, dout};
    const int64_t in_bytes[4] = {hk * 2, nk * 2, nk * 2, mn * 2};
    const void* outs[4] = {dh, dwg, dwu, run_all ? ws : nullptr};
    const int64_t out_bytes[4] = {hk * 2, nk * 2, nk * 2, run_all ? bp.workspace_bytes : 0};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 4; ++b) {
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return GLU_ERR_ALIASING;
            if (b > a && overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return GLU_ERR_ALIASING;
        }
    }
    const bool fast = ((((uintptr_t)hidden | (uintptr_t)gate_w | (uintptr_t)up_w | (uintptr_t)dwg | (uintptr_t)dwu) &
                        15u) == 0) && K % 8 == 0 && K <= kMaxFastK;
    if (validate_only) return (run_all && !fast) ? GLU_ERR_UNSUPPORTED : GLU_OK;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (!run_all) {
        // an empty sum is zero: dh when N == 0, the weight gradients when M == 0
        if (N == 0 && hk > 0) e = glu::zero_launch(dh, M, K, K, s);
        if (M == 0 && nk > 0 && e == hipSuccess) e = glu::zero_launch(dwg, N, K, K, s);
        if (M == 0 && nk > 0 && e == hipSuccess) e = glu::zero_launch(dwu, N, K, K, s);
        return e == hipSuccess ? GLU_OK : fail_launch(e);
    }
    if (!fast) return GLU_ERR_UNSUPPORTED;
    if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < bp.workspace_bytes) return GLU_ERR_WORKSPACE;
    uint16_t* gu = static_cast<uint16_t*>(ws);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + bp.off_partial);
    if (bp.path == glu::kPathFused1 || bp.path == glu::kPathSplitK) {
        e = bp.path == glu::kPathFused1
                ? glu::fused1_launch(bp, (int)M, hidden, gate_w, up_w, dout, gu, dwg, dwu, partial, (int)N, (int)K, s)
                : glu::splitk_launch(bp, (int)M, hidden, gate_w, up_w, dout, gu, dwg, dwu, partial, (int)N, (int)K,
                                     s);
        if (e == hipSuccess) e = glu::dh_reduce_launch(bp, partial, dh, K, (int)M, (int)K, s);
        return e == hipSuccess ? GLU_OK : fail_launch(e);
    }
    // g = bf16(h Wg^T), u = bf16(h Wu^T) into the workspace: the grouped GEMV, or above 32 rows of
    // hidden the tiled GEMM (which reads the weights once where the GEMV's 32-row slices would
    // read them once per slice)
    if (bp.gu_gemm) {
        // the elementwise step (dg, du) in the GEMM's epilogue
        e = glu::gemm_linear_launch((int)M, hidden, gate_w, up_w, gu, (int)N, (int)K, dout, s);
        if (e != hipSuccess) return fail_launch(e);
    } else if (bp.gu_fused == glu::kGuFusedPass) {
        // the same step in the epilogue of the forward's slice-major kernel
        const glu::MfmaConfig& c = bp.gu_cfg;
        e = glu::mfma8_act_launch((int)M, c.U, c.nsg, c.ragged, c.grid, hidden, gate_w, up_w, dout, gu, N, K, s);
        if (e != hipSuccess) return fail_launch(e);
    } else if (bp.gu_fused == glu::kGuFusedMfma4) {
        // and in the epilogue of the forward's 4-row kernel
        e = glu::mfma_act_launch(bp.gu_cfg, (int)M, hidden, gate_w, up_w, dout, gu, N, K, s);
        if (e != hipSuccess) return fail_launch(e);
    } else {
        glu_projection proj[2] = {{gate_w, gu, N, K, N}, {up_w, gu + mn, N, K, N}};
        st = run_grouped(hidden, K, proj, 2, M, K, stream, nullptr);
        if (st != GLU_OK) return st;
        e = glu::act_grad_launch(gu, dout, N, (int)M, (int)N, s);
    }
    const uint16_t* dg_all = gu;
    const uint16_t* du_all = gu + mn;
    if (bp.path == glu::kPathMfma || bp.path == glu::kPathGemm) {
        // zero-padded operand copies, then dh's partial sums over ranges of weight rows, their
        // reduction, and both weight gradients
        char* w = static_cast<char*>(ws);
        const int rows2 = bp.mp16 * bp.dh_mslices;  // dg2, du2 rows: hidden padded to whole tiles
        uint16_t* g2 = reinterpret_cast<uint16_t*>(w + bp.off_g2);
        uint16_t* u2 = g2 + (int64_t)rows2 * bp.np32;
        uint16_t* gT = reinterpret_cast<uint16_t*>(w + bp.off_gT);
        uint16_t* uT = gT + N * bp.mp32;
        uint16_t* hT = reinterpret_cast<uint16_t*>(w + bp.off_hT);
        const int m = (int)M, n = (int)N, k = (int)K;
        glu::RepackJobs jobs{};
        jobs.job[0] = {dg_all, N, g2, m, n, rows2, bp.np32, 0, 0, 0};
        jobs.job[1] = {du_all, N, u2, m, n, rows2, bp.np32, 0, 0, 0};
        jobs.job[2] = {dg_all, N, gT, m, n, bp.mp32, 0, 1, 0, 0};
        jobs.job[3] = {du_all, N, uT, m, n, bp.mp32, 0, 1, 0, 0};
        jobs.job[4] = {hidden, K, hT, m, k, bp.mp32, 0, 1, 0, 0};
        jobs.n = 5;
        if (e == hipSuccess) e = glu::repack_launch(jobs, s);
        if (e == hipSuccess) e = glu::dh_mfma_launch(bp, m, gate_w, up_w, g2, u2, partial, n, k, s);
        if (e == hipSuccess) e = glu::dh_reduce_launch(bp, partial, dh, K, m, k, s);
        if (e == hipSuccess) {
            e = bp.path == glu::kPathGemm ? glu::gemm_dw_launch(bp.mp32, hT, gT, uT, dwg, dwu, n, k, s)
                                          : glu::dw_mfma_launch(bp, hT, gT, uT, dwg, dwu, n, k, s);
        }
        return e == hipSuccess ? GLU_OK : fail_launch(e);
    }
    // 2 <= M <= 8: the contraction (weight gradients and dh's partial sums), then the reduction
    if (e == hipSuccess) {
        e = glu::contract_launch(bp, (int)M, hidden, gate_w, up_w, dg_all, du_all, dwg, dwu, partial, (int)N, (int)K,
                                 s);
    }
    if (e == hipSuccess) e = glu::dh_reduce_launch(bp, partial, dh, K, (int)M, (int)K, s);
    return e == hipSuccess ? GLU_OK : fail_launch(e);
}

void fill_plan(const Launch& L, glu_plan* p)
{
    p->kernel = L.kernel;
    p->m_per_launch = L.m_per_launch;
    p->launches = L.launches;
    p->accum_depth = L.accum_depth;
    switch (L.kernel) {
    case GLU_KERNEL_VALU: p->grid = L.valu.grid; p->block = L.valu.block; break;
    case GLU_KERNEL_MFMA: p->grid = L.mfma.grid; p->block = L.mfma.block; break;
    case GLU_KERNEL_GENERIC: p->grid = L.generic_grid; p->block = 4 * glu::kWave; break;
    case GLU_KERNEL_GEMM: p->grid = L.gemm_grid; p->block = 4 * glu::kWave; break;
    case GLU_KERNEL_ZERO: p->grid = 0; p->block = 256; break;
    default: p->grid = 0; p->block = 0; break;
    }
}

}  // namespace

namespace glu {

glu_status backward_entry(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* dout,
                          uint16_t* dh, uint16_t* dwg, uint16_t* dwu, int64_t M, int64_t N, int64_t K, void* ws,
                          int64_t ws_bytes, void* stream, bool validate_only)
{
    return run_backward(hidden, gate_w, up_w, dout, dh, dwg, dwu, M, N, K, ws, ws_bytes, stream, validate_only);
}

glu_status launch_failed(hipError_t e) { return fail_launch(e); }

glu_status backward_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes)
{
    BwdPlan bp;
    const glu_status st = plan_backward(M, N, K, &bp);
    *bytes = (st == GLU_OK && M > 0 && N > 0 && K > 0) ? bp.workspace_bytes : 0;
    return st;
}

}  // namespace glu

extern "C" {

glu_status glu_dual_gemv(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                         uint16_t* out, int64_t M, int64_t N, int64_t K, void* stream)
{
    return run(hidden, K, gate_w, K, up_w, K, out, N, M, N, K, stream, nullptr);
}

glu_status glu_dual_gemv_strided(const uint16_t* hidden, int64_t ldh, const uint16_t* gate_w, int64_t ldg,
                                 const uint16_t* up_w, int64_t ldu, uint16_t* out, int64_t ldo,
                                 int64_t M, int64_t N, int64_t K, void* stream)
{
    return run(hidden, ldh, gate_w, ldg, up_w, ldu, out, ldo, M, N, K, stream, nullptr);
}

glu_status glu_dual_gemv_tuned(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                               uint16_t* out, int64_t M, int64_t N, int64_t K, void* stream,
                               const glu_tuning* tuning)
{
    return run(hidden, K, gate_w, K, up_w, K, out, N, M, N, K, stream, tuning);
}

glu_status glu_dual_gemv_strided_tuned(const uint16_t* hidden, int64_t ldh, const uint16_t* gate_w, int64_t ldg,
                                       const uint16_t* up_w, int64_t ldu, uint16_t* out, int64_t ldo,
                                       int64_t M, int64_t N, int64_t K, void* stream, const glu_tuning* tuning)
{
    return run(hidden, ldh, gate_w, ldg, up_w, ldu, out, ldo, M, N, K, stream, tuning);
}

glu_status glu_grouped_gemv(const uint16_t* hidden, int64_t ldh, const glu_projection* proj, int n,
                            int64_t M, int64_t K, void* stream)
{
    return run_grouped(hidden, ldh, proj, n, M, K, stream, nullptr);
}

glu_status glu_grouped_gemv_tuned(const uint16_t* hidden, int64_t ldh, const glu_projection* proj, int n,
                                  int64_t M, int64_t K, void* stream, const glu_tuning* tuning)
{
    return run_grouped(hidden, ldh, proj, n, M, K, stream, tuning);
}

glu_status glu_grouped_gemv_plan(int64_t M, int64_t K, int64_t rows, int fast, glu_plan* plan)
{
    return glu_grouped_gemv_plan_tuned(M, K, rows, fast, nullptr, plan);
}

glu_status glu_grouped_gemv_plan_tuned(int64_t M, int64_t K, int64_t rows, int fast, const glu_tuning* tuning,
                                       glu_plan* plan)
{
    if (!plan) return GLU_ERR_NULL_POINTER;
    Launch L;
    const glu_status st = plan_grouped(M, K, rows, (fast & 1) != 0, (fast & 2) != 0, (fast & 4) != 0, tuning, &L);
    if (st != GLU_OK) return st;
    fill_plan(L, plan);
    if (L.kernel == GLU_KERNEL_GENERIC) plan->block = glu::kGroupedGenericWaves * glu::kWave;
    return GLU_OK;
}

glu_status glu_dual_gemv_plan(int64_t M, int64_t N, int64_t K, int aligned16, glu_plan* plan)
{
    return glu_dual_gemv_plan_tuned(M, N, K, aligned16, nullptr, plan);
}

glu_status glu_dual_gemv_plan_tuned(int64_t M, int64_t N, int64_t K, int aligned16,
                                    const glu_tuning* tuning, glu_plan* plan)
{
    if (!plan) return GLU_ERR_NULL_POINTER;
    Launch L;
    const glu_status st = plan_launch(M, N, K, aligned16 != 0, tuning, &L);
    if (st != GLU_OK) return st;
    fill_plan(L, plan);
    return GLU_OK;
}

namespace {

// profiler name of the kernel instance a launch plan runs first
void describe_launch(const Launch& L, bool grouped, char* buf, int len)
{
    const char* tf[2] = {"false", "true"};
    switch (L.kernel) {
    case GLU_KERNEL_VALU: {
        const glu::ValuConfig& c = L.valu;
        if (c.diag) {
            snprintf(buf, (size_t)len, "glu::valu_kernel<%d, %d, %d, %d, %s, %s, true>", c.M, c.R, c.U, c.NB,
                     tf[glu::valu_hidden_in_lds(c.M, c.U, c.NB)], tf[c.ragged]);
        } else {
            snprintf(buf, (size_t)len, "glu::%s<%d, %d, %d, %d, %s, %s>", grouped ? "grouped_kernel" : "valu_kernel",
                     c.M, c.R, c.U, c.NB, tf[glu::valu_hidden_in_lds(c.M, c.U, c.NB)], tf[c.ragged]);
        }
        break;
    }
    case GLU_KERNEL_MFMA: {
        const glu::MfmaConfig& c = L.mfma;
        if (grouped && c.rows == 8 && c.hidden == glu::kHiddenSlices) {
            snprintf(buf, (size_t)len, "glu::grouped_slice_kernel<%d, %d, %d, %s>", c.MT4, c.U, glu::kPassBlocks,
                     tf[c.ragged]);
        } else if (grouped && c.rows == 8) {
            snprintf(buf, (size_t)len, "glu::grouped_mfma_kernel<%d, %d, true, %s, 8>", c.MT4, c.U, tf[c.ragged]);
        } else if (grouped) {
            snprintf(buf, (size_t)len, "glu::grouped_mfma_kernel<%d, %d, %s, %s>", c.MT4, c.U,
                     tf[c.hidden == glu::kHiddenLds], tf[c.ragged]);
        } else if (c.hidden == glu::kHiddenSlices && c.rows == 8 && c.order == glu::kOrderSlices) {
            snprintf(buf, (size_t)len, "glu::mfma8_pass_kernel<%d, %d, %d, %s>", (4 * c.MT4 + 7) / 8, c.U,
                     glu::kPassBlocks, tf[c.ragged]);
        } else if (c.hidden == glu::kHiddenSlices && c.rows == 8) {
            snprintf(buf, (size_t)len, "glu::mfma8_slice_kernel<%d, %d, %d, %s>", (4 * c.MT4 + 7) / 8, c.U,
                     c.depth, tf[c.ragged]);
        } else if (c.hidden == glu::kHiddenSlices) {
            snprintf(buf, (size_t)len, "glu::mfma_slice_kernel<%d, %d, %d, %s>", c.MT4, c.U,
                     c.depth, tf[c.ragged]);
        } else {
            snprintf(buf, (size_t)len, "glu::mfma_kernel<%d, %d, %s, %s>", c.MT4, c.U,
                     tf[c.hidden == glu::kHiddenLds], tf[c.ragged]);
        }
        break;
    }
    case GLU_KERNEL_GENERIC:
        snprintf(buf, (size_t)len, "glu::%s<%d>", grouped ? "grouped_generic_kernel" : "generic_kernel",
                 L.m_per_launch);
        break;
    case GLU_KERNEL_GEMM:
        snprintf(buf, (size_t)len, "glu::gemm_kernel<%d, %d, %s, %d>", L.gemm.bn, L.gemm.bm, tf[L.gemm.ktail],
                 L.gemm.depth);
        break;
    case GLU_KERNEL_ZERO: snprintf(buf, (size_t)len, "glu::zero_kernel"); break;
    default: snprintf(buf, (size_t)len, "none"); break;
    }
}

}  // namespace

glu_status glu_dual_gemv_describe(int64_t M, int64_t N, int64_t K, int aligned16,
                                  const glu_tuning* tuning, char* buf, int len)
{
    if (!buf || len < 1) return GLU_ERR_NULL_POINTER;
    buf[0] = '\0';
    Launch L;
    const glu_status st = plan_launch(M, N, K, aligned16 != 0, tuning, &L);
    if (st != GLU_OK) return st;
    describe_launch(L, false, buf, len);
    return GLU_OK;
}

glu_status glu_grouped_gemv_describe(int64_t M, int64_t K, int64_t rows, int fast, const glu_tuning* tuning,
                                     char* buf, int len)
{
    if (!buf || len < 1) return GLU_ERR_NULL_POINTER;
    buf[0] = '\0';
    Launch L;
    const glu_status st = plan_grouped(M, K, rows, (fast & 1) != 0, (fast & 2) != 0, (fast & 4) != 0, tuning, &L);
    if (st != GLU_OK) return st;
    describe_launch(L, true, buf, len);
    return GLU_OK;
}

glu_status glu_dual_gemv_backward_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes)
{
    if (!bytes) return GLU_ERR_NULL_POINTER;
    *bytes = 0;
    glu::BwdPlan bp;
    const glu_status st = plan_backward(M, N, K, &bp);
    if (st != GLU_OK) return st;
    *bytes = (M > 0 && N > 0 && K > 0) ? bp.workspace_bytes : 0;
    return GLU_OK;
}

glu_status glu_dual_gemv_backward_plan(int64_t M, int64_t N, int64_t K, glu_plan* plan)
{
    if (!plan) return GLU_ERR_NULL_POINTER;
    glu::BwdPlan bp;
    const glu_status st = plan_backward(M, N, K, &bp);
    if (st != GLU_OK) return st;
    const bool run_all = M > 0 && N > 0 && K > 0;
    plan->kernel = run_all ? GLU_KERNEL_BACKWARD : ((M == 0) != (N == 0) && K > 0 ? GLU_KERNEL_ZERO : GLU_KERNEL_NONE);
    plan->m_per_launch = (int)M;
    // the grouped GEMV counts as one launch; the tiled GEMM for g and u, or the forward's MFMA kernel,
    // takes the elementwise step along
    const bool gu_one = bp.gu_gemm || bp.gu_fused != glu::kGuGrouped;  // dg and du in one launch
    plan->launches = run_all ? (bp.path == glu::kPathMfma || bp.path == glu::kPathGemm ? (gu_one ? 5 : 6)
                                : bp.path != glu::kPathChunks                         ? 2
                                                                                      : (gu_one ? 3 : 4))
                             : 0;
    plan->grid = run_all ? (bp.path == glu::kPathFused1   ? bp.fused_grid
                            : bp.path == glu::kPathSplitK ? bp.split_grid
                            : bp.path == glu::kPathMfma || bp.path == glu::kPathGemm
                                ? (int)((K + glu::dh_cols(bp.mp16 / 16) - 1) / glu::dh_cols(bp.mp16 / 16)) *
                                      bp.dh_splits * bp.dh_mslices
                                                          : bp.nranges * bp.nslabs)
                         : 0;
    plan->block = bp.path == glu::kPathSplitK ? bp.split_waves * glu::kWave : 256;
    plan->accum_depth = bp.accum_depth;
    return GLU_OK;
}

glu_status glu_dual_gemv_backward(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                                  const uint16_t* dout, uint16_t* dhidden, uint16_t* dgate_w, uint16_t* dup_w,
                                  int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                  void* stream)
{
    return run_backward(hidden, gate_w, up_w, dout, dhidden, dgate_w, dup_w, M, N, K, workspace, workspace_bytes,
                        stream);
}

glu_status glu_read_ceiling_plan(int64_t rows, int64_t row_bytes, const glu_tuning* tuning, glu_plan* plan)
{
    if (!plan) return GLU_ERR_NULL_POINTER;
    CeilingLaunch c;
    const glu_status st = plan_ceiling(rows, row_bytes, tuning, &c);
    if (st != GLU_OK) return st;
    *plan = glu_plan{};
    plan->kernel = rows > 0 ? GLU_KERNEL_CEILING : GLU_KERNEL_NONE;
    plan->m_per_launch = 0;
    plan->launches = rows > 0 ? 1 : 0;
    plan->grid = c.grid;
    plan->block = c.block;
    plan->accum_depth = 0;
    return GLU_OK;
}

glu_status glu_read_ceiling(const void* a, const void* b, int64_t rows, int64_t row_bytes, uint32_t* sink,
                            const glu_tuning* tuning, void* stream)
{
    CeilingLaunch c;
    glu_status st = plan_ceiling(rows, row_bytes, tuning, &c);
    if (st != GLU_OK) return st;
    if (rows == 0) return GLU_OK;
    if (!a || !b || !sink) return GLU_ERR_NULL_POINTER;
    if ((((uintptr_t)a | (uintptr_t)b) & 15u) != 0 || ((uintptr_t)sink & 3u) != 0) return GLU_ERR_MISALIGNED;
    const int64_t bytes = rows * row_bytes;
    if (overlaps(sink, 64 * 4, a, bytes) || overlaps(sink, 64 * 4, b, bytes)) return GLU_ERR_ALIASING;
    const hipError_t e = glu::read_ceiling_launch(a, b, (int)rows, c.U, c.R, c.grid, c.block, c.xcd_bands, sink,
                                                  (hipStream_t)stream);
    return e == hipSuccess ? GLU_OK : fail_launch(e);
}

glu_status glu_copy_ceiling(const void* a, const void* b, void* ca, void* cb, int64_t rows, int64_t row_bytes,
                            const glu_tuning* tuning, void* stream)
{
    if (tuning && (tuning->xcd_bands || tuning->rows_per_wave > 2)) return GLU_ERR_UNSUPPORTED;
    CeilingLaunch c;
    glu_status st = plan_ceiling(rows, row_bytes, tuning, &c);
    if (st != GLU_OK) return st;
    if (rows == 0) return GLU_OK;
    if (!glu::copy_ceiling_supported(c.U, c.R)) return GLU_ERR_UNSUPPORTED;
    if (!a || !b || !ca || !cb) return GLU_ERR_NULL_POINTER;
    if ((((uintptr_t)a | (uintptr_t)b | (uintptr_t)ca | (uintptr_t)cb) & 15u) != 0) return GLU_ERR_MISALIGNED;
    const int64_t bytes = rows * row_bytes;
    if (overlaps(ca, bytes, a, bytes) || overlaps(ca, bytes, b, bytes) || overlaps(cb, bytes, a, bytes) ||
        overlaps(cb, bytes, b, bytes) || overlaps(ca, bytes, cb, bytes)) {
        return GLU_ERR_ALIASING;
    }
    const hipError_t e = glu::copy_ceiling_launch(a, b, ca, cb, (int)rows, c.U, c.R, c.grid, c.block,
                                                  (hipStream_t)stream);
    return e == hipSuccess ? GLU_OK : fail_launch(e);
}

namespace {

glu_status check_unit_ceiling(int unit, int waves, int64_t workgroups, int64_t iterations)
{
    if (unit < GLU_UNIT_MFMA_16X16X32_BF16 || unit > GLU_UNIT_LDS_READ_B128) return GLU_ERR_UNSUPPORTED;
    if (waves < 1 || waves > 16 || workgroups < 1 || workgroups > 65536) return GLU_ERR_UNSUPPORTED;
    if (iterations < 1 || iterations > ((int64_t)1 << 20)) return GLU_ERR_UNSUPPORTED;
    return GLU_OK;
}

}  // namespace

glu_status glu_unit_ceiling_work(int unit, int waves_per_cu, int64_t workgroups, int64_t iterations, double* work)
{
    const glu_status st = check_unit_ceiling(unit, waves_per_cu, workgroups, iterations);
    if (st != GLU_OK) return st;
    if (!work) return GLU_ERR_NULL_POINTER;
    const double bodies = (double)workgroups * waves_per_cu * (double)iterations;
    *work = bodies * (unit == GLU_UNIT_MFMA_16X16X32_BF16 ? 8.0 * 16384.0
                      : unit == GLU_UNIT_MFMA_32X32X16_BF16 ? 4.0 * 32768.0 : 16.0 * 1024.0);
    return GLU_OK;
}

glu_status glu_unit_ceiling(int unit, int waves_per_cu, int64_t workgroups, int64_t iterations, uint32_t* sink,
                            void* stream)
{
    const glu_status st = check_unit_ceiling(unit, waves_per_cu, workgroups, iterations);
    if (st != GLU_OK) return st;
    if (!sink) return GLU_ERR_NULL_POINTER;
    if (((uintptr_t)sink & 3u) != 0) return GLU_ERR_MISALIGNED;
    const hipError_t e = glu::unit_ceiling_launch(unit, (int)workgroups, waves_per_cu, iterations, sink,
                                                  (hipStream_t)stream);
    return e == hipSuccess ? GLU_OK : fail_launch(e);
}

const char* glu_status_string(int status)
{
    switch (status) {
    case GLU_OK: return "GLU_OK";
    case GLU_ERR_NULL_POINTER: return "GLU_ERR_NULL_POINTER: a non-empty array is NULL";
    case GLU_ERR_BAD_SHAPE: return "GLU_ERR_BAD_SHAPE: negative or oversized M, N or K";
    case GLU_ERR_MISALIGNED: return "GLU_ERR_MISALIGNED: a pointer is not 2-byte aligned";
    case GLU_ERR_ALIASING: return "GLU_ERR_ALIASING: out overlaps an input";
    case GLU_ERR_LAUNCH: return "GLU_ERR_LAUNCH: the HIP kernel launch failed";
    case GLU_ERR_UNSUPPORTED: return "GLU_ERR_UNSUPPORTED: the requested launch shape is not available";
    case GLU_ERR_BAD_STRIDE: return "GLU_ERR_BAD_STRIDE: a row stride is shorter than its row, or the rows overflow";
    case GLU_ERR_WORKSPACE: return "GLU_ERR_WORKSPACE: the workspace is NULL, misaligned or too small";
    case GLU_ERR_SCRATCH_LIMIT:
        return "GLU_ERR_SCRATCH_LIMIT: the call needs more scratch than the library's fixed device array holds";
    default: return "unknown glu_status";
    }
}

int glu_last_hip_error(void) { return g_last_hip_error; }

int glu_version(void) { return 300; }

}  // extern "C"
