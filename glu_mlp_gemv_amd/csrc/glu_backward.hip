// Backward of the dual-weight GLU projection (up to 65536 rows of hidden per call).
//
// The segKI "Plan B" autograd Function keeps hidden, gate_w and up_w and
// returns gradients for all three, equal to those of the composite
// silu(h Wg^T) * (h Wu^T) (DeepSpeed PR #8602, comment "Plan B: Dual-Weight
// GEMV", sections "Plan B Design" and "Verification Results").  Over bf16 tensors every gradient tensor is
// rounded once to bf16, as autograd of the bf16 composite does:
//   ds = bf16(dout u), du = bf16(dout s), dg = bf16(silu'(g) ds) in fp32,
//   dh = bf16(fp32(bf16(dg Wg) + bf16(du Wu))), dWg = bf16(dg^T h), dWu = bf16(du^T h).
//
// M <= 2 with K <= 2560: one pass (fused1_kernel, below) reads each row of Wg
// and Wu once, forms G and U, dg and du, writes the row of dWg and dWu and
// accumulates dh, then dh_reduce_kernel adds the workgroups' partials.
// M <= 2 with 2560 < K <= 8192, and M = 3 or 4 with 3584 < K <= 4096: also one pass
// (splitk_kernel), K split over the lanes of a workgroup so that each lane
// keeps its columns of dh for all M rows in registers, then dh_reduce_kernel.
// Above M = 8 the contractions run on the matrix cores (glu_backward_mfma.hip).
// Otherwise, 2 <= M <= 8, four launches (after the grouped GEMV has written
// g = bf16(h Wg^T) and u = bf16(h Wu^T) into the workspace):
//  * act_grad_kernel: dg and du from g, u and dout, elementwise, in place;
//  * contract_kernel: workgroups own (row range, 512-column slab) tiles.  Each
//    wave streams its rows' 1 KiB slab pieces of Wg and Wu once, accumulates
//    dh's two contributions for the slab in fp32 registers, and writes the
//    same rows' slab of dWg and dWu (sum over the M rows of hidden, in order).
//    The 4 waves' dh sums are added in LDS in a fixed order and written as the
//    workgroup's fp32 partial;
//  * dh_reduce_kernel: sums the row ranges' partials in a fixed order (16 lane
//    groups over interleaved ranges, then the groups in order), rounds each
//    contribution and their fp32 sum to bf16 (dh_reduce_flat_kernel: the same
//    order with one lane per element group, for 16 ranges or fewer).
// No atomics: results are bitwise reproducible.
#include <algorithm>

#include "glu_backward.h"
#include "glu_device.h"
#include "glu_launch.h"
#include "glu_mfma_common.h"

namespace glu {

namespace {

constexpr int kSlab = 512;          // columns per contraction tile (8 per lane)
constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * kWave;
constexpr int kRowsPerIter = 4;     // weight rows whose loads a wave issues together
constexpr int kReduceCols = 16;     // 4-element groups of dh per reduction workgroup
constexpr int kReduceParts = 16;    // lane groups splitting the row ranges of one element
constexpr int kReduceFlatThreads = 256;  // the reduction with one lane per 4 elements (<= 16 ranges)
constexpr int64_t kReduceFlatMinElems = 131072;  // M * K from which that reduction is taken

typedef unsigned u32x4_b __attribute__((ext_vector_type(4)));


}  // namespace

// gu: [2][M][N] bf16, g then u on entry, dg then du on return; dout [M][ldd]
__global__ void __launch_bounds__(256)
act_grad_kernel(uint16_t* __restrict__ gu, const uint16_t* __restrict__ dout, int64_t ldd, int M, int N)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t MN = (int64_t)M * N;
    if (i >= MN) return;
    const int64_t m = i / N;
    const int64_t j = i - m * N;
    const float g = bf16_to_f32(gu[i]);
    const float u = bf16_to_f32(gu[MN + i]);
    const float go = bf16_to_f32(dout[m * ldd + j]);
    uint16_t dg, du;
    glu_act_grad(g, u, go, &dg, &du);
    gu[i] = dg;
    gu[MN + i] = du;
}

// M: rows of hidden (1..8).  Workgroup b: slab b % nslabs, rows
// [r * rows_per_range, min(N, (r + 1) * rows_per_range)) with r = b / nslabs.
// dgm, dum: dg and du of these M rows ([M][N]).  partial: [nranges][2][M][K] fp32.  Also the
// weight gradients: the same rows' slab of dWg and dWu.
template <int M>
__global__ void __launch_bounds__(kBwdThreads)
contract_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
                const uint16_t* __restrict__ up_w, const uint16_t* __restrict__ dgm, const uint16_t* __restrict__ dum,
                uint16_t* __restrict__ dwg, uint16_t* __restrict__ dwu, float* __restrict__ partial, int N, int K,
                int nslabs, int rows_per_range)
{
    __shared__ float red[2 * M * kSlab];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slab = blockIdx.x % nslabs;
    const int range = blockIdx.x / nslabs;
    const int c0 = slab * kSlab + lane * 8;
    const bool col_ok = c0 < K;  // K % 8 == 0: a lane's 8 columns are all inside or all outside
    const int j_begin = range * rows_per_range;
    const int j_end = min(j_begin + rows_per_range, N);

    // this lane's 8 columns of every row of hidden, as packed bf16 pairs (widened where used)
    u32x4_b hw[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        hw[m] = u32x4_b{0u, 0u, 0u, 0u};
        if (col_ok) hw[m] = *reinterpret_cast<const u32x4_b*>(hidden + (int64_t)m * K + c0);
    }
    float ag[M][8], au[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ag[m][e] = 0.0f;
            au[m][e] = 0.0f;
        }
    }

    // rows j0 + 4i (i < RPI) per iteration: their loads are issued together (fewer rows from
    // M = 4, where the dh accumulators take most of the registers; K=2560 N=9216, whole backward:
    // M = 4 75.9 -> 73.7 us with 2 rows instead of 4, M = 3 72.4 against 73.2 with 4)
    constexpr int RPI = M <= 3 ? kRowsPerIter : (M <= 6 ? kRowsPerIter / 2 : 1);
    for (int j0 = j_begin + wave; j0 < j_end; j0 += kBwdWaves * RPI) {
        u32x4_b wgv[RPI], wuv[RPI];
        float dg[RPI][M], du[RPI][M];
#pragma unroll
        for (int i = 0; i < RPI; ++i) {
            const int j = min(j0 + kBwdWaves * i, j_end - 1);  // past the range: re-read a valid row, unused
#pragma unroll
            for (int m = 0; m < M; ++m) {
                dg[i][m] = bf16_to_f32(dgm[(int64_t)m * N + j]);
                du[i][m] = bf16_to_f32(dum[(int64_t)m * N + j]);
            }
            if (col_ok) {
                wgv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_b*>(gate_w + (int64_t)j * K + c0));
                wuv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_b*>(up_w + (int64_t)j * K + c0));
            } else {
                wgv[i] = u32x4_b{0u, 0u, 0u, 0u};
                wuv[i] = u32x4_b{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < RPI; ++i) {
            const int j = j0 + kBwdWaves * i;
            if (j >= j_end) break;  // wave-uniform
            float wgf[8], wuf[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wgf[2 * q] = bf16lo(wgv[i][q]);
                wgf[2 * q + 1] = bf16hi(wgv[i][q]);
                wuf[2 * q] = bf16lo(wuv[i][q]);
                wuf[2 * q + 1] = bf16hi(wuv[i][q]);
            }
            // dh contributions (a product of two bf16 values is exact in fp32, so fma adds it unrounded)
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ag[m][e] = __builtin_fmaf(dg[i][m], wgf[e], ag[m][e]);
                    au[m][e] = __builtin_fmaf(du[i][m], wuf[e], au[m][e]);
                }
            }
            if (!col_ok) continue;
            // this row's slab of dWg and dWu: sums over the rows of hidden in order
            u32x4_b pg, pu;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint16_t og[2], ou[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    float sg = 0.0f, su = 0.0f;
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float hme = h2 ? bf16hi(hw[m][q]) : bf16lo(hw[m][q]);
                        sg = __builtin_fmaf(dg[i][m], hme, sg);
                        su = __builtin_fmaf(du[i][m], hme, su);
                    }
                    og[h2] = f32_to_bf16_rne(sg);
                    ou[h2] = f32_to_bf16_rne(su);
                }
                pg[q] = (uint32_t)og[0] | ((uint32_t)og[1] << 16);
                pu[q] = (uint32_t)ou[0] | ((uint32_t)ou[1] << 16);
            }
            __builtin_nontemporal_store(pg, reinterpret_cast<u32x4_b*>(dwg + (int64_t)j * K + c0));
            __builtin_nontemporal_store(pu, reinterpret_cast<u32x4_b*>(dwu + (int64_t)j * K + c0));
        }
    }

    // the waves' dh sums, added in the order 3, 2, 1, 0
    const int base = lane * 8;
    for (int w = kBwdWaves - 1; w >= 0; --w) {
        if (wave == w) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ig = m * kSlab + base + e;
                    const int iu = (M + m) * kSlab + base + e;
                    const float vg = (w == kBwdWaves - 1) ? ag[m][e] : red[ig] + ag[m][e];
                    const float vu = (w == kBwdWaves - 1) ? au[m][e] : red[iu] + au[m][e];
                    if (w > 0) {
                        red[ig] = vg;
                        red[iu] = vu;
                    } else if (col_ok) {
                        float* pg = partial + (((int64_t)range * 2 + 0) * M + m) * K + c0;
                        float* pu = partial + (((int64_t)range * 2 + 1) * M + m) * K + c0;
                        pg[e] = vg;
                        pu[e] = vu;
                    }
                }
            }
        }
        __syncthreads();
    }
}

// One pass for M <= 4 with K split over the lanes of a workgroup: W waves (W = blockDim / 64),
// lane t owns 16-byte chunks t + 64 W u (u < U) of every row.  Workgroup b owns the rows
// [b * rpb, min(N, (b + 1) * rpb)), taken kSplitRows at a time with the next rows' loads issued
// first.  Per batch: each wave's partial dot products (wave butterfly) go to LDS; lanes
// t < rows * M add the W wave sums in order, form (dg, du) for one (row, m) each and share them
// through LDS (and the workspace head); then every lane writes its columns of the rows of dWg and
// dWu and accumulates its columns of dh, which it writes as the workgroup's partial at the end.
template <int M, int U, bool HLDS>
__global__ void __launch_bounds__(kSplitMaxThreads)
splitk_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
              const uint16_t* __restrict__ up_w, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dgu,
              uint16_t* __restrict__ dwg, uint16_t* __restrict__ dwu, float* __restrict__ partial, int N, int K,
              int rpb)
{
    constexpr int R = split_rows(M, U);
    __shared__ float wsum[kSplitMaxWaves][R][M][2];
    __shared__ float gsh[R][M][2];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int W = blockDim.x / kWave;
    const int nchunks = K >> 3;
    const int j_begin = blockIdx.x * rpb;
    const int j_end = min(j_begin + rpb, N);
    const int64_t MN = (int64_t)M * N;

    // hidden: this lane's chunks in registers, or (HLDS) in LDS at [m][chunk], where only the lane
    // that owns a chunk writes it
    extern __shared__ u32x4_b hsh[];
    int cidx[U];
    bool ok[U];
    u32x4_b hw[HLDS ? 1 : M][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = t + kWave * W * u;
        ok[u] = c < nchunks;
        cidx[u] = ok[u] ? c : nchunks - 1;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const u32x4_b v = ok[u] ? *reinterpret_cast<const u32x4_b*>(hidden + (int64_t)m * K + (int64_t)c * 8)
                                    : u32x4_b{0u, 0u, 0u, 0u};
            if constexpr (HLDS) {
                if (ok[u]) hsh[m * nchunks + c] = v;
            } else {
                hw[m][u] = v;
            }
        }
    }
    if constexpr (HLDS) __syncthreads();  // lanes past K read the last chunk, written by another wave
    auto H = [&](int m, int u) __attribute__((always_inline)) -> u32x4_b {
        if constexpr (HLDS) {
            return hsh[m * nchunks + cidx[u]];
        } else {
            return hw[m][u];
        }
    };
    float ag[M][U][8], au[M][U][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ag[m][u][e] = 0.0f;
                au[m][u][e] = 0.0f;
            }
        }
    }

    // a batch's loads (rows past the range re-read the range's last row; they are never used)
    auto load = [&](int j0, u32x4_b (&wg)[R][U], u32x4_b (&wu)[R][U]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t j = min(j0 + r, j_end - 1);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                wg[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_b*>(gate_w + j * K + cidx[u] * 8));
                wu[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_b*>(up_w + j * K + cidx[u] * 8));
            }
        }
    };
    auto batch = [&](int j0, u32x4_b (&wg)[R][U], u32x4_b (&wu)[R][U]) __attribute__((always_inline)) {
        // partial dots of this lane's chunks, summed over the wave
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!ok[u]) {
                    wg[r][u] = u32x4_b{0u, 0u, 0u, 0u};
                    wu[r][u] = u32x4_b{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float pg = 0.0f, pu = 0.0f;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const u32x4_b hv = H(m, u);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        pg = __builtin_fmaf(bf16lo(hv[q]), bf16lo(wg[r][u][q]), pg);
                        pg = __builtin_fmaf(bf16hi(hv[q]), bf16hi(wg[r][u][q]), pg);
                        pu = __builtin_fmaf(bf16lo(hv[q]), bf16lo(wu[r][u][q]), pu);
                        pu = __builtin_fmaf(bf16hi(hv[q]), bf16hi(wu[r][u][q]), pu);
                    }
                }
                pg = wave_sum(pg);
                pu = wave_sum(pu);
                if (lane == 0) {
                    wsum[wave][r][m][0] = pg;
                    wsum[wave][r][m][1] = pu;
                }
            }
        }
        __syncthreads();
        // (row, m) pairs: the wave sums in order, then the gradient step
        if (t < R * M) {
            const int r = t / M, m = t - (t / M) * M;
            const int j = j0 + r;
            float G = 0.0f, Uv = 0.0f;
            for (int w = 0; w < W; ++w) {
                G += wsum[w][r][m][0];
                Uv += wsum[w][r][m][1];
            }
            uint16_t dgb = 0, dub = 0;
            if (j < j_end) {
                glu_act_grad(bf16_to_f32(f32_to_bf16_rne(G)), bf16_to_f32(f32_to_bf16_rne(Uv)),
                         bf16_to_f32(dout[(int64_t)m * N + j]), &dgb, &dub);
                dgu[(int64_t)m * N + j] = dgb;
                dgu[MN + (int64_t)m * N + j] = dub;
            }
            gsh[r][m][0] = bf16_to_f32(dgb);
            gsh[r][m][1] = bf16_to_f32(dub);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int j = j0 + r;
            if (j >= j_end) break;  // uniform over the workgroup
            // (dg, du) are the same in every lane: scalar registers
            float dg[M], du[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                dg[m] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gsh[r][m][0])));
                du[m] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gsh[r][m][1])));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float wgf[8], wuf[8];
                float sg[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};  // +0: sums of zeros are +0
                float su[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    wgf[2 * q] = bf16lo(wg[r][u][q]);
                    wgf[2 * q + 1] = bf16hi(wg[r][u][q]);
                    wuf[2 * q] = bf16lo(wu[r][u][q]);
                    wuf[2 * q + 1] = bf16hi(wu[r][u][q]);
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const u32x4_b hv = H(m, u);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float h0 = bf16lo(hv[q]), h1 = bf16hi(hv[q]);
                        // the weights' gradients add the M rows in order
                        sg[2 * q] = __builtin_fmaf(dg[m], h0, sg[2 * q]);
                        sg[2 * q + 1] = __builtin_fmaf(dg[m], h1, sg[2 * q + 1]);
                        su[2 * q] = __builtin_fmaf(du[m], h0, su[2 * q]);
                        su[2 * q + 1] = __builtin_fmaf(du[m], h1, su[2 * q + 1]);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ag[m][u][e] = __builtin_fmaf(dg[m], wgf[e], ag[m][u][e]);
                        au[m][u][e] = __builtin_fmaf(du[m], wuf[e], au[m][u][e]);
                    }
                }
                u32x4_b og, ou;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    og[q] = (uint32_t)f32_to_bf16_rne(sg[2 * q]) | ((uint32_t)f32_to_bf16_rne(sg[2 * q + 1]) << 16);
                    ou[q] = (uint32_t)f32_to_bf16_rne(su[2 * q]) | ((uint32_t)f32_to_bf16_rne(su[2 * q + 1]) << 16);
                }
                if (ok[u]) {
                    __builtin_nontemporal_store(og, reinterpret_cast<u32x4_b*>(dwg + (int64_t)j * K + cidx[u] * 8));
                    __builtin_nontemporal_store(ou, reinterpret_cast<u32x4_b*>(dwu + (int64_t)j * K + cidx[u] * 8));
                }
            }
        }
    };

    u32x4_b ga[R][U], ua[R][U], gb[R][U], ub[R][U];
    int j0 = j_begin;
    if (j0 < j_end) load(j0, ga, ua);
    while (j0 < j_end) {
        const int j1 = j0 + R;
        load(j1 < j_end ? j1 : j0, gb, ub);
        batch(j0, ga, ua);
        if (j1 >= j_end) break;
        const int j2 = j1 + R;
        load(j2 < j_end ? j2 : j1, ga, ua);
        batch(j1, gb, ub);
        j0 = j2;
    }
    // this lane's columns of the workgroup's dh partial
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float* pg = partial + (((int64_t)blockIdx.x * 2 + 0) * M + m) * K + (int64_t)cidx[u] * 8;
            float* pu = partial + (((int64_t)blockIdx.x * 2 + 1) * M + m) * K + (int64_t)cidx[u] * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pg[e] = ag[m][u][e];
                pu[e] = au[m][u][e];
            }
        }
    }
}

// One pass for M <= 2 rows of hidden (K <= 64 * 8 * U): wave w owns weight rows w, w + W, ... (W
// waves in the grid).  Lane l holds 16-byte chunks l, l + 64, ... of its row of Wg and Wu and of every
// row of hidden.  Per weight row j: G and U for each hidden row m (at M = 1 the diagonal of one
// MFMA per 512-element piece of the row, at M = 2 fp32 fma per lane; then the wave butterfly); dg and du (act_grad; above M = 1 lane m forms row m's pair and readlane hands it to
// the wave, lanes 0 .. M-1 store them at the workspace head); the row of dWg and dWu (the M products
// dg[m] h[m] added in order, one rounding); and dh's two contributions accumulated per lane.  The
// workgroup's waves then add their dh sums in LDS in order 0, 1, ..., and the sum becomes the
// workgroup's partial: partial[b][2][M][K].
template <int M, int U, int WAVES>
__global__ void __launch_bounds__(WAVES * kWave, fused1_hidden_in_lds(M, U) ? 2 : 1)
fused1_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
              const uint16_t* __restrict__ up_w, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dgu,
              uint16_t* __restrict__ dwg, uint16_t* __restrict__ dwu, float* __restrict__ partial, int N, int K)
{
    // HLDS: the row of hidden sits in LDS after red1 and each use reads the lane's chunk there: 20
    // registers fewer (256 at K = 2560; K=2560 N=9216, whole backward 49.4 -> 48.6 us at one wave
    // per SIMD; two waves per SIMD, which these registers would allow, measured 53.9 us)
    constexpr bool HLDS = fused1_hidden_in_lds(M, U);
    extern __shared__ float red1[];  // [2][M][K], then (HLDS) hidden's K / 8 chunks
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * WAVES + wave);
    const int nwaves = gridDim.x * WAVES;
    const int nchunks = K >> 3;
    const int64_t MN = (int64_t)M * N, MK = (int64_t)M * K;

    constexpr int HR = HLDS ? 1 : M, HU = HLDS ? 1 : U;
    u32x4_b hw[HR][HU];
    u32x4_b* const hl = reinterpret_cast<u32x4_b*>(red1 + 2 * MK);
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = lane + kWave * u;
        ok[u] = c < nchunks;
        if constexpr (!HLDS) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                hw[m][u] = ok[u] ? *reinterpret_cast<const u32x4_b*>(hidden + (int64_t)m * K + (int64_t)c * 8)
                                 : u32x4_b{0u, 0u, 0u, 0u};
            }
        }
    }
    if constexpr (HLDS) {
        for (int c = (int)threadIdx.x; c < kWave * U; c += WAVES * kWave) {
            hl[c] = c < nchunks ? *reinterpret_cast<const u32x4_b*>(hidden + (int64_t)c * 8) : u32x4_b{0u, 0u, 0u, 0u};
        }
        __syncthreads();
    }
    // chunk u of hidden row m for this lane
    auto hid = [&](int m, int u) __attribute__((always_inline)) -> u32x4_b {
        if constexpr (HLDS) {
            return hl[lane + kWave * u];
        } else {
            return hw[m][u];
        }
    };
    float ag[M][U][8], au[M][U][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ag[m][u][e] = 0.0f;
                au[m][u][e] = 0.0f;
            }
        }
    }

    // a row's loads: its chunks of Wg and Wu and its upstream gradients (issued together, so waiting
    // for one row never waits for the next row's prefetch)
    auto load_row = [&](int j, u32x4_b (&wg)[U], u32x4_b (&wu)[U], uint16_t (&go)[M]) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < M; ++m) go[m] = dout[(int64_t)m * N + j];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = min(lane + kWave * u, nchunks - 1);  // past K: re-read a valid chunk, zeroed below
            wg[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_b*>(gate_w + (int64_t)j * K + c * 8));
            wu[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_b*>(up_w + (int64_t)j * K + c * 8));
        }
    };
    auto process = [&](int j, u32x4_b (&wg)[U], u32x4_b (&wu)[U], const uint16_t (&go)[M]) __attribute__((always_inline)) {
        float pg[M], pu[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            pg[m] = 0.0f;
            pu[m] = 0.0f;
        }
        // one row of hidden: the dot products on the matrix cores, as the forward's M = 1 GEMV
        // takes them (each 512-element piece of the row dotted by the diagonal of one
        // v_mfma_f32_16x16x32_bf16; lane l holds D[4(l/16) + e][l%16], the diagonal entry in lanes
        // with l%16 / 4 == l/16 at e = l%4, zeros elsewhere for the butterfly)
        f32x4_t dgm = {0.0f, 0.0f, 0.0f, 0.0f}, dum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4_b z = {0u, 0u, 0u, 0u};
            const u32x4_b g4 = ok[u] ? wg[u] : z;
            const u32x4_b u4 = ok[u] ? wu[u] : z;
            wg[u] = g4;
            wu[u] = u4;
            if constexpr (M == 1) {
                const u32x4_b h = hid(0, u);
                dgm = mfma16(g4, h, dgm);
                dum = mfma16(u4, h, dum);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        pg[m] = __builtin_fmaf(bf16lo(hw[m][u][q]), bf16lo(g4[q]), pg[m]);
                        pg[m] = __builtin_fmaf(bf16hi(hw[m][u][q]), bf16hi(g4[q]), pg[m]);
                        pu[m] = __builtin_fmaf(bf16lo(hw[m][u][q]), bf16lo(u4[q]), pu[m]);
                        pu[m] = __builtin_fmaf(bf16hi(hw[m][u][q]), bf16hi(u4[q]), pu[m]);
                    }
                }
            }
        }
        if constexpr (M == 1) {
            const int e = lane & 3;
            const bool on = ((lane & 15) >> 2) == (lane >> 4);
            const float vg = e == 0 ? dgm[0] : (e == 1 ? dgm[1] : (e == 2 ? dgm[2] : dgm[3]));
            const float vu = e == 0 ? dum[0] : (e == 1 ? dum[1] : (e == 2 ? dum[2] : dum[3]));
            pg[0] = on ? vg : 0.0f;
            pu[0] = on ? vu : 0.0f;
        }
        float dg[M], du[M];
        if constexpr (M == 1) {
            const float G = wave_sum(pg[0]);
            const float Uv = wave_sum(pu[0]);
            uint16_t dgb, dub;
            glu_act_grad(bf16_to_f32(f32_to_bf16_rne(G)), bf16_to_f32(f32_to_bf16_rne(Uv)), bf16_to_f32(go[0]), &dgb,
                     &dub);
            if (lane == 0) {
                dgu[j] = dgb;
                dgu[N + j] = dub;
            }
            dg[0] = bf16_to_f32(dgb);
            du[0] = bf16_to_f32(dub);
        } else {
            // lane m takes hidden row m's sums and upstream gradient, forms its (dg, du) and stores it;
            // readlane then hands every row's pair to the whole wave
            float Gm = 0.0f, Um = 0.0f;
            uint16_t gom = 0;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float G = wave_sum(pg[m]);
                const float Uv = wave_sum(pu[m]);
                Gm = lane == m ? G : Gm;
                Um = lane == m ? Uv : Um;
                gom = lane == m ? go[m] : gom;
            }
            uint16_t dgb = 0, dub = 0;
            if (lane < M) {
                glu_act_grad(bf16_to_f32(f32_to_bf16_rne(Gm)), bf16_to_f32(f32_to_bf16_rne(Um)), bf16_to_f32(gom), &dgb,
                         &dub);
                dgu[(int64_t)lane * N + j] = dgb;
                dgu[MN + (int64_t)lane * N + j] = dub;
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                dg[m] = bf16_to_f32((uint16_t)__builtin_amdgcn_readlane((int)dgb, m));
                du[m] = bf16_to_f32((uint16_t)__builtin_amdgcn_readlane((int)dub, m));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4_b og, ou;
            u32x4_b hu[M];
#pragma unroll
            for (int m = 0; m < M; ++m) hu[m] = hid(m, u);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // the weights' gradients add the M products in order from +0
                float g0 = 0.0f, g1 = 0.0f, u0 = 0.0f, u1 = 0.0f;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const float h0 = bf16lo(hu[m][q]), h1 = bf16hi(hu[m][q]);
                    g0 = __builtin_fmaf(dg[m], h0, g0);
                    g1 = __builtin_fmaf(dg[m], h1, g1);
                    u0 = __builtin_fmaf(du[m], h0, u0);
                    u1 = __builtin_fmaf(du[m], h1, u1);
                    ag[m][u][2 * q] = __builtin_fmaf(dg[m], bf16lo(wg[u][q]), ag[m][u][2 * q]);
                    ag[m][u][2 * q + 1] = __builtin_fmaf(dg[m], bf16hi(wg[u][q]), ag[m][u][2 * q + 1]);
                    au[m][u][2 * q] = __builtin_fmaf(du[m], bf16lo(wu[u][q]), au[m][u][2 * q]);
                    au[m][u][2 * q + 1] = __builtin_fmaf(du[m], bf16hi(wu[u][q]), au[m][u][2 * q + 1]);
                }
                og[q] = pack_bf16x2_rne(g0, g1);
                ou[q] = pack_bf16x2_rne(u0, u1);
            }
            if (ok[u]) {
                const int c = lane + kWave * u;
                __builtin_nontemporal_store(og, reinterpret_cast<u32x4_b*>(dwg + (int64_t)j * K + c * 8));
                __builtin_nontemporal_store(ou, reinterpret_cast<u32x4_b*>(dwu + (int64_t)j * K + c * 8));
            }
        }
    };

    // the next row's loads are issued before this row is processed (two register sets alternate);
    // past the wave's last row the prefetch re-reads the current row, so no load sits behind a branch
    // (a second row in flight measured slower at M = 1: 50.5 against 48.0 us at K=2560 N=9216)
    u32x4_b ga[U], ua[U], gb[U], ub[U];
    uint16_t oa[M], ob[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        oa[m] = 0;
        ob[m] = 0;
    }
    int j = gw;
    if (j < N) load_row(j, ga, ua, oa);
    while (j < N) {
        const int j1 = j + nwaves;
        load_row(j1 < N ? j1 : j, gb, ub, ob);
        process(j, ga, ua, oa);
        if (j1 >= N) break;
        const int j2 = j1 + nwaves;
        load_row(j2 < N ? j2 : j1, ga, ua, oa);
        process(j1, gb, ub, ob);
        j = j2;
    }

    // the waves' dh sums in order 0, 1, ..., WAVES - 1
    for (int w = 0; w < WAVES; ++w) {
        if (wave == w) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!ok[u]) continue;
                    const int64_t c = (int64_t)m * K + (lane + kWave * u) * 8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float vg = w == 0 ? ag[m][u][e] : red1[c + e] + ag[m][u][e];
                        const float vu = w == 0 ? au[m][u][e] : red1[MK + c + e] + au[m][u][e];
                        if (w + 1 < WAVES) {
                            red1[c + e] = vg;
                            red1[MK + c + e] = vu;
                        } else {
                            partial[((int64_t)blockIdx.x * 2 + 0) * MK + c + e] = vg;
                            partial[((int64_t)blockIdx.x * 2 + 1) * MK + c + e] = vu;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

// dh[m][c] = bf16(fp32(bf16(sum Pg) + bf16(sum Pu))) over the row ranges' partials.  A lane
// owns 4 consecutive elements (16-byte loads); lane group p sums ranges p, p + 16, p + 32, ... in
// order, then group 0 adds the 16 group sums in order 0..15.  M * K % 4 == 0 (K % 8 == 0).
__global__ void __launch_bounds__(kReduceCols * kReduceParts)
dh_reduce_kernel(const float* __restrict__ partial, uint16_t* __restrict__ dh, int64_t ldh_out, int M, int K,
                 int nranges)
{
    typedef float f32x4_b __attribute__((ext_vector_type(4)));
    __shared__ f32x4_b part[2][kReduceParts][kReduceCols];
    const int col = threadIdx.x % kReduceCols;
    const int grp = threadIdx.x / kReduceCols;
    const int64_t MK = (int64_t)M * K;
    const int64_t i4 = (int64_t)blockIdx.x * kReduceCols + col;  // index of 4 elements
    const bool ok = i4 * 4 < MK;
    f32x4_b sg = {0.0f, 0.0f, 0.0f, 0.0f}, su = {0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
        const f32x4_b* p4 = reinterpret_cast<const f32x4_b*>(partial);
        const int64_t MK4 = MK / 4;
#pragma unroll 4
        for (int r = grp; r < nranges; r += kReduceParts) {
            sg += p4[((int64_t)r * 2 + 0) * MK4 + i4];
            su += p4[((int64_t)r * 2 + 1) * MK4 + i4];
        }
    }
    part[0][grp][col] = sg;
    part[1][grp][col] = su;
    __syncthreads();
    if (grp != 0 || !ok) return;
    f32x4_b tg = part[0][0][col], tu = part[1][0][col];
#pragma unroll
    for (int p = 1; p < kReduceParts; ++p) {
        tg += part[0][p][col];
        tu += part[1][p][col];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i4 * 4 + e;
        const int64_t m = i / K;
        const int64_t c = i - m * K;
        const float a = bf16_to_f32(f32_to_bf16_rne(tg[e]));
        const float b = bf16_to_f32(f32_to_bf16_rne(tu[e]));
        dh[m * ldh_out + c] = f32_to_bf16_rne(a + b);
    }
}

// The same sums for nranges <= kReduceParts, one lane per 4 elements: ranges 0, 1, ... added in order
// to +0.  dh_reduce_kernel adds them in the same order (each lane group holds +0 plus at most one
// range, and the groups are added in order); the +0 it puts before each range changes only a -0
// range, and a running sum that is never -0 absorbs a +0 or a -0 alike, so the bits agree.
__global__ void __launch_bounds__(kReduceFlatThreads)
dh_reduce_flat_kernel(const float* __restrict__ partial, uint16_t* __restrict__ dh, int64_t ldh_out, int M, int K,
                      int nranges)
{
    typedef float f32x4_b __attribute__((ext_vector_type(4)));
    const int64_t MK = (int64_t)M * K;
    const int64_t i4 = (int64_t)blockIdx.x * kReduceFlatThreads + threadIdx.x;  // index of 4 elements
    if (i4 * 4 >= MK) return;
    const f32x4_b* p4 = reinterpret_cast<const f32x4_b*>(partial);
    const int64_t MK4 = MK / 4;
    f32x4_b sg = {0.0f, 0.0f, 0.0f, 0.0f}, su = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int r = 0; r < nranges; ++r) {
        sg += p4[((int64_t)r * 2 + 0) * MK4 + i4];
        su += p4[((int64_t)r * 2 + 1) * MK4 + i4];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i4 * 4 + e;
        const int64_t m = i / K;
        const int64_t c = i - m * K;
        const float a = bf16_to_f32(f32_to_bf16_rne(sg[e]));
        const float b = bf16_to_f32(f32_to_bf16_rne(su[e]));
        dh[m * ldh_out + c] = f32_to_bf16_rne(a + b);
    }
}

namespace {

using ContractFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                            uint16_t*, uint16_t*, float*, int, int, int, int);

ContractFn pick_contract(int M)
{
    switch (M) {
    case 1: return contract_kernel<1>;
    case 2: return contract_kernel<2>;
    case 3: return contract_kernel<3>;
    case 4: return contract_kernel<4>;
    case 5: return contract_kernel<5>;
    case 6: return contract_kernel<6>;
    case 7: return contract_kernel<7>;
    case 8: return contract_kernel<8>;
    default: return nullptr;
    }
}



}  // namespace

BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K)
{
    BwdPlan p{};
    p.nslabs = (int)((K + kSlab - 1) / kSlab);
    if (p.nslabs < 1) p.nslabs = 1;
    int64_t ranges = (kBwdTargetBlocks + p.nslabs - 1) / p.nslabs;
    if (ranges > N) ranges = N;
    if (ranges < 1) ranges = 1;
    p.rows_per_range = (int)((N + ranges - 1) / ranges);
    if (p.rows_per_range < 1) p.rows_per_range = 1;
    p.nranges = (int)((N + p.rows_per_range - 1) / p.rows_per_range);
    if (p.nranges < 1) p.nranges = 1;
    // one pass for M <= 2 and K <= 64 * 8 * kFusedMaxU: workgroups of kFusedWaves waves, about
    // fused_waves_per_cu waves per CU, each wave the same number of rows to within one
    p.fused = M >= 1 && M <= kFusedMaxM && K >= 8 && (K / 8 + kWave - 1) / kWave <= fused_max_u((int)M);
    p.path = p.fused ? kPathFused1 : kPathChunks;
    int64_t rows_per_wave = 0;
    // split over K: K / 8 chunks over at most 8 waves of 1 or 2 chunks per lane.  Above 2 rows only
    // at one chunk per lane on all 8 waves (3584 < K <= 4096): elsewhere the four-launch path, whose
    // g and u step is the forward's 4-row kernel with the elementwise step as its epilogue, is faster
    // (K=3072 N=9216 M = 3 / 4: 79.3 / 80.8 us against 94.3 / 93.7; K=8192 N=4096 M = 3: 87.2
    // against 106.1), while at K = 4096 the split pass holds (N=12288 M = 4: 118.9 against 128.9)
    const int64_t nch = K / 8;
    const int64_t split_cap = (int64_t)kSplitMaxWaves * kWave * (M <= kSplitMaxM2 ? 2 : 1);
    const bool split_shape = M <= 2 || (nch > (int64_t)(kSplitMaxWaves - 1) * kWave && nch <= (int64_t)kSplitMaxWaves * kWave);
    if (!p.fused && M >= 1 && M <= kSplitMaxM && K >= kSplitMinK && nch <= split_cap && split_shape) {
        p.path = kPathSplitK;
        p.split_u = nch <= (int64_t)kSplitMaxWaves * kWave ? 1 : 2;
        p.split_waves = (int)((nch + (int64_t)kWave * p.split_u - 1) / ((int64_t)kWave * p.split_u));
        p.split_rpb = N > 0 ? (int)((N + kCUsForPlan - 1) / kCUsForPlan) : 1;  // about one workgroup per CU
        p.split_grid = (int)((N + p.split_rpb - 1) / p.split_rpb);
        p.nranges = p.split_grid;  // one partial of dh per workgroup
    }
    if (p.fused) {
        const int64_t target = (int64_t)kCUsForPlan * fused_waves_per_cu((int)M, (int)((K / 8 + kWave - 1) / kWave));
        rows_per_wave = N > 0 ? (N + target - 1) / target : 1;
        const int64_t waves = (N + rows_per_wave - 1) / rows_per_wave;
        p.fused_grid = (int)((waves + kFusedWaves - 1) / kFusedWaves);
        p.nranges = p.fused_grid;  // the reduction sums one partial per workgroup
    }
    auto pad256 = [](int64_t b) { return (b + 255) / 256 * 256; };
    p.gu_bytes = pad256((int64_t)2 * M * N * 2);
    int64_t mfma_bytes = 0;  // the MFMA path's operand copies
    if (M >= kBwdMfmaMinM && M <= kBwdMaxM && N > 0 && K >= 8) {
        const bool big = M > kBwdMfmaMaxM;
        p.path = big ? kPathGemm : kPathMfma;
        // dh's B operand: 1, 2 or 4 tiles of 16 rows (4 waves split evenly), above 64 rows slices of
        // 8 tiles (two per wave: each weight tile read from beyond L2 half as often as with slices of
        // 64)
        p.mp16 = M <= 16 ? 16 : (M <= 32 ? 32 : (M <= 64 ? 64 : (M <= 128 ? 128 : 256)));
        p.dh_mslices = big ? (int)((M + p.mp16 - 1) / p.mp16) : 1;
        p.mp32 = (int)((M + 31) / 32 * 32);
        p.np32 = (int)((N + 31) / 32 * 32);
        // about 512 workgroups of dh_cols columns x one range of rows (x one slice of hidden), ranges a
        // multiple of 32 rows
        const int64_t ktiles = (K + dh_cols(p.mp16 / 16) - 1) / dh_cols(p.mp16 / 16);
        const int64_t steps_all = p.np32 / 32;
        const int64_t per_split = ktiles * p.dh_mslices;
        // (above 64 rows at most that many: the 128-row kernel fits two workgroups per CU, and a second
        // round for a few would cost a whole step loop)
        // (slices of 256 rows hold one workgroup per CU: at most half as many)
        const int64_t target = p.mp16 > 128 ? kBwdTargetBlocks / 2 : kBwdTargetBlocks;
        int64_t splits = big ? target / per_split : (target + per_split - 1) / per_split;
        splits = splits < 1 ? 1 : (splits > steps_all ? steps_all : splits);
        const int64_t steps = (steps_all + splits - 1) / splits;
        p.dh_jr = (int)(steps * 32);
        p.dh_splits = (int)((N + p.dh_jr - 1) / p.dh_jr);
        p.dh_steps = (int)steps;
        // g and u: the grouped GEMV's K-slice kernel takes up to 64 rows of hidden in one launch when
        // N % 8 == 0; the tiled GEMM above that (and above 32 rows when only N % 4 == 0)
        p.gu_gemm = N % 4 == 0 && (M > 64 || (M > 32 && N % 8 != 0));
        p.nranges = p.dh_splits;
        p.off_g2 = p.gu_bytes;
        p.off_gT = p.off_g2 + pad256((int64_t)2 * p.mp16 * p.dh_mslices * p.np32 * 2);
        p.off_hT = p.off_gT + pad256((int64_t)2 * N * p.mp32 * 2);
        p.off_partial = p.off_hT + pad256((int64_t)K * p.mp32 * 2);
        mfma_bytes = p.off_partial - p.gu_bytes;
    } else {
        p.off_partial = p.gu_bytes;
    }
    p.partial_bytes = (int64_t)p.nranges * 2 * M * K * 4;  // every path keeps dh partials for all M rows
    p.workspace_bytes = p.gu_bytes + mfma_bytes + p.partial_bytes;
    // dh: within a wave its rows in order, then the waves of a workgroup, then every 16th partial,
    // then the 16 group sums
    const int reduce_depth = (p.nranges + kReduceParts - 1) / kReduceParts + kReduceParts;
    // the one-pass kernels also form G and U: a lane's 8 U products in order, the wave's
    // butterfly, then (K split) the waves of the workgroup in order
    if (p.path == kPathFused1) {
        // G and U: at M = 2 a lane's 8 products per chunk then the butterfly; at M = 1 one MFMA per
        // chunk-set (a 32-product tree, counted at twice the unit roundoff) then the butterfly
        const int u = (int)((K / 8 + kWave - 1) / kWave);
        const int gu_depth = M == 1 ? 2 * (u + 5) + 6 : 8 * u + 6;
        p.accum_depth = std::max((int)(rows_per_wave + kFusedWaves) + reduce_depth, gu_depth);
    } else if (p.path == kPathSplitK) {
        p.accum_depth = std::max(p.split_rpb + reduce_depth, 8 * p.split_u + 6 + p.split_waves);
    } else if (p.path == kPathMfma) {
        // each MFMA adds a 32-product block (a tree of depth 5) to its accumulator, counted at twice
        // the fp32 unit roundoff as the forward's MFMA kernels are: dh over a range's steps, then
        // the reduction; dW over one or two blocks of the M rows
        p.accum_depth = std::max(2 * (p.dh_steps + 5) + reduce_depth, 2 * (p.mp32 / 32 + 5));
        // g and u from the GEMM: one MFMA per 32-element block of K, plus the tile's fixed steps; from
        // the grouped GEMV: one MFMA per 64-element segment (at most), the pair sum and the tree
        p.accum_depth = std::max(p.accum_depth, p.gu_gemm ? (int)(2 * ((K + 31) / 32 + 6))
                                                          : (int)(2 * ((K + 63) / 64 + 7)));
    } else if (p.path == kPathGemm) {
        // dh as above; the weight gradients from the GEMM over the mp32 padded rows of hidden
        p.accum_depth = std::max(2 * (p.dh_steps + 5) + reduce_depth, 2 * (p.mp32 / 32 + 6));
        if (p.gu_gemm) p.accum_depth = std::max(p.accum_depth, (int)(2 * ((K + 31) / 32 + 6)));
    } else {
        p.accum_depth = (p.rows_per_range + kBwdWaves - 1) / kBwdWaves + kBwdWaves + reduce_depth;
    }
    return p;
}

hipError_t act_grad_launch(uint16_t* gu, const uint16_t* dout, int64_t ldd, int M, int N, hipStream_t stream)
{
    const int64_t n = (int64_t)M * N;
    if (n <= 0) return hipSuccess;
    const int64_t grid = (n + 255) / 256;
    hipLaunchKernelGGL(act_grad_kernel, dim3((unsigned)grid), dim3(256), 0, stream, gu, dout, ldd, M, N);
    return hipGetLastError();
}

hipError_t contract_launch(const BwdPlan& p, int M, const uint16_t* hidden, const uint16_t* gate_w,
                           const uint16_t* up_w, const uint16_t* dgm, const uint16_t* dum, uint16_t* dwg,
                           uint16_t* dwu, float* partial, int N, int K, hipStream_t stream)
{
    ContractFn fn = pick_contract(M);
    if (!fn || N < 1 || K < 8 || (K & 7) != 0) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)p.nranges * p.nslabs;
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kBwdThreads), 0, stream, hidden, gate_w, up_w, dgm, dum, dwg,
                       dwu, partial, N, K, p.nslabs, p.rows_per_range);
    return hipGetLastError();
}

hipError_t fused1_launch(const BwdPlan& p, int M, const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                        const uint16_t* dout, uint16_t* dgu, uint16_t* dwg, uint16_t* dwu, float* partial, int N, int K,
                        hipStream_t stream)
{
    using Fn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, uint16_t*,
                        uint16_t*, float*, int, int);
    static const Fn table[kFusedMaxM][kFusedMaxU] = {
        {fused1_kernel<1, 1, kFusedWaves>, fused1_kernel<1, 2, kFusedWaves>, fused1_kernel<1, 3, kFusedWaves>,
         fused1_kernel<1, 4, kFusedWaves>, fused1_kernel<1, 5, kFusedWaves>},
        {fused1_kernel<2, 1, kFusedWaves>, fused1_kernel<2, 2, kFusedWaves>, fused1_kernel<2, 3, kFusedWaves>,
         fused1_kernel<2, 4, kFusedWaves>, fused1_kernel<2, 5, kFusedWaves>},
    };
    const int U = (K / 8 + kWave - 1) / kWave;
    if (!p.fused || M < 1 || M > kFusedMaxM || U < 1 || U > fused_max_u(M) || (K & 7) != 0 || N < 1 ||
        p.fused_grid < 1) {
        return hipErrorInvalidValue;
    }
    const size_t lds = (size_t)2 * M * K * sizeof(float) + (fused1_hidden_in_lds(M, U) ? (size_t)kWave * U * 16 : 0);
    if (lds > (size_t)kLdsBudget) return hipErrorInvalidValue;
    hipLaunchKernelGGL(table[M - 1][U - 1], dim3(p.fused_grid), dim3(kFusedWaves * kWave), lds, stream, hidden,
                       gate_w, up_w, dout, dgu, dwg, dwu, partial, N, K);
    return hipGetLastError();
}

hipError_t splitk_launch(const BwdPlan& p, int M, const uint16_t* hidden, const uint16_t* gate_w,
                         const uint16_t* up_w, const uint16_t* dout, uint16_t* dgu, uint16_t* dwg, uint16_t* dwu,
                         float* partial, int N, int K, hipStream_t stream)
{
    using Fn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, uint16_t*,
                        uint16_t*, float*, int, int, int);
    // hidden in LDS where M U chunks would not fit beside the accumulators
    static const Fn table[2][kSplitMaxM] = {
        {splitk_kernel<1, 1, false>, splitk_kernel<2, 1, false>, splitk_kernel<3, 1, false>,
         splitk_kernel<4, 1, false>},
        {splitk_kernel<1, 2, false>, splitk_kernel<2, 2, true>, splitk_kernel<3, 2, true>, nullptr},
    };
    if (p.path != kPathSplitK || M < 1 || M > kSplitMaxM || p.split_u < 1 || p.split_u > 2 ||
        (p.split_u == 2 && M > kSplitMaxM2) || p.split_waves < 1 ||
        p.split_waves > kSplitMaxWaves || (int64_t)p.split_waves * kWave * p.split_u * 8 < K || (K & 7) != 0 ||
        p.split_grid < 1 || p.split_rpb < 1) {
        return hipErrorInvalidValue;
    }
    const Fn fn = table[p.split_u - 1][M - 1];
    const bool hlds = p.split_u == 2 && M >= 2;
    const size_t lds = hlds ? (size_t)M * K * 2 : 0;
    if (lds > (size_t)kLdsMax - 4096) return hipErrorInvalidValue;
    if (lds > 48 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(p.split_grid), dim3(p.split_waves * kWave), lds, stream, hidden, gate_w, up_w, dout,
                       dgu, dwg, dwu, partial, N, K, p.split_rpb);
    return hipGetLastError();
}

hipError_t dh_reduce_launch(const BwdPlan& p, const float* partial, uint16_t* dh, int64_t ldh_out, int M, int K,
                            hipStream_t stream)
{
    const int64_t n = (int64_t)M * K;
    if (n <= 0) return hipSuccess;
    if (p.nranges < 1) return hipErrorInvalidValue;
    if (p.nranges <= kReduceParts && n >= kReduceFlatMinElems) {
        // one lane per 4 elements, where that is enough lanes: the 16 lane groups would hold at most
        // one range each (K=2560 N=9216, M = 512: 33.3 -> 6.6 us; M = 64: 7.7 -> 6.6; at M = 16 the
        // 10240 lanes took 5.9 against 4.7)
        const int64_t grid = (n / 4 + kReduceFlatThreads - 1) / kReduceFlatThreads;
        if (grid > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL(dh_reduce_flat_kernel, dim3((unsigned)grid), dim3(kReduceFlatThreads), 0, stream, partial,
                           dh, ldh_out, M, K, p.nranges);
        return hipGetLastError();
    }
    const int64_t grid = (n / 4 + kReduceCols - 1) / kReduceCols;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dh_reduce_kernel, dim3((unsigned)grid), dim3(kReduceCols * kReduceParts), 0, stream, partial,
                       dh, ldh_out, M, K, p.nranges);
    return hipGetLastError();
}

}  // namespace glu
