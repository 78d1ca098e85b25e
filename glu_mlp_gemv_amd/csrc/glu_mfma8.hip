// MFMA kernels for the dual-weight GLU projection when hidden does not fit in
// LDS: groups of 8 weight rows per wave (the planner's default above 8 rows of
// hidden, up to 64 rows per launch).
//
// Same block-diagonal use of v_mfma_f32_16x16x32_bf16 as the 4-row kernel,
// with 8 rows x 2 blocks instead of 4 rows x 4 blocks:
//
//   A[i][k] = W[8g + rho][s*64 + 32*beta + k]       i = 2*rho + beta, k < 32
//   B[k][n] = h[8t + mu][s*64 + 32*beta' + k]       n = 2*mu + beta'
//
// For a 64-element segment s the blocks beta == beta' of D are the two
// 32-element partial dots of every (weight row, hidden row) pair, so half of
// D is useful rather than a quarter, and each hidden operand read from LDS
// feeds twice the weight bytes.  Lane l supplies A row l%16 and B column l%16
// as the 8 bf16 at k = 8*(l/16): weight chunk 4*beta + l/16 of the segment,
// so one 16-byte load per lane reads 8 weight rows x 128 contiguous bytes.
// D lane l holds D[4*(l/16) + e][l%16]; the useful entries are e = l%2
// (weight row 2*(l/16)) and e = 2 + l%2 (weight row 2*(l/16) + 1), and lanes
// l and l^1 hold the two blocks of the same pairs, so one DPP addition
// finishes both dot products.
//
// The W = 4 waves of a workgroup take 4 adjacent groups (32 weight rows) and
// advance through K in lockstep, sharing each stage's K-slice of hidden
// through a double-buffered LDS ring; the weights of stage s+DW are issued at
// stage s and the slice of stage s+2 is loaded at stage s and published at
// the end of stage s+1.  Against 4 rows per wave this halves, per weight
// byte, the MFMAs, the LDS operand reads, the hidden slice traffic and (with
// 512-element stages) the barriers.  That is mfma8_slice_kernel below; the
// slice-major walk over up to 3 blocks per workgroup (mfma8_pass_kernel, the
// default above 8 rows of hidden) is in glu_mfma8_pass.h, which the backward
// instantiates too.
#include "glu_device.h"
#include "glu_mfma8_pass.h"
#include "glu_mfma_common.h"

namespace glu {

// MT8: hidden-row tiles of 8 (M <= 8*MT8); U: 64-element segments per stage;
// DW: stages of weights in flight; nsg: stages per group (nsg*U*8 >= K/8).
// Dynamic LDS: 2 * 8*MT8 * U*8 * 16 bytes.  blockDim.x == 256.
template <int MT8, int U, int DW, bool RAGGED>
__global__ void __launch_bounds__(kMfmaMaxThreads)
mfma8_slice_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
                   const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
                   int M, int N, int K, RowStrides ld, int nsg)
{
    const int64_t ldo = ld.o;
    const uint32_t ldh8 = (uint32_t)(ld.h >> 3), ldg8 = (uint32_t)(ld.g >> 3), ldu8 = (uint32_t)(ld.u >> 3);
    constexpr int W = kMfmaMaxThreads / kWave;             // waves in lockstep
    constexpr int MP = 8 * MT8;                            // hidden rows in a slice (padded)
    constexpr int SC = U * 8;                              // 16-byte chunks of one row in a slice
    static_assert(SC % 16 == 0, "the LDS swizzle permutes 16-chunk blocks of a row");
    constexpr int HPT = (MP * SC + kMfmaMaxThreads - 1) / kMfmaMaxThreads;  // slice loads per thread
    constexpr int NB = DW + 1;                             // weight stages held in registers
    constexpr int L = NB % 2 == 0 ? NB : 2 * NB;           // unrolled stages: buffer and parity static
    constexpr int AHEAD = DW > 2 ? DW : 2;                 // farthest prefetch, in stages
    extern __shared__ u32x4_t hs[];                        // [2][MP][SC], chunk c of row r at c ^ lds_swz8(r)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int nchunks = K >> 3;
    const int i16 = lane & 15;
    const int rho = i16 >> 1;                   // weight row (A) and hidden row (B) of this lane, in its group / tile
    const int cw = (i16 & 1) * 4 + (lane >> 4);  // 16-byte chunk within a 128-byte segment
    const u32x4_t* h4 = reinterpret_cast<const u32x4_t*>(hidden);

    const int ngroups = (N + 7) / 8;
    const int nblocks = (ngroups + W - 1) / W;
    if ((int)blockIdx.x >= nblocks) return;  // whole workgroup
    const int my_blocks = (nblocks - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    const int nstages = my_blocks * nsg;  // the same for every wave of the workgroup

    auto group_of = [&](int s) __attribute__((always_inline)) {
        return ((int)blockIdx.x + (s / nsg) * (int)gridDim.x) * W + wave;
    };

    auto load_h = [&](int s, u32x4_t (&hr)[HPT]) __attribute__((always_inline)) {
        const int sb = s % nsg;
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
            const int e = min(i * kMfmaMaxThreads + (int)threadIdx.x, MP * SC - 1);
            const int m = min(e / SC, M - 1);  // padded rows repeat row M-1, never stored
            int c = sb * SC + (e % SC);
            if (RAGGED) c = min(c, nchunks - 1);
            hr[i] = h4[(uint32_t)m * ldh8 + (uint32_t)c];
        }
    };
    auto store_h = [&](int s, const u32x4_t (&hr)[HPT]) __attribute__((always_inline)) {
        u32x4_t* dst = hs + (s & 1) * MP * SC;
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
            const int e = i * kMfmaMaxThreads + (int)threadIdx.x;
            // XOR swizzle: the rows one read touches land in different banks
            if ((MP * SC) % kMfmaMaxThreads == 0 || e < MP * SC) dst[e ^ lds_swz8(e / SC)] = hr[i];
        }
    };
    auto load_w = [&](int s, u32x4_t (&A)[2][U]) __attribute__((always_inline)) {
        const int sb = s % nsg;
        // waves past the last group (a group count that is not a multiple of W)
        // re-read the last group, never stored
        const int g = min(group_of(s), ngroups - 1);
        const int64_t row0 = 8 * (int64_t)g;  // wave-uniform base, 32-bit lane offsets
        const uint32_t rr = (uint32_t)(min(8 * g + rho, N - 1) - 8 * g);  // 0..7: rows past N re-read row N-1
        const char* gp = reinterpret_cast<const char*>(gate_w + row0 * ld.g);
        const char* up = reinterpret_cast<const char*>(up_w + row0 * ld.u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = (sb * U + u) * 8 + cw;
            if (RAGGED) c = min(c, nchunks - 1);
            // bytes, below 8 rows at the stride
            const uint32_t offg = (rr * ldg8 + (uint32_t)c) * 16u, offu = (rr * ldu8 + (uint32_t)c) * 16u;
            A[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(gp + offg));
            A[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(up + offu));
        }
    };

    f32x4_t acc[MT8][2];

    auto finish_group = [&](int g) __attribute__((always_inline)) {
        // lane l keeps weight row 8g + 2*(l/16) + l%2 of hidden row 8t + (l%16)/2
        const bool odd = (lane & 1) != 0;
        float res[2][MT8];
#pragma unroll
        for (int t = 0; t < MT8; ++t) {
#pragma unroll
            for (int gu = 0; gu < 2; ++gu) {
                const f32x4_t d = acc[t][gu];
                float v0 = odd ? d[1] : d[0];  // weight row 2*(l/16), block l%2
                float v1 = odd ? d[3] : d[2];  // weight row 2*(l/16) + 1, block l%2
                v0 = dpp_add<0xB1>(v0);        // + the other block, from lane l^1
                v1 = dpp_add<0xB1>(v1);
                res[gu][t] = odd ? v1 : v0;
            }
        }
        const int row = 8 * g + 2 * (lane >> 4) + (lane & 1);
#pragma unroll
        for (int t = 0; t < MT8; ++t) {
            const int m = 8 * t + (i16 >> 1);
            if (m < M && row < N) out[(int64_t)m * ldo + row] = glu_epilogue(res[0][t], res[1][t]);
        }
    };

    auto compute = [&](int s, const u32x4_t (&A)[2][U]) __attribute__((always_inline)) {
        const int sb = s % nsg;
        if (sb == 0) {
#pragma unroll
            for (int t = 0; t < MT8; ++t) {
                acc[t][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                acc[t][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        const u32x4_t* src = hs + (s & 1) * MP * SC;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        // all MT8 hidden operands of a segment are read before its MFMAs
        u32x4_t b[2][MT8];
        auto read_b = [&](int u, u32x4_t (&bt)[MT8]) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < MT8; ++t) bt[t] = src[(8 * t + rho) * SC + ((u * 8 + cw) ^ lds_swz8(rho))];
        };
        read_b(0, b[0]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u + 1 < U) read_b(u + 1, b[(u + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);  // the next segment's reads stay ahead of these MFMAs
            const bool ok = !RAGGED || (sb * U + u) * 8 + cw < nchunks;
            const u32x4_t ag = RAGGED ? (ok ? A[0][u] : z) : A[0][u];
            const u32x4_t au = RAGGED ? (ok ? A[1][u] : z) : A[1][u];
#pragma unroll
            for (int t = 0; t < MT8; ++t) {
                u32x4_t bt = b[u & 1][t];
                if constexpr (RAGGED) bt = ok ? bt : z;
                acc[t][0] = mfma16(ag, bt, acc[t][0]);
                acc[t][1] = mfma16(au, bt, acc[t][1]);
            }
        }
        if (sb == nsg - 1) finish_group(group_of(s));
    };

    u32x4_t A[NB][2][U];  // weights of stage s live in A[s % NB]
    u32x4_t hr[2][HPT];   // hidden slice of stage s lives in hr[s % 2] from stage s-2 to s-1

    // stage s at unrolled position Q = s % L: prefetch, compute, publish, wait.
    // In the steady state (TAIL false) every prefetch is live and nothing
    // branches around a load, so the waits can leave all prefetches in flight.
    auto stage = [&](auto Qc, auto tailc, int s) __attribute__((always_inline)) {
        constexpr int Q = decltype(Qc)::value;
        constexpr bool TAIL = decltype(tailc)::value;
        if (!TAIL || s + 2 < nstages) load_h(s + 2, hr[Q % 2]);          // hr[s % 2] was published at s-1
        if (!TAIL || s + DW < nstages) load_w(s + DW, A[(Q + DW) % NB]);  // consumed at s-1
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any of this stage's math
        compute(s, A[Q % NB]);
        if (!TAIL || s + 1 < nstages) store_h(s + 1, hr[(Q + 1) % 2]);
        __syncthreads();
    };
    auto steady = [&](auto Qc, int s) __attribute__((always_inline)) { stage(Qc, std::false_type{}, s); };
    auto tail = [&](auto Qc, int s) __attribute__((always_inline)) { stage(Qc, std::true_type{}, s); };

    load_h(0, hr[0]);
    if (1 < nstages) load_h(1, hr[1]);
#pragma unroll
    for (int j = 0; j < DW; ++j) {
        if (j < nstages) load_w(j, A[j]);
    }
    store_h(0, hr[0]);
    __syncthreads();
    int s0 = 0;
    for (; s0 + L + AHEAD <= nstages; s0 += L) run_stages<0, L>(steady, s0, nstages);
    for (; s0 < nstages; s0 += L) run_stages<0, L>(tail, s0, nstages);
}

namespace {

using Mfma8Fn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int, RowStrides, int);

// 8 < M <= 32: stages of 8 segments (512 elements); 32 < M <= 64: stages of 4 (256 elements), which
// keep the accumulators of 3 blocks and 8 tiles of hidden rows within the registers
Mfma8Fn pick_pass(int mt8, int U, bool ragged)
{
    if (U == 8) {
        switch (mt8) {
        case 2: return ragged ? mfma8_pass_kernel<2, 8, kPassBlocks, true> : mfma8_pass_kernel<2, 8, kPassBlocks, false>;
        case 3: return ragged ? mfma8_pass_kernel<3, 8, kPassBlocks, true> : mfma8_pass_kernel<3, 8, kPassBlocks, false>;
        case 4: return ragged ? mfma8_pass_kernel<4, 8, kPassBlocks, true> : mfma8_pass_kernel<4, 8, kPassBlocks, false>;
        default: return nullptr;
        }
    }
    if (U == 4) {
        switch (mt8) {
        case 5: return ragged ? mfma8_pass_kernel<5, 4, kPassBlocks, true> : mfma8_pass_kernel<5, 4, kPassBlocks, false>;
        case 6: return ragged ? mfma8_pass_kernel<6, 4, kPassBlocks, true> : mfma8_pass_kernel<6, 4, kPassBlocks, false>;
        case 7: return ragged ? mfma8_pass_kernel<7, 4, kPassBlocks, true> : mfma8_pass_kernel<7, 4, kPassBlocks, false>;
        case 8: return ragged ? mfma8_pass_kernel<8, 4, kPassBlocks, true> : mfma8_pass_kernel<8, 4, kPassBlocks, false>;
        default: return nullptr;
        }
    }
    return nullptr;
}

template <int MT8, bool RG>
Mfma8Fn pick8_u(int U, int depth)
{
    // 8 or 16 segments (16 or 32 KiB per wave) of weights in flight
    if (U == 4 && depth == 2) return mfma8_slice_kernel<MT8, 4, 2, RG>;
    if (U == 4 && depth == 4) return mfma8_slice_kernel<MT8, 4, 4, RG>;
    if (U == 8 && depth == 1) return mfma8_slice_kernel<MT8, 8, 1, RG>;
    if (U == 8 && depth == 2) return mfma8_slice_kernel<MT8, 8, 2, RG>;
    return nullptr;
}

Mfma8Fn pick8(int mt8, int U, int depth, bool ragged)
{
    switch (mt8) {
    case 1: return ragged ? pick8_u<1, true>(U, depth) : pick8_u<1, false>(U, depth);
    case 2: return ragged ? pick8_u<2, true>(U, depth) : pick8_u<2, false>(U, depth);
    case 3: return ragged ? pick8_u<3, true>(U, depth) : pick8_u<3, false>(U, depth);
    case 4: return ragged ? pick8_u<4, true>(U, depth) : pick8_u<4, false>(U, depth);
    default: return nullptr;
    }
}

}  // namespace

size_t mfma8_slice_lds_bytes(int mt8, int u) { return (size_t)2 * 8 * mt8 * u * 8 * 16; }

int mfma8_slice_depth(int u) { return u == 4 ? 2 : u == 8 ? 1 : 0; }  // the default

bool mfma8_supported(int mt8, int U, int depth, bool ragged, int block, int order)
{
    if (block != kMfmaMaxThreads) return false;
    if (mfma8_slice_lds_bytes(mt8, U) > (size_t)kLdsBudget) return false;
    if (order == kOrderSlices) return depth == 1 && pick_pass(mt8, U, ragged) != nullptr;
    return order == kOrderBlocks && pick8(mt8, U, depth, ragged) != nullptr;
}

int64_t mfma8_blocks(int64_t N) { return ((N + 7) / 8 + kMfmaMaxThreads / kWave - 1) / (kMfmaMaxThreads / kWave); }

hipError_t mfma8_launch(int M, int U, int depth, int order, int nsg, bool ragged, int grid, const uint16_t* hidden,
                        const uint16_t* gate_w, const uint16_t* up_w, uint16_t* out, int64_t N, int64_t K,
                        RowStrides ld, hipStream_t stream)
{
    if (order == kOrderSlices) {
        const int mt8 = pass_tiles(M, U);
        // the slice-major kernel serves at most kPassBlocks blocks per workgroup
        Mfma8Fn fp = nullptr;
        if (depth == 1 && (int64_t)grid * kPassBlocks >= mfma8_blocks(N)) fp = pick_pass(mt8, U, ragged);
        if (!fp || M < 1 || M > 8 * mt8) return hipErrorInvalidValue;
        hipLaunchKernelGGL(fp, dim3(grid), dim3(kMfmaMaxThreads), mfma8_slice_lds_bytes(mt8, U), stream,
                           hidden, gate_w, up_w, out, M, (int)N, (int)K, ld, nsg);
        return hipGetLastError();
    }
    const int mt8 = (M + 7) / 8;
    Mfma8Fn fn = order == kOrderBlocks ? pick8(mt8, U, depth, ragged) : nullptr;
    if (!fn || M < 1 || M > 8 * mt8) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kMfmaMaxThreads), mfma8_slice_lds_bytes(mt8, U), stream,
                       hidden, gate_w, up_w, out, M, (int)N, (int)K, ld, nsg);
    return hipGetLastError();
}

}  // namespace glu
