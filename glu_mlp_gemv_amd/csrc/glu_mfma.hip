// MFMA kernel for the dual-weight GLU projection at batch 2 <= M <= 32.
//
// The pages route small batches to a tensor-core fused GLU kernel and larger
// ones to a library GEMM (DeepSpeed PR #9057, commit notes on the Ampere GLU
// routing and the WMMA fused kernel kept for small M).  On gfx950 the product
// stays bound by streaming the weights from HBM, and how the weights are read
// decides the speed: a wave has to stream whole weight rows, neighbouring
// waves neighbouring rows, in full 128-byte lines.  The usual MFMA operand
// layout (16 weight rows x 64 bytes per load) breaks both rules, so this
// kernel feeds v_mfma_f32_16x16x32_bf16 a block-diagonal problem instead:
//
//   A[i][k] = W[4g + rho][s*128 + 32*beta + k]      i = 4*rho + beta, k < 32
//   B[k][n] = h[4t + mu][s*128 + 32*beta' + k]      n = 4*mu + beta'
//   D[i][n] = sum over k of A[i][k] * B[k][n]
//
// For a 128-element segment s of 4 weight rows and 4 hidden rows, the
// diagonal blocks beta == beta' of D are the four 32-element partial dots of
// every (weight row, hidden row) pair; the other 3/4 of D is discarded.  Lane
// l supplies A row l%16 and B column l%16 as the 8 bf16 at k = 8*(l/16), so
// one 16-byte load per lane reads 4 weight rows x 256 contiguous bytes, and
// accumulating D over all segments of K sums every block.  D lane l holds
// D[4*(l/16) + e][l%16]: the useful entry is e = l%4, and the four lanes of a
// quad hold the four blocks of one pair (weight row 4g + l/16, hidden row
// 4t + (l%16)/4), so two DPP additions finish the dot products.
//
// A wave owns groups of 4 weight rows (persistent: groups w, w+W, ...) and
// streams a group in stages of U segments; the loads of stage s+1 are issued
// before the MFMAs of stage s.  hidden [M,K] is staged in LDS when it fits in
// 64 KiB, else read from L2 with each stage's weights.  MFMA work is 1/4 useful, which still
// leaves the matrix cores far from busy at M <= 32.  That walk (mfma_body, wrapped by mfma_kernel)
// is in glu_mfma4.h, which the backward instantiates too.
#include "glu_device.h"
#include "glu_mfma4.h"
#include "glu_mfma_common.h"

namespace glu {

// The same block-diagonal product when hidden does not fit in LDS: the W = 4
// waves of a workgroup take the 4 adjacent row groups of a block and advance
// through K in lockstep, one stage of U segments at a time, and the workgroup
// keeps only the K-slice of hidden that a stage needs (all M rows) in a
// double-buffered LDS ring.  What keeps HBM busy is the depth of the weight
// pipeline: the weights of stage s+DW are issued at stage s (DW*U segments,
// 2*DW*U KiB per wave, in flight), and the hidden slice of stage s+2 is
// loaded at stage s and written to LDS at the end of stage s+1, so neither
// the L2 latency of hidden nor the HBM latency of the weights sits between
// two stages.  One barrier per stage separates the slice writes from reads.
// Dynamic LDS: 2 * 4*MT4 * U*16 * 16 bytes.  blockDim.x == 256.
template <int MT4, int U, int DW, bool RAGGED>
__global__ void __launch_bounds__(kMfmaMaxThreads)
mfma_slice_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
                  const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
                  int M, int N, int K, RowStrides ld, int nsg)
{
    const int64_t ldo = ld.o;
    const uint32_t ldh8 = (uint32_t)(ld.h >> 3), ldg8 = (uint32_t)(ld.g >> 3), ldu8 = (uint32_t)(ld.u >> 3);
    constexpr int W = kMfmaMaxThreads / kWave;             // waves in lockstep
    constexpr int MP = 4 * MT4;                            // hidden rows in a slice (padded)
    constexpr int SC = U * 16;                             // 16-byte chunks of one row in a slice
    constexpr int HPT = (MP * SC + kMfmaMaxThreads - 1) / kMfmaMaxThreads;  // slice loads per thread
    constexpr int NB = DW + 1;                             // weight stages held in registers
    constexpr int L = NB % 2 == 0 ? NB : 2 * NB;           // unrolled stages: buffer and parity static
    constexpr int AHEAD = DW > 2 ? DW : 2;                 // farthest prefetch, in stages
    extern __shared__ u32x4_t hs[];                        // [2][MP][SC], chunk c of row r at c ^ lds_swz4(r)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int nchunks = K >> 3;
    const int i16 = lane & 15;
    const int rho_a = i16 >> 2;
    const int cseg = (i16 & 3) * 4 + (lane >> 4);
    const u32x4_t* h4 = reinterpret_cast<const u32x4_t*>(hidden);

    const int ngroups = (N + 3) / 4;
    const int nblocks = (ngroups + W - 1) / W;
    if ((int)blockIdx.x >= nblocks) return;  // whole workgroup
    const int my_blocks = (nblocks - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    const int nstages = my_blocks * nsg;  // the same for every wave of the workgroup

    auto group_of = [&](int s) __attribute__((always_inline)) { return ((int)blockIdx.x + (s / nsg) * (int)gridDim.x) * W + wave; };

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
            if ((MP * SC) % kMfmaMaxThreads == 0 || e < MP * SC) dst[e ^ lds_swz4(e / SC)] = hr[i];
        }
    };
    auto load_w = [&](int s, u32x4_t (&A)[2][U]) __attribute__((always_inline)) {
        const int sb = s % nsg;
        // the last workgroup's waves can sit past the last group when the group
        // count is not a multiple of W: they re-read the last group, never stored
        const int g = min(group_of(s), ngroups - 1);
        const int64_t row0 = 4 * (int64_t)g;  // wave-uniform base, 32-bit lane offsets
        const uint32_t rr = (uint32_t)(min(4 * g + rho_a, N - 1) - 4 * g);  // 0..3: rows past N re-read row N-1
        const char* gp = reinterpret_cast<const char*>(gate_w + row0 * ld.g);
        const char* up = reinterpret_cast<const char*>(up_w + row0 * ld.u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = (sb * U + u) * 16 + cseg;
            if (RAGGED) c = min(c, nchunks - 1);
            // bytes, below 4 rows at the stride
            const uint32_t offg = (rr * ldg8 + (uint32_t)c) * 16u, offu = (rr * ldu8 + (uint32_t)c) * 16u;
            A[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(gp + offg));
            A[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(up + offu));
        }
    };

    f32x4_t acc[MT4][2];

    auto finish_group = [&](int g) __attribute__((always_inline)) {
        const int e = lane & 3;
        float res[2][(MT4 + 3) / 4];
#pragma unroll
        for (int t = 0; t < MT4; ++t) {
#pragma unroll
            for (int gu = 0; gu < 2; ++gu) {
                const f32x4_t d = acc[t][gu];
                float v = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
                v = dpp_add<0xB1>(v);
                v = dpp_add<0x4E>(v);
                if (e == (t & 3)) res[gu][t >> 2] = v;
            }
        }
        const int row = 4 * g + (lane >> 4);
#pragma unroll
        for (int k = 0; k < (MT4 + 3) / 4; ++k) {
            const int t = 4 * k + e;
            const int m = 4 * t + ((lane & 15) >> 2);
            if (t < MT4 && m < M && row < N) {
                out[(int64_t)m * ldo + row] = glu_epilogue(res[0][k], res[1][k]);
            }
        }
    };

    auto compute = [&](int s, const u32x4_t (&A)[2][U]) __attribute__((always_inline)) {
        const int sb = s % nsg;
        if (sb == 0) {
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
                acc[t][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                acc[t][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        const u32x4_t* src = hs + (s & 1) * MP * SC;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        // all MT4 hidden operands of a segment are read before its MFMAs, so
        // the LDS latency is paid once per segment rather than once per tile
        u32x4_t b[2][MT4];
        auto read_b = [&](int u, u32x4_t (&bt)[MT4]) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < MT4; ++t) bt[t] = src[(4 * t + rho_a) * SC + ((u * 16 + cseg) ^ lds_swz4(rho_a))];
        };
        read_b(0, b[0]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u + 1 < U) read_b(u + 1, b[(u + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);  // the next segment's reads stay ahead of these MFMAs
            const bool ok = !RAGGED || (sb * U + u) * 16 + cseg < nchunks;
            const u32x4_t ag = RAGGED ? (ok ? A[0][u] : z) : A[0][u];
            const u32x4_t au = RAGGED ? (ok ? A[1][u] : z) : A[1][u];
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
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
    // branches around a load, so the waits can leave all prefetches in flight;
    // the last stages (TAIL true) skip what lies past the end.
    auto stage = [&](auto Qc, auto tailc, int s) __attribute__((always_inline)) {
        constexpr int Q = decltype(Qc)::value;
        constexpr bool TAIL = decltype(tailc)::value;
        if (!TAIL || s + 2 < nstages) load_h(s + 2, hr[Q % 2]);     // hr[s % 2] was published at s-1
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

using MfmaFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int, RowStrides, int);

template <int MT4, bool HL, bool RG>
MfmaFn pick_u(int U)
{
    switch (U) {
    case 2: return mfma_kernel<MT4, 2, HL, RG>;
    case 4: return mfma_kernel<MT4, 4, HL, RG>;
    case 5: return mfma_kernel<MT4, 5, HL, RG>;
    case 8: return mfma_kernel<MT4, 8, HL, RG>;
    default: return nullptr;
    }
}

template <int MT4, bool RG>
MfmaFn pick_slice_u(int U, int depth)
{
    // 8 segments (16 KiB per wave) of weights in flight
    if (U == 2 && depth == 4) return mfma_slice_kernel<MT4, 2, 4, RG>;
    if (U == 4 && depth == 2) return mfma_slice_kernel<MT4, 4, 2, RG>;
    return nullptr;
}

template <int MT4>
MfmaFn pick_flags(const MfmaConfig& c)
{
    switch (c.hidden) {
    case kHiddenLds: return c.ragged ? pick_u<MT4, true, true>(c.U) : pick_u<MT4, true, false>(c.U);
    case kHiddenL2: return c.ragged ? pick_u<MT4, false, true>(c.U) : pick_u<MT4, false, false>(c.U);
    case kHiddenSlices:
        if (c.block != kMfmaMaxThreads) return nullptr;
        return c.ragged ? pick_slice_u<MT4, true>(c.U, c.depth) : pick_slice_u<MT4, false>(c.U, c.depth);
    default: return nullptr;
    }
}

MfmaFn pick(const MfmaConfig& c)
{
    switch (c.MT4) {
    case 1: return pick_flags<1>(c);
    case 2: return pick_flags<2>(c);
    case 3: return pick_flags<3>(c);
    case 4: return pick_flags<4>(c);
    case 5: return pick_flags<5>(c);
    case 6: return pick_flags<6>(c);
    case 7: return pick_flags<7>(c);
    case 8: return pick_flags<8>(c);
    default: return nullptr;
    }
}

}  // namespace

size_t mfma_slice_lds_bytes(int mt4, int u) { return (size_t)2 * 4 * mt4 * u * 16 * 16; }

int mfma_slice_depth(int u) { return u > 0 ? 8 / u : 0; }

size_t mfma_hidden_lds_bytes(int m, int64_t k)
{
    const int64_t nchunks = k / 8;
    return (size_t)m * (size_t)(nchunks % 4 == 0 ? nchunks : nchunks + 1) * 16;
}

bool mfma_supported(const MfmaConfig& c)
{
    if (c.rows == 8) {
        return c.hidden == kHiddenSlices &&
               mfma8_supported((4 * c.MT4 + 7) / 8, c.U, c.depth, c.ragged, c.block, c.order);
    }
    if (c.rows != 4) return false;
    if (c.block < kWave || c.block > kMfmaMaxThreads || c.block % kWave != 0) return false;
    if (c.hidden == kHiddenSlices && mfma_slice_lds_bytes(c.MT4, c.U) > (size_t)kLdsBudget) return false;
    return pick(c) != nullptr;
}

hipError_t mfma_launch(const MfmaConfig& c, int M, const uint16_t* hidden, const uint16_t* gate_w,
                       const uint16_t* up_w, uint16_t* out, int64_t N, int64_t K, RowStrides ld,
                       hipStream_t stream)
{
    if (c.rows == 8) {
        if (c.hidden != kHiddenSlices) return hipErrorInvalidValue;
        return mfma8_launch(M, c.U, c.depth, c.order, c.nsg, c.ragged, c.grid, hidden, gate_w, up_w, out, N, K, ld,
                            stream);
    }
    MfmaConfig cm = c;
    cm.MT4 = (M + 3) / 4;
    MfmaFn fn = pick(cm);
    if (!fn || M < 1 || M > 4 * cm.MT4) return hipErrorInvalidValue;
    size_t lds = 0;
    if (cm.hidden == kHiddenLds) lds = mfma_hidden_lds_bytes(M, K);
    if (cm.hidden == kHiddenSlices) lds = mfma_slice_lds_bytes(cm.MT4, cm.U);
    hipLaunchKernelGGL(fn, dim3(cm.grid), dim3(cm.block), lds, stream,
                       hidden, gate_w, up_w, out, M, (int)N, (int)K, ld, cm.nsg);
    return hipGetLastError();
}

}  // namespace glu
