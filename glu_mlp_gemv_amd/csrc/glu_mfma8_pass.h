// The slice-major 8-row MFMA walk (mfma8_pass_body), shared by the forward's kernel
// (mfma8_pass_kernel, instantiated in glu_mfma8.hip) and the backward's (mfma8_pass_act_kernel in
// glu_mfma8_act.hip: the same walk with the backward's elementwise step as the epilogue).  The layout of the operands and of the accumulators is the
// 8-row block-diagonal one described at the top of glu_mfma8.hip.
#pragma once

#include "glu_backward.h"
#include "glu_device.h"
#include "glu_mfma_common.h"

namespace glu {

// K-slice-major order.  A workgroup owns jb <= JBMAX blocks of W groups (its blocks
// blockIdx.x + j*gridDim.x, j < jb) and walks K once for all of them: stage t is
// (slice t / jb, block t % jb), and the waves keep jb sets of accumulators.  Each
// K-slice of hidden is then loaded and published to LDS once per workgroup and
// serves jb stages, so the slice traffic through L2 and the vector memory path,
// and the barriers, are 1/jb of those of the block-by-block order above, for
// the same weight stream (8 rows x 128 contiguous bytes per load, one stage of
// weights in flight).  The slice of K-range sb+1 is loaded into registers at the
// first stage of slice sb and written to the other LDS buffer after its last
// stage, then one barrier publishes it: every wave has finished slice sb-1 (the
// previous barrier) before that buffer is overwritten.  The per-lane summation
// order of an output is that of mfma8_slice_kernel: results are bitwise equal.
// ACT: the backward's first step instead of the GLU epilogue.  From the rounded G and U and the
// upstream gradient dout ([M][N], rows ld.o apart) the lanes form dg and du (glu_act_grad) and store
// them at out (dg, [M][N]) and out + M * ld.o (du); dout is unused otherwise.
template <int MT8, int U, int JBMAX, bool RAGGED, bool ACT>
__device__ __forceinline__ void
mfma8_pass_body(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
                const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
                int M, int N, int K, RowStrides ld, int nsg, const uint16_t* __restrict__ dout)
{
    const int64_t ldo = ld.o;
    const uint32_t ldh8 = (uint32_t)(ld.h >> 3), ldg8 = (uint32_t)(ld.g >> 3), ldu8 = (uint32_t)(ld.u >> 3);
    constexpr int W = kMfmaMaxThreads / kWave;
    constexpr int MP = 8 * MT8;
    constexpr int SC = U * 8;
    static_assert(SC % 16 == 0, "the LDS swizzle permutes 16-chunk blocks of a row");
    constexpr int HPT = (MP * SC + kMfmaMaxThreads - 1) / kMfmaMaxThreads;
    extern __shared__ u32x4_t hs[];  // [2][MP][SC], chunk c of row r at c ^ lds_swz8(r)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K >> 3;
    const int i16 = lane & 15;
    const int rho = i16 >> 1;
    const int cw = (i16 & 1) * 4 + (lane >> 4);
    const u32x4_t* h4 = reinterpret_cast<const u32x4_t*>(hidden);

    const int ngroups = (N + 7) / 8;
    const int nblocks = (ngroups + W - 1) / W;
    if ((int)blockIdx.x >= nblocks) return;  // whole workgroup
    // blocks of this workgroup; the host launches at least ceil(nblocks / JBMAX) workgroups
    const int jb = (nblocks - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;

    auto group_of = [&](int j) __attribute__((always_inline)) {
        return ((int)blockIdx.x + j * (int)gridDim.x) * W + wave;
    };
    auto load_h = [&](int sb, u32x4_t (&hr)[HPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
            const int e = min(i * kMfmaMaxThreads + (int)threadIdx.x, MP * SC - 1);
            const int m = min(e / SC, M - 1);  // padded rows repeat row M-1, never stored
            int c = sb * SC + (e % SC);
            if (RAGGED) c = min(c, nchunks - 1);
            hr[i] = h4[(uint32_t)m * ldh8 + (uint32_t)c];
        }
    };
    auto store_h = [&](int sb, const u32x4_t (&hr)[HPT]) __attribute__((always_inline)) {
        u32x4_t* dst = hs + (sb & 1) * MP * SC;
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
            const int e = i * kMfmaMaxThreads + (int)threadIdx.x;
            if ((MP * SC) % kMfmaMaxThreads == 0 || e < MP * SC) dst[e ^ lds_swz8(e / SC)] = hr[i];
        }
    };
    auto load_w = [&](int sb, int j, u32x4_t (&A)[2][U]) __attribute__((always_inline)) {
        const int g = min(group_of(j), ngroups - 1);  // past the last group: re-read it, never stored
        const int64_t row0 = 8 * (int64_t)g;
        const uint32_t rr = (uint32_t)(min(8 * g + rho, N - 1) - 8 * g);
        const char* gp = reinterpret_cast<const char*>(gate_w + row0 * ld.g);
        const char* up = reinterpret_cast<const char*>(up_w + row0 * ld.u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = (sb * U + u) * 8 + cw;
            if (RAGGED) c = min(c, nchunks - 1);
            const uint32_t offg = (rr * ldg8 + (uint32_t)c) * 16u, offu = (rr * ldu8 + (uint32_t)c) * 16u;
            A[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(gp + offg));
            A[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(up + offu));
        }
    };

    // ACT: this lane's upstream gradients of group g (hidden rows 8t + (l%16)/2, its weight row),
    // loaded with the last stage's prefetches so that their latency hides behind its MFMAs
    auto load_go = [&](int g, uint16_t (&go)[MT8]) __attribute__((always_inline)) {
        const int row = 8 * g + 2 * (lane >> 4) + (lane & 1);
#pragma unroll
        for (int t = 0; t < MT8; ++t) {
            const int m = 8 * t + (i16 >> 1);
            go[t] = (m < M && row < N) ? dout[(int64_t)m * ldo + row] : (uint16_t)0;
        }
    };

    auto finish_group = [&](int g, const f32x4_t (&acc)[MT8][2], const uint16_t (&go)[MT8]) __attribute__((always_inline)) {
        const bool odd = (lane & 1) != 0;
        float res[2][MT8];
#pragma unroll
        for (int t = 0; t < MT8; ++t) {
#pragma unroll
            for (int gu = 0; gu < 2; ++gu) {
                const f32x4_t d = acc[t][gu];
                float v0 = odd ? d[1] : d[0];
                float v1 = odd ? d[3] : d[2];
                v0 = dpp_add<0xB1>(v0);
                v1 = dpp_add<0xB1>(v1);
                res[gu][t] = odd ? v1 : v0;
            }
        }
        const int row = 8 * g + 2 * (lane >> 4) + (lane & 1);
#pragma unroll
        for (int t = 0; t < MT8; ++t) {
            const int m = 8 * t + (i16 >> 1);
            if (m < M && row < N) {
                if constexpr (ACT) {
                    uint16_t dg, du;
                    glu_act_grad(bf16_to_f32(f32_to_bf16_rne(res[0][t])), bf16_to_f32(f32_to_bf16_rne(res[1][t])),
                                 bf16_to_f32(go[t]), &dg, &du);
                    out[(int64_t)m * ldo + row] = dg;
                    out[((int64_t)M + m) * ldo + row] = du;
                } else {
                    out[(int64_t)m * ldo + row] = glu_epilogue(res[0][t], res[1][t]);
                }
            }
        }
    };

    auto compute = [&](int sb, const u32x4_t (&A)[2][U], f32x4_t (&acc)[MT8][2]) __attribute__((always_inline)) {
        if (sb == 0) {
#pragma unroll
            for (int t = 0; t < MT8; ++t) {
                acc[t][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                acc[t][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        const u32x4_t* src = hs + (sb & 1) * MP * SC;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        u32x4_t b[2][MT8];
        auto read_b = [&](int u, u32x4_t (&bt)[MT8]) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < MT8; ++t) bt[t] = src[(8 * t + rho) * SC + ((u * 8 + cw) ^ lds_swz8(rho))];
        };
        read_b(0, b[0]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u + 1 < U) read_b(u + 1, b[(u + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
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
    };

    auto body = [&](auto JBc) __attribute__((always_inline)) {
        constexpr int JB = decltype(JBc)::value;
        constexpr int L = 2 * JB;  // stages per unrolled step: weight slot t % 2 and block t % JB are static
        u32x4_t A[2][2][U];        // weights of stage t in A[t % 2]
        u32x4_t hr[HPT];           // the next K-slice of hidden, between its load and its publication
        f32x4_t acc[JB][MT8][2];
        uint16_t go[MT8];          // ACT: the upstream gradients of the block being finished

        // stage t = (sb, j) at unrolled position Q = t % L; TAIL stages guard what the last slice lacks
        auto stage = [&](auto Qc, auto tailc, int sb) __attribute__((always_inline)) {
            constexpr int Q = decltype(Qc)::value;
            constexpr bool TAIL = decltype(tailc)::value;
            constexpr int j = Q % JB;
            constexpr int slot = Q % 2;
            const bool more = !TAIL || sb + 1 < nsg;
            if constexpr (j == 0) {
                if (more) load_h(sb + 1, hr);
            }
            if constexpr (j + 1 < JB) {
                load_w(sb, j + 1, A[1 - slot]);
            } else {
                if (more) load_w(sb + 1, 0, A[1 - slot]);
            }
            if constexpr (ACT) {
                if (TAIL && sb == nsg - 1) load_go(group_of(j), go);
            }
            __builtin_amdgcn_sched_barrier(0);  // the prefetches are issued before any of this stage's math
            compute(sb, A[slot], acc[j]);
            if constexpr (j == JB - 1) {
                if (more) store_h(sb + 1, hr);
                __syncthreads();
            }
            if (TAIL && sb == nsg - 1) finish_group(group_of(j), acc[j], go);
        };
        auto steps = [&](auto tailc, int sp) __attribute__((always_inline)) {
            // slices sp and sp + 1: positions Q = 0 .. L-1, slice sp + Q / JB
            auto one = [&](auto Qc) __attribute__((always_inline)) {
                constexpr int Q = decltype(Qc)::value;
                if (!decltype(tailc)::value || sp + Q / JB < nsg) stage(Qc, tailc, sp + Q / JB);
            };
            for_positions<0, L>(one);
        };

        load_h(0, hr);
        load_w(0, 0, A[0]);
        store_h(0, hr);
        __syncthreads();
        int sp = 0;
        for (; sp + 2 < nsg; sp += 2) steps(std::false_type{}, sp);  // every slice here has a next one
        steps(std::true_type{}, sp);                                   // the last one or two slices
    };

    if constexpr (JBMAX >= 3) {
        if (jb >= 3) {
            body(std::integral_constant<int, 3>{});
            return;
        }
    }
    if constexpr (JBMAX >= 2) {
        if (jb == 2) {
            body(std::integral_constant<int, 2>{});
            return;
        }
    }
    body(std::integral_constant<int, 1>{});
}

// The forward's kernel: the walk above with the GLU epilogue.
template <int MT8, int U, int JBMAX, bool RAGGED>
__global__ void __launch_bounds__(kMfmaMaxThreads)
mfma8_pass_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
                  const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
                  int M, int N, int K, RowStrides ld, int nsg)
{
    mfma8_pass_body<MT8, U, JBMAX, RAGGED, false>(hidden, gate_w, up_w, out, M, N, K, ld, nsg, nullptr);
}

// Tiles of 8 hidden rows the pass kernel runs for M rows: a last slice with fewer rows than the
// kernels are built for runs on their smallest tile count (padded rows repeat row M - 1 and are never
// stored)
inline int pass_tiles(int M, int U)
{
    const int mt8 = (M + 7) / 8;
    return U == 4 ? (mt8 < 5 ? 5 : mt8) : (mt8 < 2 ? 2 : mt8);
}

}  // namespace glu
