// The 4-row block-diagonal MFMA walk with hidden in LDS or read from L2 (mfma_body), shared by the
// forward's kernel (mfma_kernel, instantiated in glu_mfma.hip, whose header describes the operand
// layout) and the backward's (mfma_act_kernel in glu_mfma_act.hip: the same walk with the
// backward's elementwise step as the epilogue).
#pragma once

#include "glu_backward.h"
#include "glu_device.h"
#include "glu_mfma_common.h"

namespace glu {

// MT4: hidden-row tiles of 4 (M <= 4*MT4); U: 128-element segments per stage;
// nsg: stages per group (nsg * U * 16 >= K/8, equality unless RAGGED).
// Dynamic LDS when HLDS: M * K * 2 bytes, or M * (K/8 + 1) * 16 when K/8 is not a multiple of 4.
// ACT: the backward's first step instead of the GLU epilogue: from the rounded G and U and the
// upstream gradient dout ([M][N], rows ld.o apart, loaded with the group's last stage) the lanes
// form dg and du (glu_act_grad) and store them at out (dg) and out + M * ld.o (du).
template <int MT4, int U, bool HLDS, bool RAGGED, bool ACT>
__device__ __forceinline__ void
mfma_body(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
          const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
          int M, int N, int K, RowStrides ld, int nsg, const uint16_t* __restrict__ dout)
{
    const int64_t ldo = ld.o;
    const uint32_t ldh8 = (uint32_t)(ld.h >> 3), ldg8 = (uint32_t)(ld.g >> 3), ldu8 = (uint32_t)(ld.u >> 3);
    extern __shared__ u32x4_t h_lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    // wave-uniform, stated so that the stage loop compiles to scalar control flow
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + threadIdx.x / kWave);
    const int nwaves = gridDim.x * wpb;
    const int nchunks = K >> 3;
    const int i16 = lane & 15;
    const int rho_a = i16 >> 2;              // weight row of this lane's A data
    const int cseg = (i16 & 3) * 4 + (lane >> 4);  // 16-byte chunk within a 256-byte segment
    const u32x4_t* h4 = reinterpret_cast<const u32x4_t*>(hidden);

    // the hidden rows one read touches must fall in different LDS banks: chunk
    // c of row m sits at c ^ lds_swz4(m) when K/8 is a multiple of 4, else rows
    // are padded by one chunk
    const bool hswz = (nchunks & 3) == 0;
    const int hpitch = hswz ? nchunks : nchunks + 1;
    if constexpr (HLDS) {
        for (int i = threadIdx.x; i < M * nchunks; i += blockDim.x) {
            const int m = i / nchunks;
            const int c = i - m * nchunks;
            h_lds[m * hpitch + (hswz ? c ^ lds_swz4(m) : c)] = h4[m * ldh8 + c];
        }
        __syncthreads();
    }

    const int ngroups = (N + 3) / 4;
    if (wave_id >= ngroups) return;  // no barrier follows
    const int my_groups = (ngroups - 1 - wave_id) / nwaves + 1;
    const int nstages = my_groups * nsg;

    // hidden rows of this lane's B data, one per tile (rows past M repeat row M-1, never stored)
    int hrow[MT4];
#pragma unroll
    for (int t = 0; t < MT4; ++t) hrow[t] = min(4 * t + rho_a, M - 1);

    constexpr int BT = HLDS ? 1 : MT4;  // hidden operands carried with a stage (L2 path only)
    constexpr int BU = HLDS ? 1 : U;
    constexpr int KT = (MT4 + 3) / 4;   // outputs per lane per group
    constexpr int GQ = ACT ? KT : 1;    // upstream gradients carried with a group's last stage (ACT)
    const int e4 = lane & 3;

    auto load = [&](int s, u32x4_t (&A)[2][U], u32x4_t (&Bq)[BT][BU], uint16_t (&Gq)[GQ]) {
        const int gi = s / nsg;
        const int sb = s - gi * nsg;
        const int g = wave_id + gi * nwaves;
        if constexpr (ACT) {
            if (sb == nsg - 1) {
                const int row = 4 * g + (lane >> 4);
#pragma unroll
                for (int k = 0; k < KT; ++k) {
                    const int t = 4 * k + e4;
                    const int m = 4 * t + ((lane & 15) >> 2);
                    Gq[k] = (t < MT4 && m < M && row < N) ? dout[(int64_t)m * ldo + row] : (uint16_t)0;
                }
            }
        }
        // a wave-uniform base for the group plus a 32-bit lane offset, so the
        // addresses never share registers with loads still in flight
        const int64_t row0 = 4 * (int64_t)g;
        const uint32_t rr = (uint32_t)(min(4 * g + rho_a, N - 1) - 4 * g);  // rows past N re-read row N-1, never stored
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
        if constexpr (!HLDS) {
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int c = (sb * U + u) * 16 + cseg;
                    if (RAGGED) c = min(c, nchunks - 1);
                    const uint32_t off = ((uint32_t)hrow[t] * ldh8 + (uint32_t)c) * 16u;
                    Bq[t][u] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(hidden) + off);
                }
            }
        }
    };

    f32x4_t acc[MT4][2];

    auto finish_group = [&](int g, const uint16_t (&Gq)[GQ]) {
        // useful entry e = lane % 4, then the quad sum over the four blocks
        const int e = e4;
        float res[2][KT];
#pragma unroll
        for (int t = 0; t < MT4; ++t) {
#pragma unroll
            for (int gu = 0; gu < 2; ++gu) {
                const f32x4_t d = acc[t][gu];
                float v = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
                v = dpp_add<0xB1>(v);  // lane ^ 1
                v = dpp_add<0x4E>(v);  // lane ^ 2
                if (e == (t & 3)) res[gu][t >> 2] = v;
            }
        }
        // lane l keeps tiles t with t % 4 == l % 4: hidden row 4t + (l%16)/4, weight row 4g + l/16
        const int row = 4 * g + (lane >> 4);
#pragma unroll
        for (int k = 0; k < (MT4 + 3) / 4; ++k) {
            const int t = 4 * k + e;
            const int m = 4 * t + ((lane & 15) >> 2);
            if (t < MT4 && m < M && row < N) {
                if constexpr (ACT) {
                    uint16_t dg, du;
                    glu_act_grad(bf16_to_f32(f32_to_bf16_rne(res[0][k])), bf16_to_f32(f32_to_bf16_rne(res[1][k])),
                                 bf16_to_f32(Gq[k]), &dg, &du);
                    out[(int64_t)m * ldo + row] = dg;
                    out[((int64_t)M + m) * ldo + row] = du;
                } else {
                    out[(int64_t)m * ldo + row] = glu_epilogue(res[0][k], res[1][k]);
                }
            }
        }
    };

    auto compute = [&](int s, const u32x4_t (&A)[2][U], const u32x4_t (&Bq)[BT][BU], const uint16_t (&Gq)[GQ]) {
        const int gi = s / nsg;
        const int sb = s - gi * nsg;
        if (sb == 0) {
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
                acc[t][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                acc[t][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (sb * U + u) * 16 + cseg;
            const bool ok = !RAGGED || c < nchunks;
            const int cc = RAGGED ? min(c, nchunks - 1) : c;
            const u32x4_t ag = RAGGED ? (ok ? A[0][u] : z) : A[0][u];
            const u32x4_t au = RAGGED ? (ok ? A[1][u] : z) : A[1][u];
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
                u32x4_t b;
                if constexpr (HLDS) {
                    b = h_lds[hrow[t] * hpitch + (hswz ? cc ^ lds_swz4(hrow[t]) : cc)];
                } else {
                    b = Bq[t][u];
                }
                if constexpr (RAGGED) b = ok ? b : z;
                acc[t][0] = mfma16(ag, b, acc[t][0]);
                acc[t][1] = mfma16(au, b, acc[t][1]);
            }
        }
        if (sb == nsg - 1) finish_group(wave_id + gi * nwaves, Gq);
    };

    u32x4_t a0[2][U], a1[2][U], b0[BT][BU], b1[BT][BU];
    uint16_t q0[GQ], q1[GQ];
    load(0, a0, b0, q0);
    int s = 0;
    while (true) {
        if (s + 1 >= nstages) {
            compute(s, a0, b0, q0);
            break;
        }
        load(s + 1, a1, b1, q1);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any of this stage\'s math
        compute(s, a0, b0, q0);
        ++s;
        if (s + 1 >= nstages) {
            compute(s, a1, b1, q1);
            break;
        }
        load(s + 1, a0, b0, q0);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any of this stage\'s math
        compute(s, a1, b1, q1);
        ++s;
    }
}

// The forward's kernel: the walk above with the GLU epilogue.
template <int MT4, int U, bool HLDS, bool RAGGED>
__global__ void __launch_bounds__(kMfmaMaxThreads)
mfma_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
            const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
            int M, int N, int K, RowStrides ld, int nsg)
{
    mfma_body<MT4, U, HLDS, RAGGED, false>(hidden, gate_w, up_w, out, M, N, K, ld, nsg, nullptr);
}

}  // namespace glu
