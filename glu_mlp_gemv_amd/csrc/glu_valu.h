// VALU GEMV for the dual-weight GLU projection at small batch (M <= 8).
//
// The decode-time projection is bound by streaming the two weight matrices
// from HBM once (DeepSpeed PR #8602, comment "Plan B: Dual-Weight GEMV",
// section on why library-level bandwidth is reachable at batch 1: each weight
// element is read and multiplied once).  Layout of the work on gfx950:
//
//  * waves are persistent: wave w of W owns the row groups w, w+W, w+2W, ...
//    (R consecutive output rows per group, gate and up row of each), so
//    neighbouring waves stream neighbouring rows and every wave owns the same
//    number of groups to within one;
//  * a row group is streamed in NB stages; in a stage lane l reads the U
//    16-byte chunks c = (b*U + i)*64 + l (8 bf16 each) of every row of the
//    group: one global_load_dwordx4 per chunk, consecutive lanes on
//    consecutive chunks, so a wave instruction reads 1 KiB of one row;
//  * two register buffers form a pipeline: the loads of stage s+1 are issued
//    before the arithmetic of stage s, so a wave always has one stage in
//    flight while it computes; no load sits behind a branch (a K that does not
//    fill the last stage clamps the chunk index and zeroes the value);
//  * hidden [M,K] is held in registers when it fits (M * NB * U chunks <= 16),
//    else staged once per workgroup in LDS;
//  * each lane accumulates in fp32 in a fixed order (stage by stage, chunk by
//    chunk, k increasing inside a chunk), a DPP/swizzle/permlane butterfly sums
//    the 64 lanes, and lane slot*M*R + m*R + r keeps the result; the rounding
//    epilogue runs once per 64 results on all lanes at once.
//
// Arithmetic: FMA on exactly widened bf16 (the bf16 x bf16 product is exact
// in fp32, so each step rounds once).  The per-lane order does not depend on
// M or R, so every row of a batched call is bitwise equal to the M=1 call on
// that row.
//
// DIAG (M = 1): the same loads, with the dot products on the matrix cores.  A
// wave's chunk-set of a row (lane l: chunk l of the set) is fed to
// v_mfma_f32_16x16x32_bf16 as A = the weight chunks and B = the hidden chunks
// exactly as loaded: lane l supplies A row l%16 and B column l%16 at K-block
// l/16, so D[i][i] = sum over q < 4 of (weight chunk i+16q) . (hidden chunk
// i+16q), while the off-diagonal entries pair unrelated chunks and are never
// read.  The U chunk-sets of a row accumulate into one D; lane l holds
// D[4(l/16)+e][l%16], so the 16 diagonal entries sit in lanes 0-3, 20-23,
// 40-43 and 60-63 (e = l%4), and the wave butterfly over those values (zeros
// elsewhere, which add exactly) gives the row's dot product.  This removes
// the widening and the FMAs from the vector ALU (about 200 instructions per
// row and wave) while keeping the streaming pattern of whole 1 KiB row pieces.
#pragma once

#include <type_traits>

#include "glu_device.h"
#include "glu_launch.h"
#include "glu_mfma_common.h"

namespace glu {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

// acc += sum over the 8 bf16 pairs of a chunk, k increasing (products exact in fp32)
__device__ __forceinline__ float dot_chunk(const u32x4& h, const u32x4& w, float acc)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(bf16lo(h[e]), bf16lo(w[e]), acc);
        acc = __builtin_fmaf(bf16hi(h[e]), bf16hi(w[e]), acc);
    }
    return acc;
}

// hidden [M,K], gate_w/up_w [N,K] (16-byte aligned, K % 8 == 0), out [M,N], rows at the strides of ld.
// NB <= 2; NB * U * 64 >= K/8, with equality unless RAGGED.  Dynamic LDS: M * K * 2 bytes when HLDS, else none.
// DIAG launches at most 4 waves per workgroup (one per SIMD at the default 4): a wave may then
// hold its MFMA operands, accumulators and two stages of loads in up to 512 registers.
template <int M, int R, int U, int NB, bool HLDS, bool RAGGED, bool DIAG = false>
__global__ void __launch_bounds__(DIAG ? kMfmaMaxThreads : kValuMaxThreads)
valu_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
            const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
            int N, int K, RowStrides ld)
{
    static_assert(NB == 1 || NB == 2, "a row group streams in one or two batches");
    static_assert(!DIAG || (M == 1 && !HLDS), "the matrix-core dot products serve one row of hidden in registers");
    const int64_t ldo = ld.o;
    const int ldh8 = (int)(ld.h >> 3);  // hidden row stride in 16-byte chunks
    constexpr int MR = M * R;
    constexpr int SLOTS = kWave / MR;  // row groups whose results one epilogue pass holds
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    // wave-uniform, stated so that the stage loop compiles to scalar control flow
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + threadIdx.x / kWave);
    const int nwaves = gridDim.x * wpb;
    const int nchunks = K >> 3;
    const u32x4* h4 = reinterpret_cast<const u32x4*>(hidden);

    extern __shared__ u32x4 h_lds[];
    u32x4 hreg[HLDS ? 1 : M][HLDS ? 1 : NB][HLDS ? 1 : U];
    if constexpr (HLDS) {
        for (int i = threadIdx.x; i < M * nchunks; i += blockDim.x) {
            const int m = i / nchunks;
            h_lds[i] = h4[m * ldh8 + (i - m * nchunks)];
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    const int c = (b * U + i) * kWave + lane;
                    const int cc = RAGGED ? min(c, nchunks - 1) : c;
                    hreg[m][b][i] = h4[m * ldh8 + cc];
                }
            }
        }
    }

    const int ngroups = (N + R - 1) / R;
    if (wave_id >= ngroups) return;  // no barrier follows
    const int my_groups = (ngroups - 1 - wave_id) / nwaves + 1;
    const int nstages = my_groups * NB;

    auto load = [&](int s, u32x4 (&wg)[R][U], u32x4 (&wu)[R][U]) {
        const int gi = s / NB;
        const int b = s - gi * NB;
        const int g = wave_id + gi * nwaves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(g * R + r, N - 1);  // rows past N re-read row N-1, never stored
            const u32x4* gp = reinterpret_cast<const u32x4*>(gate_w + (int64_t)row * ld.g);
            const u32x4* up = reinterpret_cast<const u32x4*>(up_w + (int64_t)row * ld.u);
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int c = (b * U + i) * kWave + lane;
                const int cc = RAGGED ? min(c, nchunks - 1) : c;
                wg[r][i] = ld_nt(gp + cc);
                wu[r][i] = ld_nt(up + cc);
            }
        }
    };

    float ag[M][R], au[M][R];
    f32x4_t dg[R], du[R];  // DIAG: the row's D of gate and up
    float resG = 0.0f, resU = 0.0f;

    // Results of group gi sit in lanes (gi % SLOTS)*MR + m*R + r; the epilogue
    // runs when a window of SLOTS groups is full or the last group is done.
    // Both follow from the group index alone (no loop-carried counter).
    auto flush = [&](int gi_last) {
        const int win0 = gi_last - gi_last % SLOTS;
        if (lane < (gi_last - win0 + 1) * MR) {
            const int gl = lane / MR;
            const int rem = lane - gl * MR;
            const int m = rem / R;
            const int r = rem - m * R;
            const int row = (wave_id + (win0 + gl) * nwaves) * R + r;
            if (row < N) {
                out[(int64_t)m * ldo + row] = glu_epilogue(resG, resU);
            }
        }
    };

    // the chunks of batch B (a compile-time index, so hidden registers are never indexed at run time)
    auto accumulate = [&](auto Bc, const u32x4 (&wg)[R][U], const u32x4 (&wu)[R][U]) {
        constexpr int B = decltype(Bc)::value;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if constexpr (DIAG) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int c = (B * U + i) * kWave + lane;
                const bool ok = !RAGGED || c < nchunks;
                const u32x4 h = RAGGED ? (ok ? hreg[0][B][i] : z) : hreg[0][B][i];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const u32x4 xg = RAGGED ? (ok ? wg[r][i] : z) : wg[r][i];
                    const u32x4 xu = RAGGED ? (ok ? wu[r][i] : z) : wu[r][i];
                    dg[r] = mfma16(xg, h, dg[r]);
                    du[r] = mfma16(xu, h, du[r]);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int c = (B * U + i) * kWave + lane;
            const bool ok = !RAGGED || c < nchunks;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                u32x4 h;
                if constexpr (HLDS) {
                    h = h_lds[m * nchunks + (RAGGED ? min(c, nchunks - 1) : c)];
                } else {
                    h = hreg[m][B][i];
                }
                if constexpr (RAGGED) h = ok ? h : z;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const u32x4 xg = RAGGED ? (ok ? wg[r][i] : z) : wg[r][i];
                    const u32x4 xu = RAGGED ? (ok ? wu[r][i] : z) : wu[r][i];
                    ag[m][r] = dot_chunk(h, xg, ag[m][r]);
                    au[m][r] = dot_chunk(h, xu, au[m][r]);
                }
            }
        }
    };

    auto compute = [&](int s, const u32x4 (&wg)[R][U], const u32x4 (&wu)[R][U]) {
        const int gi = s / NB;
        const int b = s - gi * NB;
        if (b == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    ag[m][r] = 0.0f;
                    au[m][r] = 0.0f;
                }
            }
            if constexpr (DIAG) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    dg[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    du[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
        }
        if constexpr (NB == 1) {
            accumulate(std::integral_constant<int, 0>{}, wg, wu);
        } else {
            if (b == 0) {
                accumulate(std::integral_constant<int, 0>{}, wg, wu);
            } else {
                accumulate(std::integral_constant<int, 1>{}, wg, wu);
            }
        }
        if (b == NB - 1) {
            const int slot = gi % SLOTS;
            if constexpr (DIAG) {
                // lane l holds D[4(l/16) + e][l%16]: the diagonal entry e = l%4 in lanes with l%16 / 4 == l/16
                const int e = lane & 3;
                const bool diag = ((lane & 15) >> 2) == (lane >> 4);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    auto pick = [&](const f32x4_t& d) {
                        const float v = e == 0 ? d[0] : (e == 1 ? d[1] : (e == 2 ? d[2] : d[3]));
                        return diag ? v : 0.0f;
                    };
                    ag[0][r] = pick(dg[r]);
                    au[0][r] = pick(du[r]);
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float gs = wave_sum(ag[m][r]);
                    const float us = wave_sum(au[m][r]);
                    if (lane == slot * MR + m * R + r) {
                        resG = gs;
                        resU = us;
                    }
                }
            }
            if (slot == SLOTS - 1 || gi == my_groups - 1) flush(gi);
        }
    };

    u32x4 aG[R][U], aU[R][U], bG[R][U], bU[R][U];
    load(0, aG, aU);
    int s = 0;
    while (true) {
        if (s + 1 >= nstages) {
            compute(s, aG, aU);
            break;
        }
        load(s + 1, bG, bU);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any of this stage\'s math
        compute(s, aG, aU);
        ++s;
        if (s + 1 >= nstages) {
            compute(s, bG, bU);
            break;
        }
        load(s + 1, aG, aU);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any of this stage\'s math
        compute(s, bG, bU);
        ++s;
    }
}

template <int M, int R, int U, int NB, bool RAGGED, bool DIAG = false>
constexpr ValuFn valu_fn()
{
    return valu_kernel<M, R, U, NB, valu_hidden_in_lds(M, U, NB), RAGGED, DIAG>;
}

// U in 1..8 for NB == 1, 5..8 for NB == 2 (NB == 2 arises only when K/8 > 512).
template <int M, int R, int NB, bool RAGGED, bool DIAG = false>
ValuFn valu_pick_u(int U)
{
    switch (U) {
    case 1: if constexpr (NB == 1) return valu_fn<M, R, 1, NB, RAGGED, DIAG>(); else return nullptr;
    case 2: if constexpr (NB == 1) return valu_fn<M, R, 2, NB, RAGGED, DIAG>(); else return nullptr;
    case 3: if constexpr (NB == 1) return valu_fn<M, R, 3, NB, RAGGED, DIAG>(); else return nullptr;
    case 4: if constexpr (NB == 1) return valu_fn<M, R, 4, NB, RAGGED, DIAG>(); else return nullptr;
    case 5: return valu_fn<M, R, 5, NB, RAGGED, DIAG>();
    case 6: return valu_fn<M, R, 6, NB, RAGGED, DIAG>();
    case 7: return valu_fn<M, R, 7, NB, RAGGED, DIAG>();
    case 8: return valu_fn<M, R, 8, NB, RAGGED, DIAG>();
    default: return nullptr;
    }
}

template <int M, int R, bool DIAG = false>
ValuFn valu_pick_m(int U, int NB, bool ragged)
{
    if (NB == 1) return ragged ? valu_pick_u<M, R, 1, true, DIAG>(U) : valu_pick_u<M, R, 1, false, DIAG>(U);
    if (NB == 2) return ragged ? valu_pick_u<M, R, 2, true, DIAG>(U) : valu_pick_u<M, R, 2, false, DIAG>(U);
    return nullptr;
}

}  // namespace glu
