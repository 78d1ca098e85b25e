// Dual GEMM with the GLU epilogue for large batches (M > 32): the same
// G = h Wg^T, U = h Wu^T and the same four bf16 roundings as the GEMV kernels,
// computed as tiled MFMA products.
//
// A workgroup of 4 waves owns a BN x BM output tile (BN weight rows of both
// matrices, BM rows of hidden) and walks K in stages of 64 elements: the BN
// gate rows, the BN up rows and the BM hidden rows of the stage (128 bytes
// each) are loaded with 16-byte loads, 8 lanes per row, into one of two LDS
// buffers, while the waves compute on the other.  Each wave computes a
// BN/2 x BM/2 quarter of both G and U with v_mfma_f32_16x16x32_bf16 in the
// standard operand layout: lane l reads 16 bytes of weight row l % 16 (A) and
// of hidden row l % 16 (B) at the same K chunk, so each hidden element in a
// B operand serves 16 weight rows.  In LDS, chunk c (16 bytes) of row r sits
// at c ^ ((r >> 1) & 7) of a 128-byte row: with the operand reads' lane
// pattern (rows l % 16, chunks 4s + l / 16) every 16-lane group of a
// ds_read_b128 then touches 16 distinct 16-byte slots of 256 bytes.
// Tiles are ordered so that the consecutive workgroups an XCD receives (the
// hardware deals workgroups to the 8 XCDs in turn) share weight tiles, which
// then come from that XCD's L2 for every M tile after the first.
#include "glu_backward.h"
#include "glu_device.h"
#include "glu_launch.h"
#include "glu_mfma_common.h"

namespace glu {

namespace {

constexpr int kStageK = 64;         // K elements per stage
constexpr int kStageChunks = 8;     // 16-byte chunks per row per stage
constexpr int kGemmThreads = 256;   // 4 waves in a 2 x 2 arrangement

__device__ __forceinline__ int gemm_swz(int r) { return (r >> 1) & 7; }

}  // namespace

// BN: weight rows per tile (64 or 128); BM: hidden rows per tile (64 or 128).
// KTAIL: K is not a multiple of 64 (chunks past K are read as zeros).
// PF: stages whose global loads are in flight while a stage computes (1 to 4;
// from 2 on, PF register sets rotate and a stage's data has PF stages of
// compute to arrive).
// nbm: M tiles; the grid holds ceil(N / BN) * nbm workgroups.
// LIN: write bf16(G) and bf16(U) instead of the GLU product: G to out, U to out2 (the
// backward's [2][M][N] workspace head).
// ACT (with LIN, not TRANS): the backward's elementwise step on the rounded G and U and the upstream
// gradient dout ([M][N], row stride ldo): dG to out, dU to out2 instead of G and U.
// TRANS (with LIN): the MFMA operands swap places, so each lane holds 4 consecutive hidden rows
// of one weight row, and G, U are stored transposed, out[n][m] and out2[n][m] (rows ldo apart;
// M a multiple of 4).  The backward's weight gradients are this product with dg^T, du^T as the
// two weights and hidden^T as the hidden (contraction over the rows of hidden).
template <int BN, int BM, bool KTAIL, int PF, bool LIN = false, bool TRANS = false, bool ACT = false>
__global__ void __launch_bounds__(kGemmThreads)
gemm_kernel(const uint16_t* __restrict__ hidden, int64_t ldh, const uint16_t* __restrict__ gate, int64_t ldg,
            const uint16_t* __restrict__ up, int64_t ldu, uint16_t* __restrict__ out, uint16_t* __restrict__ out2,
            int64_t ldo, int M, int N, int K, int nbm, int vec_out, const uint16_t* __restrict__ dout)
{
    static_assert(LIN || !TRANS, "the transposed store is a form of the linear epilogue");
    static_assert(!ACT || (LIN && !TRANS), "the elementwise step follows the row-major linear epilogue");
    constexpr int ROWS = 2 * BN + BM;                           // LDS rows per stage
    constexpr int LPT = ROWS * kStageChunks / kGemmThreads;     // 16-byte loads per thread per stage
    constexpr int WN = BN / 2, WM = BM / 2;
    constexpr int TN = WN / 16, TM = WM / 16;
    static_assert(ROWS * kStageChunks % kGemmThreads == 0, "whole loads per thread");
    static_assert(BN % 32 == 0 && BM % 32 == 0, "each load round covers 32 rows of one operand");

    extern __shared__ u32x4_t lds[];  // [2][ROWS][8]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;

    // workgroup -> tile: XCD x takes a contiguous run of tiles
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int per = G >> 3, rem = G & 7, xcd = bid & 7, slot = bid >> 3;
    const int t = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
    const int nb = t / nbm;
    const int mb = t - nb * nbm;
    const int n0 = nb * BN, m0 = mb * BM;
    const int nchunks = K >> 3;
    const int nstages = (nchunks + kStageChunks - 1) / kStageChunks;

    // this thread's loads: row r of the stage (gate rows, up rows, hidden rows), chunk c
    const char* src[LPT];
    int lidx[LPT];
    const int c_ld = tid & (kStageChunks - 1);
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
        const int r = (tid + q * kGemmThreads) / kStageChunks;
        const uint16_t* p;
        if (r < BN) {
            p = gate + (int64_t)min(n0 + r, N - 1) * ldg;
        } else if (r < 2 * BN) {
            p = up + (int64_t)min(n0 + r - BN, N - 1) * ldu;
        } else {
            p = hidden + (int64_t)min(m0 + r - 2 * BN, M - 1) * ldh;
        }
        src[q] = reinterpret_cast<const char*>(p);
        lidx[q] = r * kStageChunks + (c_ld ^ gemm_swz(r));
    }

    // a stage's loads land in a register set; ok: the chunk lies inside K (else it is stored as zeros)
    u32x4_t P[PF][LPT];
    bool okp[PF];
    auto gload = [&](int s, u32x4_t (&pf)[LPT], bool& ok) __attribute__((always_inline)) {
        const int kc = s * kStageChunks + c_ld;
        const int kcc = KTAIL ? min(kc, nchunks - 1) : kc;
        ok = !KTAIL || kc < nchunks;
#pragma unroll
        for (int q = 0; q < LPT; ++q) {
            pf[q] = *reinterpret_cast<const u32x4_t*>(src[q] + (int64_t)kcc * 16);
        }
    };
    auto lstore = [&](int buf, const u32x4_t (&pf)[LPT], bool ok) __attribute__((always_inline)) {
        u32x4_t* dst = lds + buf * (ROWS * kStageChunks);
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < LPT; ++q) dst[lidx[q]] = KTAIL ? (ok ? pf[q] : z) : pf[q];
    };

    f32x4_t ag[TN][TM], au[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            ag[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            au[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

    const int i16 = lane & 15;
    const int q16 = lane >> 4;
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const u32x4_t* L = lds + buf * (ROWS * kStageChunks);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int c = 4 * sub + q16;
            u32x4_t b[TM];
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int r = 2 * BN + wm * WM + 16 * j + i16;
                b[j] = L[r * kStageChunks + (c ^ gemm_swz(r))];
            }
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int rg = wn * WN + 16 * i + i16;
                const int ru = BN + rg;
                const u32x4_t a_g = L[rg * kStageChunks + (c ^ gemm_swz(rg))];
                const u32x4_t a_u = L[ru * kStageChunks + (c ^ gemm_swz(ru))];
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    if constexpr (TRANS) {
                        ag[i][j] = mfma16(b[j], a_g, ag[i][j]);
                        au[i][j] = mfma16(b[j], a_u, au[i][j]);
                    } else {
                        ag[i][j] = mfma16(a_g, b[j], ag[i][j]);
                        au[i][j] = mfma16(a_u, b[j], au[i][j]);
                    }
                }
            }
        }
    };

    if constexpr (PF == 1) {
        gload(0, P[0], okp[0]);
        lstore(0, P[0], okp[0]);
        __syncthreads();
        for (int s = 0; s < nstages; ++s) {
            if (s + 1 < nstages) gload(s + 1, P[0], okp[0]);
            compute(s & 1);
            if (s + 1 < nstages) lstore((s + 1) & 1, P[0], okp[0]);
            __syncthreads();
        }
    } else {
        // A ring of PF register sets: stage s's loads sit in set s % PF.  Stage s refills its own set
        // (stored to LDS at the end of stage s - 1) with stage s + PF, computes, then stores stage
        // s + 1's set into the other LDS buffer.  In the steady state every refill is live and
        // nothing branches around a load, so the waits leave PF - 1 stages of loads in flight.
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            if (s < nstages) gload(s, P[s], okp[s]);
        }
        lstore(0, P[0], okp[0]);
        __syncthreads();
        auto stage = [&](auto Qc, auto tailc, int s) __attribute__((always_inline)) {
            constexpr int Q = decltype(Qc)::value;
            constexpr bool TAIL = decltype(tailc)::value;
            if (!TAIL || s + PF < nstages) gload(s + PF, P[Q], okp[Q]);
            compute(s & 1);
            if (!TAIL || s + 1 < nstages) lstore((s + 1) & 1, P[(Q + 1) % PF], okp[(Q + 1) % PF]);
            __syncthreads();
        };
        auto steady = [&](auto Qc, int s) __attribute__((always_inline)) { stage(Qc, std::false_type{}, s); };
        auto tail = [&](auto Qc, int s) __attribute__((always_inline)) { stage(Qc, std::true_type{}, s); };
        int s0 = 0;
        for (; s0 + 2 * PF <= nstages; s0 += PF) run_stages<0, PF>(steady, s0, nstages);
        for (; s0 < nstages; s0 += PF) run_stages<0, PF>(tail, s0, nstages);
    }

    if constexpr (TRANS) {
        // lane l holds G and U of weight row l % 16, hidden rows 4(l/16) + e, of each 16 x 16 tile
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const int n = n0 + wn * WN + 16 * i + i16;
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int m = m0 + wm * WM + 16 * j + 4 * q16;
                if (n < N && m < M) {  // M % 4 == 0 for this form (checked by the launcher)
                    uint2 wg, wu;
                    wg.x = (uint32_t)f32_to_bf16_rne(ag[i][j][0]) | ((uint32_t)f32_to_bf16_rne(ag[i][j][1]) << 16);
                    wg.y = (uint32_t)f32_to_bf16_rne(ag[i][j][2]) | ((uint32_t)f32_to_bf16_rne(ag[i][j][3]) << 16);
                    wu.x = (uint32_t)f32_to_bf16_rne(au[i][j][0]) | ((uint32_t)f32_to_bf16_rne(au[i][j][1]) << 16);
                    wu.y = (uint32_t)f32_to_bf16_rne(au[i][j][2]) | ((uint32_t)f32_to_bf16_rne(au[i][j][3]) << 16);
                    *reinterpret_cast<uint2*>(out + (int64_t)n * ldo + m) = wg;
                    *reinterpret_cast<uint2*>(out2 + (int64_t)n * ldo + m) = wu;
                }
            }
        }
        return;
    }
    // lane l holds G and U of weight rows 4(l/16) + e, hidden row l % 16, of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int n = n0 + wn * WN + 16 * i + 4 * q16;
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int m = m0 + wm * WM + 16 * j + i16;
            if constexpr (LIN) {
                if (m < M && n + 3 < N) {  // N % 4 == 0 for this form (checked by the launcher)
                    uint2 wg, wu;
                    if constexpr (ACT) {
                        uint16_t dg[4], du[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            glu_act_grad(bf16_to_f32(f32_to_bf16_rne(ag[i][j][e])),
                                         bf16_to_f32(f32_to_bf16_rne(au[i][j][e])),
                                         bf16_to_f32(dout[(int64_t)m * ldo + n + e]), &dg[e], &du[e]);
                        }
                        wg.x = (uint32_t)dg[0] | ((uint32_t)dg[1] << 16);
                        wg.y = (uint32_t)dg[2] | ((uint32_t)dg[3] << 16);
                        wu.x = (uint32_t)du[0] | ((uint32_t)du[1] << 16);
                        wu.y = (uint32_t)du[2] | ((uint32_t)du[3] << 16);
                        *reinterpret_cast<uint2*>(out + (int64_t)m * ldo + n) = wg;
                        *reinterpret_cast<uint2*>(out2 + (int64_t)m * ldo + n) = wu;
                        continue;
                    }
                    wg.x = (uint32_t)f32_to_bf16_rne(ag[i][j][0]) | ((uint32_t)f32_to_bf16_rne(ag[i][j][1]) << 16);
                    wg.y = (uint32_t)f32_to_bf16_rne(ag[i][j][2]) | ((uint32_t)f32_to_bf16_rne(ag[i][j][3]) << 16);
                    wu.x = (uint32_t)f32_to_bf16_rne(au[i][j][0]) | ((uint32_t)f32_to_bf16_rne(au[i][j][1]) << 16);
                    wu.y = (uint32_t)f32_to_bf16_rne(au[i][j][2]) | ((uint32_t)f32_to_bf16_rne(au[i][j][3]) << 16);
                    *reinterpret_cast<uint2*>(out + (int64_t)m * ldo + n) = wg;
                    *reinterpret_cast<uint2*>(out2 + (int64_t)m * ldo + n) = wu;
                }
                continue;
            }
            uint16_t v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = glu_epilogue(ag[i][j][e], au[i][j][e]);
            if (m < M) {
                uint16_t* o = out + (int64_t)m * ldo + n;
                if (vec_out && n + 3 < N) {
                    uint2 w;
                    w.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
                    w.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
                    *reinterpret_cast<uint2*>(o) = w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (n + e < N) o[e] = v[e];
                    }
                }
            }
        }
    }
}

namespace {

using GemmFn = void (*)(const uint16_t*, int64_t, const uint16_t*, int64_t, const uint16_t*, int64_t, uint16_t*,
                        uint16_t*, int64_t, int, int, int, int, int, const uint16_t*);

template <int BN, int BM>
GemmFn pick_tail(bool ktail, int pf)
{
    if (pf == 1) return ktail ? gemm_kernel<BN, BM, true, 1> : gemm_kernel<BN, BM, false, 1>;
    if (pf == 2) return ktail ? gemm_kernel<BN, BM, true, 2> : gemm_kernel<BN, BM, false, 2>;
    if (pf == 3) return ktail ? gemm_kernel<BN, BM, true, 3> : gemm_kernel<BN, BM, false, 3>;
    if (pf == 4) return ktail ? gemm_kernel<BN, BM, true, 4> : gemm_kernel<BN, BM, false, 4>;
    return nullptr;
}

GemmFn pick(int bn, int bm, bool ktail, int pf)
{
    if (bn == 64 && bm == 64) return pick_tail<64, 64>(ktail, pf);
    if (bn == 64 && bm == 128) return pick_tail<64, 128>(ktail, pf);
    if (bn == 128 && bm == 64) return pick_tail<128, 64>(ktail, pf);
    if (bn == 128 && bm == 128) return pick_tail<128, 128>(ktail, pf);
    return nullptr;
}

}  // namespace

size_t gemm_lds_bytes(int bn, int bm)
{
    return (size_t)2 * (size_t)(2 * bn + bm) * kStageChunks * 16;
}

bool gemm_supported(const GemmConfig& c)
{
    return pick(c.bn, c.bm, c.ktail, c.depth) != nullptr && gemm_lds_bytes(c.bn, c.bm) <= (size_t)kLdsMax;
}

int64_t gemm_grid(const GemmConfig& c, int64_t M, int64_t N)
{
    return ((N + c.bn - 1) / c.bn) * ((M + c.bm - 1) / c.bm);
}

hipError_t gemm_launch(const GemmConfig& c, int M, const uint16_t* hidden, const uint16_t* gate_w,
                       const uint16_t* up_w, uint16_t* out, int N, int K, const RowStrides& ld, hipStream_t stream)
{
    GemmFn fn = pick(c.bn, c.bm, c.ktail, c.depth);
    if (!fn || M < 1 || N < 1 || K < 8 || (K & 7) != 0) return hipErrorInvalidValue;
    const bool ktail = (K % kStageK) != 0;
    if (ktail != c.ktail) return hipErrorInvalidValue;
    const int64_t grid = gemm_grid(c, M, N);
    if (grid < 1 || grid > 0x7fffffff) return hipErrorInvalidValue;
    const int nbm = (M + c.bm - 1) / c.bm;
    const size_t lds = gemm_lds_bytes(c.bn, c.bm);
    if (lds > (size_t)kLdsBudget) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    // 8-byte output stores need 8-byte aligned rows
    const int vec_out = (((uintptr_t)out & 7u) == 0 && (ld.o & 3) == 0) ? 1 : 0;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kGemmThreads), lds, stream, hidden, ld.h, gate_w, ld.g, up_w,
                       ld.u, out, out, ld.o, M, N, K, nbm, vec_out, nullptr);
    return hipGetLastError();
}

hipError_t gemm_linear_launch(int M, const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                              uint16_t* gu, int N, int K, const uint16_t* dout, hipStream_t stream)
{
    // 64 x 64 tiles, two stages of loads in flight; N % 4 == 0 so that each lane's 4 outputs of a
    // row are whole 8-byte stores inside the row.  With dout: the elementwise step in the epilogue
    if (M < 1 || N < 4 || (N & 3) != 0 || K < 8 || (K & 7) != 0) return hipErrorInvalidValue;
    const bool ktail = (K % kStageK) != 0;
    GemmFn fn = dout ? (ktail ? gemm_kernel<64, 64, true, 2, true, false, true>
                              : gemm_kernel<64, 64, false, 2, true, false, true>)
                     : (ktail ? gemm_kernel<64, 64, true, 2, true> : gemm_kernel<64, 64, false, 2, true>);
    const int64_t nbm = (M + 63) / 64;
    const int64_t grid = ((N + 63) / 64) * nbm;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kGemmThreads), gemm_lds_bytes(64, 64), stream, hidden, (int64_t)K,
                       gate_w, (int64_t)K, up_w, (int64_t)K, gu, gu + (int64_t)M * N, (int64_t)N, M, N, K, (int)nbm, 1,
                       dout);
    return hipGetLastError();
}

hipError_t gemm_dw_launch(int mp, const uint16_t* hT, const uint16_t* dgT, const uint16_t* duT, uint16_t* dwg,
                          uint16_t* dwu, int N, int K, hipStream_t stream)
{
    // dWg[j][k] = bf16(sum_m dgT[j][m] hT[k][m]), dWu likewise: the linear GEMM with dgT, duT as the
    // weights (N rows), hT as the hidden (K rows), a contraction of mp (padded rows of hidden, zeros
    // past M), stored transposed.  64 x 64 tiles, two stages of loads in flight.
    if (mp < 32 || (mp & 31) != 0 || N < 1 || K < 8 || (K & 7) != 0) return hipErrorInvalidValue;
    const bool ktail = (mp % kStageK) != 0;
    GemmFn fn = ktail ? gemm_kernel<64, 64, true, 2, true, true> : gemm_kernel<64, 64, false, 2, true, true>;
    const int64_t nbm = (K + 63) / 64;
    const int64_t grid = ((N + 63) / 64) * nbm;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kGemmThreads), gemm_lds_bytes(64, 64), stream, hT, (int64_t)mp,
                       dgT, (int64_t)mp, duT, (int64_t)mp, dwg, dwu, (int64_t)K, K, N, mp, (int)nbm, 1, nullptr);
    return hipGetLastError();
}

}  // namespace glu
