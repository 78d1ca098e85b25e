// Backward of the dual-weight GLU projection above 8 rows of hidden: the three
// contractions as v_mfma_f32_16x16x32_bf16 products.  Up to 64 rows as below;
// above, dh_mfma_kernel runs over slices of 128 rows of hidden (two 16-row
// tiles per wave; above 128 rows slices of 256, four tiles per wave) and the
// weight gradients are one tiled GEMM (gemm_dw_launch, glu_gemm.hip) on the
// same transposed copies.
//
// After the grouped GEMV and the elementwise step (or the tiled GEMM with that
// step in its epilogue) have left dg and du ([2][M][N] bf16) at the workspace
// head, repack_kernel writes zero-padded
// operand copies:
//  * dg2, du2 [Mp16][Np]: dg and du with rows padded to 16, 32 or 64 and
//    columns to a multiple of 32 (the B operand of dh, contraction over j);
//  * dgT, duT [N][Mp32] and hT [K][Mp32]: dg, du and hidden transposed, the
//    contraction index m padded to a multiple of 32 (both operands of dW).
// Padding is +0, so it adds exact zeros to every sum.
//
// dw_mfma_kernel: dWg^T = hT . dgT^T as a [K][N] product, and dWu likewise.
// The contraction over the M rows takes one or two MFMAs per 16 x 16 tile.
// A wave owns 64 x 64 tiles of (k, j), one after another. Lane l holds k = 4(l/16)+e, j = l%16 of a
// tile; lanes l and l ^ 16 trade a tile of each pair so that every lane
// stores 8 consecutive k of one row of dW as one 16-byte store.
//
// dh_mfma_kernel: partial[split][mat][m][k] = sum over the split's rows j of
// dG[m][j] W[j][k], as D[k][m] with the contraction over j, 32 rows per MFMA.
// A workgroup of 4 waves owns 128 columns k (64 above 64 rows of hidden) and
// one range of rows j. Per 32-row step:
//  1. every thread loads two 16-byte chunks (one above 64 rows) of Wg and of
//     Wu (8 columns of one row each, 64 columns apart), issued D steps ahead;
//  2. writes them transposed into LDS (rows past the range as zeros), pairing
//     two rows per 32-bit write through a DPP exchange;
//  3. after one barrier each wave reads its A operands (16 k x 32 j each)
//     from there and its B operands (dg2, du2: 16 rows m x 32 j) from the
//     workspace. A wave owns one 16-row tile of hidden and 8 / (tiles)
//     column subtiles (above 64 rows two tiles and all 4 subtiles), so no
//     two waves load the same B operand.
// The weights are read once. dh_reduce_kernel then adds the splits' partials
// in a fixed order and applies dh's roundings.
// No atomics anywhere: the results are bitwise reproducible.
#include "glu_backward.h"
#include "glu_device.h"
#include "glu_mfma_common.h"

namespace glu {

namespace {

constexpr int kRepackThreads = 256;
constexpr int kRepackTile = 64;       // columns per transposing workgroup, and rows of dst at most
constexpr int kMfmaBwdThreads = 256;  // 4 waves
constexpr int kDwTile = 64;           // k and j extent of a wave's dW tile
// dW tiles per wave at KS = 1 (the grid's waves stride over the tiles; at KS = 2 one per wave):
// K=2560 N=9216, whole backward: M = 16 94.4 -> 91.7 us, M = 32 111.9 -> 110.1 (5760 tiles against
// 4096 resident waves at one tile per wave); at M = 64 (KS = 2) three per wave took 133.9 against
// 131.6
constexpr int kDwTilesPerWave = 3;
constexpr int kDhStep = 32;           // weight rows per dh step (one MFMA contraction)
constexpr int kDhTS = 40;             // elements per LDS row of the transposed tile (32 rows j + 8 of padding,
                                      // 80 bytes: 16-byte aligned A reads, spread over the banks)
constexpr int kDhDepth = 4;           // steps whose loads are in flight

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
}

}  // namespace

// One launch for all the copies; workgroup b serves the job whose range of workgroups holds b.
// transpose == 0: dst[r][c] = src[r][c] (Rp rows of Cp elements), one element per thread, or with
// vec 8 (one 16-byte load and store).
// transpose != 0: dst[c][r] = src[r][c] (C rows of Rp elements): a workgroup moves a tile of 64
// columns x 64 rows (rows 64 rt .. of src, rt = the workgroup's row tile) through LDS, reading rows
// of src and writing rows of dst, both contiguous (with vec in 16-byte pieces on both sides).
// Entries with r >= R or c >= C are +0.  vec requires 16-byte aligned src and dst, ld, C and the
// padded row length (Cp, or Rp when transposing) multiples of 8: a piece of 8 is then wholly inside
// or wholly outside the source.
__global__ void __launch_bounds__(kRepackThreads)
repack_kernel(RepackJobs jobs)
{
    __shared__ uint16_t tile[kRepackTile][kRepackTile + 2];  // [r][c]; odd word stride spreads the banks
    const int64_t b = blockIdx.x;
    int q = 0;
    while (q + 1 < jobs.n && b >= jobs.job[q + 1].first_block) ++q;  // uniform over the workgroup
    const RepackJob& jb = jobs.job[q];
    const int64_t bl = b - jb.first_block;
    if (bl < 0 || bl >= jb.nblocks) return;  // whole workgroup
    const u32x4_t z = {0u, 0u, 0u, 0u};
    if (!jb.transpose) {
        if (jb.vec) {
            const int64_t cp8 = jb.Cp / 8;
            const int64_t x = bl * kRepackThreads + threadIdx.x;  // piece of 8
            if (x >= (int64_t)jb.Rp * cp8) return;  // no barrier in this branch
            const int64_t r = x / cp8, c = (x - r * cp8) * 8;
            const u32x4_t v =
                (r < jb.R && c < jb.C) ? *reinterpret_cast<const u32x4_t*>(jb.src + r * jb.ld + c) : z;
            *reinterpret_cast<u32x4_t*>(jb.dst + 8 * x) = v;
            return;
        }
        const int64_t x = bl * kRepackThreads + threadIdx.x;
        if (x >= (int64_t)jb.Rp * jb.Cp) return;  // no barrier in this branch
        const int64_t r = x / jb.Cp, c = x - (x / jb.Cp) * jb.Cp;
        jb.dst[x] = (r < jb.R && c < jb.C) ? jb.src[r * jb.ld + c] : (uint16_t)0;
        return;
    }
    const int rtiles = (jb.Rp + kRepackTile - 1) / kRepackTile;
    const int64_t c0 = (bl / rtiles) * kRepackTile;
    const int r0 = (int)(bl % rtiles) * kRepackTile;
    const int rn = min(kRepackTile, jb.Rp - r0);  // rows of dst's row segment this tile writes
    if (jb.vec) {
        // 64 rows x 8 pieces of 8 columns
        for (int i = threadIdx.x; i < kRepackTile * (kRepackTile / 8); i += kRepackThreads) {
            const int r = i / (kRepackTile / 8), cc = 8 * (i % (kRepackTile / 8));
            const int64_t c = c0 + cc;
            const u32x4_t v = (r0 + r < jb.R && c < jb.C)
                                  ? *reinterpret_cast<const u32x4_t*>(jb.src + (int64_t)(r0 + r) * jb.ld + c)
                                  : z;
            __builtin_memcpy(&tile[r][cc], &v, sizeof(v));  // columns cc .. cc + 7 of tile row r
        }
    } else {
        for (int i = threadIdx.x; i < kRepackTile * kRepackTile; i += kRepackThreads) {
            const int r = i / kRepackTile, cc = i % kRepackTile;
            const int64_t c = c0 + cc;
            tile[r][cc] = (r0 + r < jb.R && c < jb.C) ? jb.src[(int64_t)(r0 + r) * jb.ld + c] : (uint16_t)0;
        }
    }
    __syncthreads();
    if (jb.vec) {
        // dst row c: rn / 8 pieces of 8 consecutive r
        const int rp8 = rn / 8;
        for (int i = threadIdx.x; i < kRepackTile * rp8; i += kRepackThreads) {
            const int cc = i / rp8, r = 8 * (i % rp8);
            const int64_t c = c0 + cc;
            if (c < jb.C) {
                u32x4_t v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = (uint32_t)tile[r + 2 * e][cc] | ((uint32_t)tile[r + 2 * e + 1][cc] << 16);
                }
                *reinterpret_cast<u32x4_t*>(jb.dst + c * jb.Rp + r0 + r) = v;
            }
        }
    } else {
        for (int i = threadIdx.x; i < kRepackTile * rn; i += kRepackThreads) {
            const int cc = i / rn, r = i % rn;
            const int64_t c = c0 + cc;
            if (c < jb.C) jb.dst[c * jb.Rp + r0 + r] = tile[r][cc];
        }
    }
}

// KS = Mp32 / 32 (1 or 2).  ktiles = ceil(K / 64); wave tiles ntiles = ktiles * ceil(N / 64).
// Persistent: wave w takes tiles w, w + W, w + 2W, ... (W waves in the grid), one after another.
// (Loading the next tile's operands during the current tile's stores takes a second register set:
// 2 waves per SIMD instead of 4 at KS = 1, and the whole backward measured slower at M = 64.)
template <int KS>
__global__ void __launch_bounds__(kMfmaBwdThreads)
dw_mfma_kernel(const uint16_t* __restrict__ hT, const uint16_t* __restrict__ dgT, const uint16_t* __restrict__ duT,
               uint16_t* __restrict__ dwg, uint16_t* __restrict__ dwu, int N, int K, int ktiles, int64_t ntiles)
{
    constexpr int MP = 32 * KS;
    constexpr int T = kDwTile / 16;  // 16 x 16 tiles per side
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * (kMfmaBwdThreads / kWave);
    int64_t tile = (int64_t)blockIdx.x * (kMfmaBwdThreads / kWave) + (threadIdx.x / kWave);
    if (tile >= ntiles) return;  // whole wave; no barriers below
    const int i16 = lane & 15, q = lane >> 4;

    auto load = [&](int64_t tl, u32x4_t (&a)[KS][T], u32x4_t (&bg)[KS][T], u32x4_t (&bu)[KS][T]) {
        const int k0 = (int)(tl % ktiles) * kDwTile;
        const int64_t j0 = (tl / ktiles) * kDwTile;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                // rows past K or N re-read the last row: their results are never stored
                const int64_t k = min(k0 + 16 * t + i16, K - 1);
                const int64_t j = min(j0 + 16 * t + i16, (int64_t)N - 1);
                a[ks][t] = *reinterpret_cast<const u32x4_t*>(hT + k * MP + 32 * ks + 8 * q);
                bg[ks][t] = *reinterpret_cast<const u32x4_t*>(dgT + j * MP + 32 * ks + 8 * q);
                bu[ks][t] = *reinterpret_cast<const u32x4_t*>(duT + j * MP + 32 * ks + 8 * q);
            }
        }
    };

    auto emit = [&](int64_t tl, const u32x4_t (&a)[KS][T], const u32x4_t (&bg)[KS][T],
                    const u32x4_t (&bu)[KS][T]) {
        const int k0 = (int)(tl % ktiles) * kDwTile;
        const int64_t j0 = (tl / ktiles) * kDwTile;
#pragma unroll
        for (int tj = 0; tj < T; ++tj) {
            f32x4_t cg[T], cu[T];
#pragma unroll
            for (int tk = 0; tk < T; ++tk) {
                cg[tk] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                cu[tk] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    cg[tk] = mfma16(a[ks][tk], bg[ks][tj], cg[tk]);
                    cu[tk] = mfma16(a[ks][tk], bu[ks][tj], cu[tk]);
                }
            }
            // Lane (l%16, q = l/16) holds columns 16 tk + 4q .. +3 of row j for each tile tk.  Lanes q
            // and q ^ 1 (l ^ 16) trade one tile of a pair (tk, tk + 1): the even q then holds 8
            // consecutive columns of tile tk, the odd q 8 of tile tk + 1, so each lane stores 16 bytes
            // and four lanes write 64 contiguous bytes of the row.  Plain stores: nontemporal ones
            // measured 1.3-1.7x slower for the whole backward.
            const int64_t j = j0 + 16 * tj + i16;
            const bool oddq = (q & 1) != 0;
#pragma unroll
            for (int tk = 0; tk < T; tk += 2) {
#pragma unroll
                for (int mat = 0; mat < 2; ++mat) {
                    const f32x4_t& c0 = mat == 0 ? cg[tk] : cu[tk];
                    const f32x4_t& c1 = mat == 0 ? cg[tk + 1] : cu[tk + 1];
                    const uint32_t a0 = pack_bf16x2(c0[0], c0[1]), a1 = pack_bf16x2(c0[2], c0[3]);
                    const uint32_t b0 = pack_bf16x2(c1[0], c1[1]), b1 = pack_bf16x2(c1[2], c1[3]);
                    const uint32_t s0 = oddq ? a0 : b0, s1 = oddq ? a1 : b1;
                    const uint32_t r0 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)s0, 0x401F);  // lane ^ 16
                    const uint32_t r1 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)s1, 0x401F);
                    const u32x4_t v = oddq ? u32x4_t{r0, r1, b0, b1} : u32x4_t{a0, a1, r0, r1};
                    const int k = k0 + 16 * (tk + (oddq ? 1 : 0)) + 4 * (q & 2);  // a multiple of 8: k < K covers k + 7
                    if (j < N && k < K) *reinterpret_cast<u32x4_t*>((mat == 0 ? dwg : dwu) + j * K + k) = v;
                }
            }
        }
    };

    u32x4_t a[KS][T], bg[KS][T], bu[KS][T];
    for (; tile < ntiles; tile += nwaves) {
        load(tile, a, bg, bu);
        emit(tile, a, bg, bu);
    }
}

// MT = Mp16 / 16 (1, 2, 4, 8 or 16).  Workgroup b: columns [KK (t % ktiles), +KK), rows j of split
// t / ktiles: [split * jr, min(N, (split + 1) * jr)), jr a multiple of 32, where t = b with one
// slice of rows of hidden.  Above 64 rows (mslices >= 1, MT = 8 or 16) t = b' / mslices and the
// workgroup takes rows 16 MT (b' % mslices) .. + 16 MT - 1 of hidden, b' being b renumbered so that the workgroups one
// XCD receives (the hardware deals them to the 8 XCDs in turn) are consecutive: the slices of one
// (column tile, split) then run on one XCD and read its weight tile from that XCD's L2 after the
// first.  g2, u2: dg2, du2 ([mslices * Mp16][np] with np a multiple of 32).  partial:
// [splits][2][M][K] fp32.
// KK = dh_cols(MT) columns k per workgroup: 128 up to MT = 4 (8 column subtiles; each thread loads two
// 16-byte chunks of its weight row per step, so a workgroup reads 256 contiguous bytes of each row),
// 64 at MT = 8 and 16.
template <int MT>
__global__ void __launch_bounds__(kMfmaBwdThreads)
dh_mfma_kernel(const uint16_t* __restrict__ gate_w, const uint16_t* __restrict__ up_w,
               const uint16_t* __restrict__ g2, const uint16_t* __restrict__ u2, float* __restrict__ partial, int M,
               int N, int K, int np, int ktiles, int jr, int mslices)
{
    constexpr int D = MT > 8 ? 2 : kDhDepth;  // 16 row tiles: four per wave, so two steps in flight
    constexpr int KK = dh_cols(MT);
    constexpr int NKS = KK / 16;  // column subtiles of 16
    constexpr int HALVES = KK / 64;
    __shared__ __align__(16) uint16_t tw[2][2][KK * kDhTS];  // [buffer][matrix][k][j]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    int bt = (int)blockIdx.x;
    if (mslices > 1) {
        const int G = (int)gridDim.x, per = G >> 3, rem = G & 7, xcd = bt & 7, slot = bt >> 3;
        bt = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
    }
    const int mbase = 16 * MT * (bt % mslices);
    bt /= mslices;
    const int k0 = (bt % ktiles) * KK;
    const int split = bt / ktiles;
    const int jb = split * jr;
    const int je = min(jb + jr, N);
    const int nsteps = (je - jb + kDhStep - 1) / kDhStep;  // >= 1: the plan leaves no split empty
    const int i16 = lane & 15, q = lane >> 4;
    // the NKS x MT (column subtile, row tile) pairs: up to MT = 4 wave w takes row tile w % MT of hidden
    // and the KT column subtiles from (w / MT) KT on; at MT = 8 (16) it takes row tiles w, w + 4 (and
    // w + 8, w + 12) and all column subtiles.  No two waves load the same B operand.
    constexpr int RT = MT > 4 ? MT / 4 : 1;             // row tiles per wave
    constexpr int KT = MT > 4 ? NKS : MT * NKS / 4;     // column subtiles per wave
    const int mt = MT > 4 ? wave : wave % MT;  // the wave's first row tile; the others 4 apart
    const int ks0 = MT > 4 ? 0 : (wave / MT) * KT;

    // this thread's weight chunks: row r_ld of the step, columns k0 + 64 h + 8 c_ld .. + 7 (h < HALVES)
    const int r_ld = tid >> 3, c_ld = tid & 7;
    bool col_ok[HALVES];
    int kc[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        col_ok[h] = k0 + 64 * h + 8 * c_ld < K;
        kc[h] = col_ok[h] ? k0 + 64 * h + 8 * c_ld : K - 8;  // in bounds; such columns are stored as zeros
    }

    auto load = [&](int s, u32x4_t (&w)[HALVES][2], u32x4_t (&b)[RT][2]) __attribute__((always_inline)) {
        const int64_t j = min(jb + kDhStep * s + r_ld, N - 1);  // rows past the range: stored as zeros
#pragma unroll
        for (int h = 0; h < HALVES; ++h) {
            w[h][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(gate_w + j * K + kc[h]));
            w[h][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(up_w + j * K + kc[h]));
        }
        // B: rows m = 16 (mt + 4 r) + l%16 of dg2 and du2, columns jb + 32 s + 8 (l/16) .. + 7 (zero
        // past N)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int64_t off = (int64_t)(mbase + 16 * (mt + 4 * r) + i16) * np + jb + kDhStep * s + 8 * q;
            b[r][0] = *reinterpret_cast<const u32x4_t*>(g2 + off);
            b[r][1] = *reinterpret_cast<const u32x4_t*>(u2 + off);
        }
    };
    // Transposed publication.  Rows r and r ^ 1 of a chunk column sit in lanes l and l ^ 8, which
    // trade half their chunk through one DPP row rotation by 8: the even row's thread then holds
    // columns 8c .. 8c+3 and the odd row's 8c+4 .. 8c+7 of both rows, and writes them as four
    // 32-bit (row, row + 1) pairs.  Element (k, j) sits at T[k][8 ((j >> 3) ^ ((k >> 4) & 3)) + (j & 7)]:
    // the 64 lanes of one write then hit 64 different banks (the second 64 columns repeat the first
    // ones' pattern, KK * kDhTS / 2 words further on: a multiple of the 64 banks), and an A read of
    // column subtile ks still takes 16 contiguous bytes per lane.
    const bool odd = (r_ld & 1) != 0;
    auto publish = [&](int buf, int s, const u32x4_t (&w)[HALVES][2]) __attribute__((always_inline)) {
        const bool row_ok = jb + kDhStep * s + r_ld < je;
        const int jo = r_ld & 6;  // the pair's first row within its block of 8
#pragma unroll
        for (int hm = 0; hm < 2 * HALVES; ++hm) {
            const int h = hm >> 1, mat = hm & 1;
            const int kb = 64 * h + 8 * c_ld + (odd ? 4 : 0);
            const u32x4_t z = {0u, 0u, 0u, 0u};
            const u32x4_t v = (row_ok && col_ok[h]) ? w[h][mat] : z;
            const uint32_t s0 = odd ? v[0] : v[2], s1 = odd ? v[1] : v[3];
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0x128, 0xF, 0xF, false);
            const uint32_t r1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0x128, 0xF, 0xF, false);
            // lo: four columns of the even row, hi: the same columns of the odd row
            const uint32_t lo0 = odd ? r0 : v[0], lo1 = odd ? r1 : v[1];
            const uint32_t hi0 = odd ? v[2] : r0, hi1 = odd ? v[3] : r1;
            const uint32_t pr[4] = {(lo0 & 0xFFFFu) | (hi0 << 16), (lo0 >> 16) | (hi0 & 0xFFFF0000u),
                                    (lo1 & 0xFFFFu) | (hi1 << 16), (lo1 >> 16) | (hi1 & 0xFFFF0000u)};
            uint32_t* t = reinterpret_cast<uint32_t*>(&tw[buf][mat][0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = kb + e;
                t[(k * kDhTS + 8 * (wave ^ ((k >> 4) & 3)) + jo) >> 1] = pr[e];
            }
        }
    };

    f32x4_t acc[2][RT][KT];
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
#pragma unroll
            for (int t = 0; t < KT; ++t) acc[mat][r][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    auto compute = [&](int buf, const u32x4_t (&b)[RT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int mat = 0; mat < 2; ++mat) {
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int ks = ks0 + t;  // column subtile: k >> 4 == ks, the read's swizzle
                const u32x4_t a =
                    *reinterpret_cast<const u32x4_t*>(&tw[buf][mat][(16 * ks + i16) * kDhTS + 8 * (q ^ (ks & 3))]);
#pragma unroll
                for (int r = 0; r < RT; ++r) acc[mat][r][t] = mfma16(a, b[r][mat], acc[mat][r][t]);
            }
        }
    };

    u32x4_t W[D][HALVES][2];
    u32x4_t B[D][RT][2];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        if (s < nsteps) load(s, W[s], B[s]);
    }
    // step s (s % D == Q): publish its weights, one barrier, its MFMAs, then refill its registers
    // with step s + D.  D is even, so the LDS buffer s & 1 is Q & 1.  In the steady state every
    // refill is live and nothing branches around a load, so the waits leave D - 1 steps in flight.
    auto stage = [&](auto Qc, auto tailc, int s) __attribute__((always_inline)) {
        constexpr int Q = decltype(Qc)::value;
        constexpr bool TAIL = decltype(tailc)::value;
        publish(Q & 1, s, W[Q]);
        __syncthreads();
        compute(Q & 1, B[Q]);
        if (!TAIL || s + D < nsteps) load(s + D, W[Q], B[Q]);
    };
    auto steady = [&](auto Qc, int s) __attribute__((always_inline)) { stage(Qc, std::false_type{}, s); };
    auto tail = [&](auto Qc, int s) __attribute__((always_inline)) { stage(Qc, std::true_type{}, s); };
    int s0 = 0;
    for (; s0 + 2 * D <= nsteps; s0 += D) run_stages<0, D>(steady, s0, nsteps);
    for (; s0 < nsteps; s0 += D) run_stages<0, D>(tail, s0, nsteps);

    // lane l holds D[4(l/16) + e][l%16]: columns k = k0 + 16 ks + 4(l/16) + e of row
    // m = 16 (mt + 4 r) + l%16
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int m = mbase + 16 * (mt + 4 * r) + i16;
#pragma unroll
        for (int mat = 0; mat < 2; ++mat) {
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int k = k0 + 16 * (ks0 + t) + 4 * q;
                if (m < M && k < K) {
                    *reinterpret_cast<f32x4_t*>(partial + (((int64_t)split * 2 + mat) * M + m) * K + k) =
                        acc[mat][r][t];
                }
            }
        }
    }
}

hipError_t repack_launch(RepackJobs jobs, hipStream_t stream)
{
    if (jobs.n < 1 || jobs.n > kMaxRepackJobs) return hipErrorInvalidValue;
    int64_t grid = 0;
    for (int q = 0; q < jobs.n; ++q) {
        RepackJob& j = jobs.job[q];
        if (j.R > j.Rp || j.R < 0 || j.C < 0) return hipErrorInvalidValue;
        if (!j.transpose && j.C > j.Cp) return hipErrorInvalidValue;
        const bool al = (((uintptr_t)j.src | (uintptr_t)j.dst) & 15u) == 0 && j.ld % 8 == 0 && j.C % 8 == 0;
        j.vec = al && (j.transpose ? j.Rp % 8 == 0 : j.Cp % 8 == 0) ? 1 : 0;
        const int64_t per_thread = j.vec ? 8 : 1;
        j.nblocks = j.transpose ? ((int64_t)j.C + kRepackTile - 1) / kRepackTile *
                                      (((int64_t)j.Rp + kRepackTile - 1) / kRepackTile)
                                : ((int64_t)j.Rp * j.Cp / per_thread + kRepackThreads - 1) / kRepackThreads;
        j.first_block = grid;
        grid += j.nblocks;
    }
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(repack_kernel, dim3((unsigned)grid), dim3(kRepackThreads), 0, stream, jobs);
    return hipGetLastError();
}

hipError_t dw_mfma_launch(const BwdPlan& p, const uint16_t* hT, const uint16_t* dgT, const uint16_t* duT,
                          uint16_t* dwg, uint16_t* dwu, int N, int K, hipStream_t stream)
{
    const int ktiles = (K + kDwTile - 1) / kDwTile;
    const int64_t ntiles = (int64_t)ktiles * ((N + kDwTile - 1) / kDwTile);
    const int64_t per_wave = p.mp32 == 32 ? kDwTilesPerWave : 1;
    const int64_t grid = (ntiles + 4 * per_wave - 1) / (4 * per_wave);
    if (p.path != kPathMfma || N < 1 || K < 8 || (K & 7) != 0 || grid < 1 || grid > 0x7fffffff) {  // M <= 64
        return hipErrorInvalidValue;
    }
    if (p.mp32 == 32) {
        hipLaunchKernelGGL(dw_mfma_kernel<1>, dim3((unsigned)grid), dim3(kMfmaBwdThreads), 0, stream, hT, dgT, duT,
                           dwg, dwu, N, K, ktiles, ntiles);
    } else if (p.mp32 == 64) {
        hipLaunchKernelGGL(dw_mfma_kernel<2>, dim3((unsigned)grid), dim3(kMfmaBwdThreads), 0, stream, hT, dgT, duT,
                           dwg, dwu, N, K, ktiles, ntiles);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t dh_mfma_launch(const BwdPlan& p, int M, const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* g2,
                          const uint16_t* u2, float* partial, int N, int K, hipStream_t stream)
{
    using Fn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, float*, int, int, int,
                        int, int, int, int);
    static const Fn table[16] = {dh_mfma_kernel<1>, dh_mfma_kernel<2>, nullptr, dh_mfma_kernel<4>,
                                 nullptr,           nullptr,           nullptr, dh_mfma_kernel<8>,
                                 nullptr,           nullptr,           nullptr, nullptr,
                                 nullptr,           nullptr,           nullptr, dh_mfma_kernel<16>};
    const int mt = p.mp16 / 16;
    const int ktiles = (K + dh_cols(mt) - 1) / dh_cols(mt);
    const int ms = p.dh_mslices;
    // slices of 128 rows (MT = 8) above 64 rows of hidden, one slice of up to 64 rows below
    if ((p.path != kPathMfma && p.path != kPathGemm) || mt < 1 || mt > 16 || !table[mt - 1] || ms < 1 ||
        (p.path == kPathGemm) != (mt >= 8) || (ms > 1 && mt < 8) || M < 1 || M > (int64_t)ms * p.mp16 ||
        N < 1 || K < 8 || (K & 7) != 0 ||
        p.dh_jr < kDhStep || p.dh_jr % kDhStep != 0 || p.np32 < N || p.np32 % kDhStep != 0 || p.dh_splits < 1 ||
        (int64_t)(p.dh_splits - 1) * p.dh_jr >= N || (int64_t)p.dh_splits * p.dh_jr < N ||
        p.dh_splits != p.nranges) {
        return hipErrorInvalidValue;
    }
    const int64_t grid = (int64_t)ktiles * p.dh_splits * ms;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(table[mt - 1], dim3((unsigned)grid), dim3(kMfmaBwdThreads), 0, stream, gate_w, up_w, g2, u2,
                       partial, M, N, K, p.np32, ktiles, p.dh_jr, ms);
    return hipGetLastError();
}

}  // namespace glu
