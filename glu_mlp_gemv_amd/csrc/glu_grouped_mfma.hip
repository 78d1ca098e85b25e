// Grouped GEMV at batch M >= 2: the block-diagonal MFMA layouts of the dual
// kernels (glu_mfma.hip: 4 rows x 4 blocks; glu_mfma8.hip: 8 rows x 2 blocks,
// here for 8 < M <= 32 with hidden in LDS) with one weight stream.
//
// The virtual row space of the n projections (glu_grouped.hip) is cut into
// groups of 4 rows; every projection's row count is a multiple of 4, so a
// group never straddles two projections and is addressed as a wave-uniform
// base plus 32-bit lane offsets.  v_mfma_f32_16x16x32_bf16 takes A = the
// group's 4 weight rows x 4 K-blocks of 32 (one 16-byte load per lane reads
// 4 rows x 256 contiguous bytes) and B = 4 hidden rows x the same blocks; the
// diagonal blocks of D are the partial dots, summed over segments in the
// accumulator and over blocks by two DPP steps.  Persistent waves stream
// their groups in stages of U segments with a two-buffer register pipeline.
// hidden lives whole in LDS (XOR-swizzled, conflict-free operand reads) or,
// when it does not fit, is read from L2 with each stage.  The epilogue rounds
// each sum once to bf16 and writes it to its projection's output row.
#include "glu_device.h"
#include "glu_grouped.h"
#include "glu_mfma_common.h"

namespace glu {

namespace {

// base of virtual row `row` (a multiple of 4) and the stride of its projection
struct GroupRef {
    const uint16_t* w;
    int64_t ldw;
};

__device__ __forceinline__ GroupRef group_ref(const GroupDesc& d, int row)
{
    const uint16_t* w = d.w[0];
    int64_t ldw = d.ldw[0];
    int local = row;
#pragma unroll
    for (int t = 1; t < kGroupMax; ++t) {
        const bool in = t < d.n && row >= d.row0[t];
        w = in ? d.w[t] : w;
        ldw = in ? d.ldw[t] : ldw;
        local = in ? row - d.row0[t] : local;
    }
    return GroupRef{w + (int64_t)local * ldw, ldw};
}

}  // namespace

// ROWS = 4: MT4 hidden-row tiles of 4 (M <= 4*MT4), U segments of 128 elements per stage, 4 weight
// rows x 4 K-blocks per MFMA.  ROWS = 8 (hidden in LDS, K/8 a multiple of 16): MT4 tiles of 8
// hidden rows (M <= 8*MT4), U segments of 64 elements, 8 weight rows x 2 K-blocks per MFMA as in
// the dual kernel's 8-row layout (half of D useful: per weight byte half the MFMAs and LDS reads).
// nsg: stages per group (nsg*U*segment >= K/8, equality unless RAGGED); d.rows % ROWS == 0.
// Dynamic LDS when HLDS: M * K * 2 bytes, or M * (K/8 + 1) * 16 when K/8 is not a multiple of 4
// (up to the 160 KiB of one workgroup: M = 32 at K = 2560).
template <int MT4, int U, bool HLDS, bool RAGGED, int ROWS = 4>
__global__ void __launch_bounds__(kMfmaMaxThreads)
grouped_mfma_kernel(const uint16_t* __restrict__ hidden, int64_t ldh, int M, int K, GroupDesc d, int nsg)
{
    static_assert(ROWS == 4 || (ROWS == 8 && HLDS), "8 rows per group with hidden in LDS only");
    constexpr int SEGC = ROWS == 4 ? 16 : 8;  // 16-byte chunks of a row per segment
    extern __shared__ u32x4_t h_lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + threadIdx.x / kWave);
    const int nwaves = gridDim.x * wpb;
    const int nchunks = K >> 3;
    const uint32_t ldh8 = (uint32_t)(ldh >> 3);
    const int i16 = lane & 15;
    // weight row of this lane's A data (also its hidden row within a tile) and its 16-byte chunk of
    // a segment: 4 rows x 4 blocks of 32, or 8 rows x 2 blocks
    const int rho_a = ROWS == 4 ? i16 >> 2 : i16 >> 1;
    const int cseg = ROWS == 4 ? (i16 & 3) * 4 + (lane >> 4) : (i16 & 1) * 4 + (lane >> 4);
    auto swz = [](int r) __attribute__((always_inline)) { return ROWS == 4 ? lds_swz4(r) : lds_swz8(r); };
    const u32x4_t* h4 = reinterpret_cast<const u32x4_t*>(hidden);

    const bool hswz = (nchunks & 3) == 0;
    const int hpitch = hswz ? nchunks : nchunks + 1;
    if constexpr (HLDS) {
        // kStageLoads loads in flight per lane (indices past the end re-read the last chunk), then their stores
        constexpr int kStageLoads = 8;
        const int total = M * nchunks;
        for (int i0 = threadIdx.x; i0 < total; i0 += kStageLoads * (int)blockDim.x) {
            u32x4_t v[kStageLoads];
#pragma unroll
            for (int q = 0; q < kStageLoads; ++q) {
                const int i = min(i0 + q * (int)blockDim.x, total - 1);
                const int m = i / nchunks;
                v[q] = h4[(uint32_t)m * ldh8 + (uint32_t)(i - m * nchunks)];
            }
#pragma unroll
            for (int q = 0; q < kStageLoads; ++q) {
                const int i = i0 + q * (int)blockDim.x;
                if (i < total) {
                    const int m = i / nchunks;
                    const int c = i - m * nchunks;
                    h_lds[m * hpitch + (hswz ? c ^ swz(m) : c)] = v[q];
                }
            }
        }
        __syncthreads();
    }

    const int ngroups = d.rows / ROWS;
    if (wave_id >= ngroups) return;  // no barrier follows
    const int my_groups = (ngroups - 1 - wave_id) / nwaves + 1;
    const int nstages = my_groups * nsg;

    int hrow[MT4];  // hidden rows of this lane's B data (rows past M repeat row M-1, never stored)
#pragma unroll
    for (int t = 0; t < MT4; ++t) hrow[t] = min(ROWS * t + rho_a, M - 1);

    constexpr int BT = HLDS ? 1 : MT4;
    constexpr int BU = HLDS ? 1 : U;

    auto load = [&](int s, u32x4_t (&A)[U], u32x4_t (&Bq)[BT][BU]) {
        const int gi = s / nsg;
        const int sb = s - gi * nsg;
        const GroupRef ref = group_ref(d, ROWS * (wave_id + gi * nwaves));
        const char* wp = reinterpret_cast<const char*>(ref.w);
        const uint32_t ldw8 = (uint32_t)(ref.ldw >> 3);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = (sb * U + u) * SEGC + cseg;
            if (RAGGED) c = min(c, nchunks - 1);
            const uint32_t off = ((uint32_t)rho_a * ldw8 + (uint32_t)c) * 16u;  // bytes, below ROWS rows at the stride
            A[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp + off));
        }
        if constexpr (!HLDS) {
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int c = (sb * U + u) * SEGC + cseg;
                    if (RAGGED) c = min(c, nchunks - 1);
                    const uint32_t off = ((uint32_t)hrow[t] * ldh8 + (uint32_t)c) * 16u;
                    Bq[t][u] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(hidden) + off);
                }
            }
        }
    };

    f32x4_t acc[MT4];

    auto finish_group = [&](int g) {
        if constexpr (ROWS == 8) {
            // lanes l and l^1 hold the two blocks of the same (weight row, hidden row) pairs:
            // entries l%2 (weight row 2(l/16)) and 2 + l%2 (row 2(l/16) + 1); one DPP step adds them
            const bool odd = (lane & 1) != 0;
            const int row = 8 * g + 2 * (lane >> 4) + (lane & 1);
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
                const f32x4_t dd = acc[t];
                float v0 = odd ? dd[1] : dd[0];
                float v1 = odd ? dd[3] : dd[2];
                v0 = dpp_add<0xB1>(v0);  // lane ^ 1
                v1 = dpp_add<0xB1>(v1);
                const int m = 8 * t + (i16 >> 1);
                if (m < M) group_store(d, m, row, f32_to_bf16_rne(odd ? v1 : v0));
            }
            return;
        }
        // useful entry e = lane % 4, then the quad sum over the four blocks
        const int e = lane & 3;
        float res[(MT4 + 3) / 4];
#pragma unroll
        for (int t = 0; t < MT4; ++t) {
            const f32x4_t dd = acc[t];
            float v = e == 0 ? dd[0] : e == 1 ? dd[1] : e == 2 ? dd[2] : dd[3];
            v = dpp_add<0xB1>(v);  // lane ^ 1
            v = dpp_add<0x4E>(v);  // lane ^ 2
            if (e == (t & 3)) res[t >> 2] = v;
        }
        // lane l keeps tiles t with t % 4 == l % 4: hidden row 4t + (l%16)/4, virtual row 4g + l/16
        const int row = 4 * g + (lane >> 4);
#pragma unroll
        for (int k = 0; k < (MT4 + 3) / 4; ++k) {
            const int t = 4 * k + e;
            const int m = 4 * t + ((lane & 15) >> 2);
            if (t < MT4 && m < M) group_store(d, m, row, f32_to_bf16_rne(res[k]));
        }
    };

    auto compute = [&](int s, const u32x4_t (&A)[U], const u32x4_t (&Bq)[BT][BU]) {
        const int gi = s / nsg;
        const int sb = s - gi * nsg;
        if (sb == 0) {
#pragma unroll
            for (int t = 0; t < MT4; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (sb * U + u) * SEGC + cseg;
            const bool ok = !RAGGED || c < nchunks;
            const int cc = RAGGED ? min(c, nchunks - 1) : c;
            const u32x4_t a = RAGGED ? (ok ? A[u] : z) : A[u];
#pragma unroll
            for (int t = 0; t < MT4; ++t) {
                u32x4_t b;
                if constexpr (HLDS) {
                    b = h_lds[hrow[t] * hpitch + (hswz ? cc ^ swz(hrow[t]) : cc)];
                } else {
                    b = Bq[t][u];
                }
                if constexpr (RAGGED) b = ok ? b : z;
                acc[t] = mfma16(a, b, acc[t]);
            }
        }
        if (sb == nsg - 1) finish_group(wave_id + gi * nwaves);
    };

    u32x4_t a0[U], a1[U], b0[BT][BU], b1[BT][BU];
    load(0, a0, b0);
    int s = 0;
    while (true) {
        if (s + 1 >= nstages) {
            compute(s, a0, b0);
            break;
        }
        load(s + 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any of this stage's math
        compute(s, a0, b0);
        ++s;
        if (s + 1 >= nstages) {
            compute(s, a1, b1);
            break;
        }
        load(s + 1, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute(s, a1, b1);
        ++s;
    }
}

// 8-row layout with hidden staged in K-slices (above 8 rows of hidden): the slice-major walk of the
// dual kernel's mfma8_pass_kernel with one weight stream.  The W = 4 waves of a workgroup own
// blocks of 4 consecutive 8-row groups (blocks blockIdx.x + j * gridDim.x, j < jb <= JBMAX) and walk
// K once for all of them: stage t is (slice t / jb, block t % jb).  Each K-slice of all M hidden rows
// (U * 64 elements) is loaded once per workgroup into registers one slice ahead, published to the
// other half of a two-slice LDS ring after the slice's last stage, and read by every block's stage;
// one barrier per slice.  Instead of staging all of hidden into every workgroup's LDS before its
// first weight load (M * K * 2 bytes: 160 KiB at M = 32, K = 2560, as much traffic as a 31 MB
// projection set's weights over the chip), the slices stream under the weights.  The per-output
// summation order is that of the 8-row grouped kernel with hidden whole in LDS: bitwise equal.
// Dynamic LDS: 2 * 8 * MT8 * U * 8 * 16 bytes.  blockDim.x == 256.
template <int MT8, int U, int JBMAX, bool RAGGED>
__global__ void __launch_bounds__(kMfmaMaxThreads)
grouped_slice_kernel(const uint16_t* __restrict__ hidden, int64_t ldh, int M, int K, GroupDesc d, int nsg)
{
    constexpr int W = kMfmaMaxThreads / kWave;
    constexpr int MP = 8 * MT8;
    constexpr int SC = U * 8;  // 16-byte chunks of a row in one slice
    static_assert(SC % 16 == 0, "the LDS swizzle permutes 16-chunk blocks of a row");
    constexpr int HPT = (MP * SC + kMfmaMaxThreads - 1) / kMfmaMaxThreads;
    extern __shared__ u32x4_t hs[];  // [2][MP][SC], chunk c of row r at c ^ lds_swz8(r)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K >> 3;
    const uint32_t ldh8 = (uint32_t)(ldh >> 3);
    const int i16 = lane & 15;
    const int rho = i16 >> 1;                     // weight row (A) and hidden row (B) in its group / tile
    const int cw = (i16 & 1) * 4 + (lane >> 4);  // 16-byte chunk within a 64-element segment
    const u32x4_t* h4 = reinterpret_cast<const u32x4_t*>(hidden);

    const int ngroups = d.rows / 8;
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
    auto load_w = [&](int sb, int j, u32x4_t (&A)[U]) __attribute__((always_inline)) {
        const int g = min(group_of(j), ngroups - 1);  // past the last group: re-read it, never stored
        const GroupRef ref = group_ref(d, 8 * g);     // wave-uniform base, 32-bit lane offsets
        const char* wp = reinterpret_cast<const char*>(ref.w);
        const uint32_t ldw8 = (uint32_t)(ref.ldw >> 3);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int c = (sb * U + u) * 8 + cw;
            if (RAGGED) c = min(c, nchunks - 1);
            A[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp + ((uint32_t)rho * ldw8 + (uint32_t)c) * 16u));
        }
    };

    auto finish_group = [&](int g, const f32x4_t (&acc)[MT8]) __attribute__((always_inline)) {
        if (g >= ngroups) return;
        // lanes l and l^1 hold the two blocks of the same (weight row, hidden row) pairs:
        // entries l%2 (weight row 2(l/16)) and 2 + l%2 (row 2(l/16) + 1); one DPP step adds them
        const bool odd = (lane & 1) != 0;
        const int row = 8 * g + 2 * (lane >> 4) + (lane & 1);
#pragma unroll
        for (int t = 0; t < MT8; ++t) {
            const f32x4_t dd = acc[t];
            float v0 = odd ? dd[1] : dd[0];
            float v1 = odd ? dd[3] : dd[2];
            v0 = dpp_add<0xB1>(v0);  // lane ^ 1
            v1 = dpp_add<0xB1>(v1);
            const int m = 8 * t + (i16 >> 1);
            if (m < M) group_store(d, m, row, f32_to_bf16_rne(odd ? v1 : v0));
        }
    };

    auto compute = [&](int sb, const u32x4_t (&A)[U], f32x4_t (&acc)[MT8]) __attribute__((always_inline)) {
        if (sb == 0) {
#pragma unroll
            for (int t = 0; t < MT8; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
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
            const u32x4_t a = RAGGED ? (ok ? A[u] : z) : A[u];
#pragma unroll
            for (int t = 0; t < MT8; ++t) {
                u32x4_t bt = b[u & 1][t];
                if constexpr (RAGGED) bt = ok ? bt : z;
                acc[t] = mfma16(a, bt, acc[t]);
            }
        }
    };

    auto body = [&](auto JBc) __attribute__((always_inline)) {
        constexpr int JB = decltype(JBc)::value;
        constexpr int L = 2 * JB;  // stages per unrolled step: weight slot t % 2 and block t % JB are static
        u32x4_t A[2][U];           // weights of stage t in A[t % 2]
        u32x4_t hr[HPT];           // the next K-slice of hidden, between its load and its publication
        f32x4_t acc[JB][MT8];

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
            __builtin_amdgcn_sched_barrier(0);  // the prefetches are issued before any of this stage's math
            compute(sb, A[slot], acc[j]);
            if constexpr (j == JB - 1) {
                if (more) store_h(sb + 1, hr);
                __syncthreads();
            }
            if (TAIL && sb == nsg - 1) finish_group(group_of(j), acc[j]);
        };
        auto steps = [&](auto tailc, int sp) __attribute__((always_inline)) {
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

namespace {

using GroupedMfmaFn = void (*)(const uint16_t*, int64_t, int, int, GroupDesc, int);

template <int MT4, bool HL, bool RG>
GroupedMfmaFn pick_u(int U)
{
    switch (U) {
    case 2: return grouped_mfma_kernel<MT4, 2, HL, RG>;
    case 4: if constexpr (HL) return grouped_mfma_kernel<MT4, 4, HL, RG>; else return nullptr;
    case 5: if constexpr (HL) return grouped_mfma_kernel<MT4, 5, HL, RG>; else return nullptr;
    default: return nullptr;
    }
}

// 8 rows per group: tiles of 8 hidden rows (MT8 = 2 to 4: 8 < M <= 32), hidden in LDS
template <int MT8, bool RG>
GroupedMfmaFn pick8_u(int U)
{
    switch (U) {
    case 5: return grouped_mfma_kernel<MT8, 5, true, RG, 8>;
    case 8: return grouped_mfma_kernel<MT8, 8, true, RG, 8>;
    default: return nullptr;
    }
}

// 5 to 8 tiles of hidden rows (33..64 rows): stages of 4 or 8 segments (a 64 or 128 KiB ring)
template <int U>
GroupedMfmaFn pick_slices64(int mt8, bool ragged)
{
    switch (mt8) {
    case 5: return ragged ? grouped_slice_kernel<5, U, kPassBlocks, true> : grouped_slice_kernel<5, U, kPassBlocks, false>;
    case 6: return ragged ? grouped_slice_kernel<6, U, kPassBlocks, true> : grouped_slice_kernel<6, U, kPassBlocks, false>;
    case 7: return ragged ? grouped_slice_kernel<7, U, kPassBlocks, true> : grouped_slice_kernel<7, U, kPassBlocks, false>;
    case 8: return ragged ? grouped_slice_kernel<8, U, kPassBlocks, true> : grouped_slice_kernel<8, U, kPassBlocks, false>;
    default: return nullptr;
    }
}

// 2 to 4 tiles (9..32 rows; 8 or fewer run on 2): stages of 8 segments
GroupedMfmaFn pick_slices(int mt8, int U, bool ragged)
{
    if (mt8 >= 5) return U == 8 ? pick_slices64<8>(mt8, ragged) : (U == 4 ? pick_slices64<4>(mt8, ragged) : nullptr);
    if (U != 8) return nullptr;
    switch (mt8) {
    case 2: return ragged ? grouped_slice_kernel<2, 8, kPassBlocks, true> : grouped_slice_kernel<2, 8, kPassBlocks, false>;
    case 3: return ragged ? grouped_slice_kernel<3, 8, kPassBlocks, true> : grouped_slice_kernel<3, 8, kPassBlocks, false>;
    case 4: return ragged ? grouped_slice_kernel<4, 8, kPassBlocks, true> : grouped_slice_kernel<4, 8, kPassBlocks, false>;
    default: return nullptr;
    }
}

size_t slices_lds_bytes(int mt8, int U) { return (size_t)2 * 8 * mt8 * U * 8 * 16; }

GroupedMfmaFn pick8(int mt8, int U, bool ragged)
{
    switch (mt8) {
    case 2: return ragged ? pick8_u<2, true>(U) : pick8_u<2, false>(U);
    case 3: return ragged ? pick8_u<3, true>(U) : pick8_u<3, false>(U);
    case 4: return ragged ? pick8_u<4, true>(U) : pick8_u<4, false>(U);
    default: return nullptr;
    }
}

template <int MT4>
GroupedMfmaFn pick_flags(int U, bool hlds, bool ragged)
{
    if (hlds) return ragged ? pick_u<MT4, true, true>(U) : pick_u<MT4, true, false>(U);
    return ragged ? pick_u<MT4, false, true>(U) : pick_u<MT4, false, false>(U);
}

GroupedMfmaFn pick(int mt4, int U, bool hlds, bool ragged)
{
    switch (mt4) {
    case 1: return pick_flags<1>(U, hlds, ragged);
    case 2: return pick_flags<2>(U, hlds, ragged);
    case 3: return pick_flags<3>(U, hlds, ragged);
    case 4: return pick_flags<4>(U, hlds, ragged);
    case 5: return pick_flags<5>(U, hlds, ragged);
    case 6: return pick_flags<6>(U, hlds, ragged);
    case 7: return pick_flags<7>(U, hlds, ragged);
    case 8: return pick_flags<8>(U, hlds, ragged);
    default: return nullptr;
    }
}

}  // namespace

bool grouped_mfma_supported(const MfmaConfig& c)
{
    if (c.block < kWave || c.block > kMfmaMaxThreads || c.block % kWave != 0) return false;
    if (c.rows == 8 && c.hidden == kHiddenSlices) {
        return c.block == kMfmaMaxThreads && pick_slices(c.MT4, c.U, c.ragged) &&
               slices_lds_bytes(c.MT4, c.U) <= (size_t)kLdsMax;
    }
    if (c.rows == 8) return c.hidden == kHiddenLds && pick8(c.MT4, c.U, c.ragged) != nullptr;
    if (c.rows != 4 || (c.hidden != kHiddenLds && c.hidden != kHiddenL2)) return false;
    return pick(c.MT4, c.U, c.hidden == kHiddenLds, c.ragged) != nullptr;
}

hipError_t grouped_mfma_launch(const MfmaConfig& c, int M, const uint16_t* hidden, int64_t ldh, int64_t K,
                               const GroupDesc& d, hipStream_t stream)
{
    const bool hlds = c.hidden == kHiddenLds;
    GroupedMfmaFn fn;
    if (c.rows == 8 && c.hidden == kHiddenSlices) {
        // 4 waves in lockstep; every workgroup owns at most kPassBlocks blocks of 4 groups.  A last
        // slice with fewer rows than the kernels are built for runs on their smallest tile count
        // (padded rows repeat row M - 1 and are never stored)
        const int mt0 = (M + 7) / 8;
        const int mt8 = c.U == 4 ? (mt0 < 5 ? 5 : mt0) : (mt0 < 2 ? 2 : mt0);
        fn = c.block == kMfmaMaxThreads ? pick_slices(mt8, c.U, c.ragged) : nullptr;
        const int64_t blocks = (d.rows / 8 + 3) / 4;
        if (!fn || M < 1 || M > 8 * mt8 || d.rows % 8 != 0 || (int64_t)c.grid * kPassBlocks < blocks) {
            return hipErrorInvalidValue;
        }
        const size_t lds = slices_lds_bytes(mt8, c.U);
        if (lds > (size_t)kLdsMax) return hipErrorInvalidValue;
        if (lds > (size_t)kLdsBudget) {
            // past 64 KiB of dynamic LDS the launch states its size to the runtime first
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(fn, dim3(c.grid), dim3(c.block), lds, stream, hidden, ldh, M, (int)K, d, c.nsg);
        return hipGetLastError();
    }
    if (c.rows == 8) {
        // the 8-row layout's XOR swizzle permutes 16-chunk blocks of a row of hidden in LDS
        if (!hlds || (K / 8) % 16 != 0 || d.rows % 8 != 0) return hipErrorInvalidValue;
        // a last slice of 8 rows or fewer runs on 2 tiles: padded rows repeat row M - 1, never stored
        fn = pick8(M <= 8 ? 2 : (M + 7) / 8, c.U, c.ragged);
    } else {
        fn = pick((M + 3) / 4, c.U, hlds, c.ragged);
    }
    if (!fn || M < 1 || d.rows % 4 != 0) return hipErrorInvalidValue;
    const size_t lds = hlds ? mfma_hidden_lds_bytes(M, K) : 0;
    if (lds > (size_t)kLdsMax) return hipErrorInvalidValue;
    if (lds > (size_t)kLdsBudget) {
        // past 64 KiB of dynamic LDS the launch states its size to the runtime first
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(c.grid), dim3(c.block), lds, stream, hidden, ldh, M, (int)K, d, c.nsg);
    return hipGetLastError();
}

}  // namespace glu
