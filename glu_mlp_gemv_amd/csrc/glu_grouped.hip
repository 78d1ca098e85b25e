// Grouped GEMV: n projections of one hidden, out_i = bf16(hidden @ W_i^T),
// each W_i read in place (no concatenated copy).
//
// The pages route the QKV and GatedDeltaNet input projections (three or four
// weight matrices applied to the same hidden) through single/triple/quad
// GEMV kernels, later unified behind one grouped_linear(x, weights,
// glu_epilogue) dispatcher (DeepSpeed PR #9057, commit notes); their segment
// fusion concatenates the four GDN weights into one [qkv|z|b|a] block to get
// one GEMM.  Here the n weights stay separate: the kernel streams them as one
// virtual row space of sum N_i rows, and resolves each row to its projection
// through a small table passed with the launch.  The epilogue is the bf16
// rounding of one nn.Linear output (no GLU).
//
// Work layout is that of the dual kernel's VALU GEMV (glu_valu.h): persistent
// waves own groups of R consecutive virtual rows (neighbouring waves,
// neighbouring rows), lane l streams the 16-byte chunks l, l+64, ... of each
// row with nontemporal loads, two register buffers pipeline the next group's
// loads under this group's arithmetic, hidden sits in registers or LDS, a
// butterfly sums the lanes and the epilogue runs on all lanes once per 64
// results.  A row's summation order is fixed by K alone, so its result does
// not depend on M, R or on which other projections share the launch.
#include "glu_grouped.h"
#include "glu_valu.h"

namespace glu {

namespace {

struct RowRef {
    const uint16_t* w;
    int64_t ldw;
    int local;  // row within its projection
};

// the projection that owns virtual row `row` (rows at or past d.rows are never stored)
__device__ __forceinline__ RowRef row_ref(const GroupDesc& d, int row)
{
    RowRef r{d.w[0], d.ldw[0], row};
#pragma unroll
    for (int t = 1; t < kGroupMax; ++t) {
        const bool in = t < d.n && row >= d.row0[t];
        r.w = in ? d.w[t] : r.w;
        r.ldw = in ? d.ldw[t] : r.ldw;
        r.local = in ? row - d.row0[t] : r.local;
    }
    return r;
}

}  // namespace

// hidden [M,K] at row stride ldh (16-byte aligned rows, K % 8 == 0), the
// projections of d.  NB <= 2; NB * U * 64 >= K/8, equality unless RAGGED.
// Dynamic LDS: M * K * 2 bytes when HLDS, else none.
template <int M, int R, int U, int NB, bool HLDS, bool RAGGED>
__global__ void __launch_bounds__(kValuMaxThreads)
grouped_kernel(const uint16_t* __restrict__ hidden, int64_t ldh, int K, GroupDesc d)
{
    static_assert(NB == 1 || NB == 2, "a row group streams in one or two batches");
    constexpr int MR = M * R;
    constexpr int SLOTS = kWave / MR;
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + threadIdx.x / kWave);
    const int nwaves = gridDim.x * wpb;
    const int nchunks = K >> 3;
    const int ldh8 = (int)(ldh >> 3);
    const int rows = d.rows;
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
                    hreg[m][b][i] = h4[m * ldh8 + (RAGGED ? min(c, nchunks - 1) : c)];
                }
            }
        }
    }

    const int ngroups = (rows + R - 1) / R;
    if (wave_id >= ngroups) return;  // no barrier follows
    const int my_groups = (ngroups - 1 - wave_id) / nwaves + 1;
    const int nstages = my_groups * NB;

    auto load = [&](int s, u32x4 (&wv)[R][U]) {
        const int gi = s / NB;
        const int b = s - gi * NB;
        const int g = wave_id + gi * nwaves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const RowRef ref = row_ref(d, min(g * R + r, rows - 1));  // rows past the end re-read the last, never stored
            const u32x4* wp = reinterpret_cast<const u32x4*>(ref.w + (int64_t)ref.local * ref.ldw);
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int c = (b * U + i) * kWave + lane;
                wv[r][i] = ld_nt(wp + (RAGGED ? min(c, nchunks - 1) : c));
            }
        }
    };

    float acc[M][R];
    float res = 0.0f;

    // results of group gi sit in lanes (gi % SLOTS)*MR + m*R + r
    auto flush = [&](int gi_last) {
        const int win0 = gi_last - gi_last % SLOTS;
        if (lane < (gi_last - win0 + 1) * MR) {
            const int gl = lane / MR;
            const int rem = lane - gl * MR;
            const int m = rem / R;
            const int r = rem - m * R;
            const int row = (wave_id + (win0 + gl) * nwaves) * R + r;
            if (row < rows) group_store(d, m, row, f32_to_bf16_rne(res));
        }
    };

    auto accumulate = [&](auto Bc, const u32x4 (&wv)[R][U]) {
        constexpr int B = decltype(Bc)::value;
        const u32x4 z = {0u, 0u, 0u, 0u};
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
                    const u32x4 x = RAGGED ? (ok ? wv[r][i] : z) : wv[r][i];
                    acc[m][r] = dot_chunk(h, x, acc[m][r]);
                }
            }
        }
    };

    auto compute = [&](int s, const u32x4 (&wv)[R][U]) {
        const int gi = s / NB;
        const int b = s - gi * NB;
        if (b == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;
            }
        }
        if constexpr (NB == 1) {
            accumulate(std::integral_constant<int, 0>{}, wv);
        } else {
            if (b == 0) {
                accumulate(std::integral_constant<int, 0>{}, wv);
            } else {
                accumulate(std::integral_constant<int, 1>{}, wv);
            }
        }
        if (b == NB - 1) {
            const int slot = gi % SLOTS;
#pragma unroll
            for (int m = 0; m < M; ++m) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float sum = wave_sum(acc[m][r]);
                    if (lane == slot * MR + m * R + r) res = sum;
                }
            }
            if (slot == SLOTS - 1 || gi == my_groups - 1) flush(gi);
        }
    };

    u32x4 a[R][U], bb[R][U];
    load(0, a);
    int s = 0;
    while (true) {
        if (s + 1 >= nstages) {
            compute(s, a);
            break;
        }
        load(s + 1, bb);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any of this stage's math
        compute(s, a);
        ++s;
        if (s + 1 >= nstages) {
            compute(s, bb);
            break;
        }
        load(s + 1, a);
        __builtin_amdgcn_sched_barrier(0);
        compute(s, bb);
        ++s;
    }
}

// Any alignment (2-byte), any K >= 1, any strides: one wave per virtual row.
template <int M>
__global__ void __launch_bounds__(kGroupedGenericWaves * kWave)
grouped_generic_kernel(const uint16_t* __restrict__ hidden, int64_t ldh, int64_t K, GroupDesc d)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int row = (int)(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave);
    if (row >= d.rows) return;  // whole wave leaves together
    const RowRef ref = row_ref(d, row);
    const uint16_t* wrow = ref.w + (int64_t)ref.local * ref.ldw;
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;
    for (int64_t k = lane; k < K; k += kWave) {
        const float wk = bf16_to_f32(wrow[k]);
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(bf16_to_f32(hidden[m * ldh + k]), wk, acc[m]);
    }
    float res = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float sum = wave_sum(acc[m]);
        if (lane == m) res = sum;
    }
    if (lane < M) group_store(d, lane, row, f32_to_bf16_rne(res));
}

namespace {

using GroupedFn = void (*)(const uint16_t*, int64_t, int, GroupDesc);

template <int M, int R, int U, int NB, bool RAGGED>
constexpr GroupedFn grouped_fn()
{
    return grouped_kernel<M, R, U, NB, valu_hidden_in_lds(M, U, NB), RAGGED>;
}

template <int M, int R, int NB, bool RAGGED>
GroupedFn pick_u(int U)
{
    switch (U) {
    case 1: if constexpr (NB == 1) return grouped_fn<M, R, 1, NB, RAGGED>(); else return nullptr;
    case 2: if constexpr (NB == 1) return grouped_fn<M, R, 2, NB, RAGGED>(); else return nullptr;
    case 3: if constexpr (NB == 1) return grouped_fn<M, R, 3, NB, RAGGED>(); else return nullptr;
    case 4: if constexpr (NB == 1) return grouped_fn<M, R, 4, NB, RAGGED>(); else return nullptr;
    case 5: return grouped_fn<M, R, 5, NB, RAGGED>();
    case 6: return grouped_fn<M, R, 6, NB, RAGGED>();
    case 7: return grouped_fn<M, R, 7, NB, RAGGED>();
    case 8: return grouped_fn<M, R, 8, NB, RAGGED>();
    default: return nullptr;
    }
}

template <int M, int R>
GroupedFn pick_nb(int U, int NB, bool ragged)
{
    if (NB == 1) return ragged ? pick_u<M, R, 1, true>(U) : pick_u<M, R, 1, false>(U);
    if (NB == 2) return ragged ? pick_u<M, R, 2, true>(U) : pick_u<M, R, 2, false>(U);
    return nullptr;
}

template <int M>
GroupedFn pick_r(int R, int U, int NB, bool ragged)
{
    if (R == 1) return pick_nb<M, 1>(U, NB, ragged);
    if (R == 2) return pick_nb<M, 2>(U, NB, ragged);
    return nullptr;
}

GroupedFn pick(const ValuConfig& c)
{
    switch (c.M) {
    case 1: return pick_r<1>(c.R, c.U, c.NB, c.ragged);
    case 2: return pick_r<2>(c.R, c.U, c.NB, c.ragged);
    case 3: return pick_r<3>(c.R, c.U, c.NB, c.ragged);
    case 4: return pick_r<4>(c.R, c.U, c.NB, c.ragged);
    case 5: return c.R == 1 ? pick_nb<5, 1>(c.U, c.NB, c.ragged) : nullptr;
    case 6: return c.R == 1 ? pick_nb<6, 1>(c.U, c.NB, c.ragged) : nullptr;
    case 7: return c.R == 1 ? pick_nb<7, 1>(c.U, c.NB, c.ragged) : nullptr;
    case 8: return c.R == 1 ? pick_nb<8, 1>(c.U, c.NB, c.ragged) : nullptr;
    default: return nullptr;
    }
}

}  // namespace

bool grouped_supported(const ValuConfig& c)
{
    if (c.block < kWave || c.block > kValuMaxThreads || c.block % kWave != 0) return false;
    return pick(c) != nullptr;
}

hipError_t grouped_launch(const ValuConfig& c, const uint16_t* hidden, int64_t ldh, int64_t K, const GroupDesc& d,
                          hipStream_t stream)
{
    GroupedFn fn = pick(c);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = valu_hidden_in_lds(c.M, c.U, c.NB) ? (size_t)c.M * (size_t)K * sizeof(uint16_t) : 0;
    hipLaunchKernelGGL(fn, dim3(c.grid), dim3(c.block), lds, stream, hidden, ldh, (int)K, d);
    return hipGetLastError();
}

hipError_t grouped_generic_launch(int M, const uint16_t* hidden, int64_t ldh, int64_t K, const GroupDesc& d,
                                  hipStream_t stream)
{
    using Fn = void (*)(const uint16_t*, int64_t, int64_t, GroupDesc);
    static const Fn table[8] = {
        grouped_generic_kernel<1>, grouped_generic_kernel<2>, grouped_generic_kernel<3>, grouped_generic_kernel<4>,
        grouped_generic_kernel<5>, grouped_generic_kernel<6>, grouped_generic_kernel<7>, grouped_generic_kernel<8>,
    };
    if (M < 1 || M > 8) return hipErrorInvalidValue;
    const int64_t grid = ((int64_t)d.rows + kGroupedGenericWaves - 1) / kGroupedGenericWaves;
    hipLaunchKernelGGL(table[M - 1], dim3((unsigned)grid), dim3(kGroupedGenericWaves * kWave), 0, stream,
                       hidden, ldh, K, d);
    return hipGetLastError();
}

}  // namespace glu
