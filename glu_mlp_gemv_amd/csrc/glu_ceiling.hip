// Streaming-read ceiling: the HBM access of the M = 1 VALU GEMV with its
// arithmetic taken out, as a yardstick for what that kernel can reach.
//
// The decode projection is bound by reading both weight matrices once (DeepSpeed
// PR #8602, comment "Plan B: Dual-Weight GEMV", section on why library-level
// bandwidth is reachable at batch 1, which puts the remaining gap down to launch
// overhead and the access pattern).  This kernel reads two [rows, row_bytes]
// matrices exactly as valu_kernel reads gate_w and up_w: persistent waves own the
// row groups w, w+W, ... of R rows, lane l loads the 16-byte chunks l, l+64, ...
// of every row with nontemporal global_load_dwordx4, and two register buffers
// keep the next group's loads in flight while the current group is consumed.
// Consuming a group is an XOR of its words into one register; a store that
// depends on that register (taken only for one 32-bit value) keeps the loads
// alive.  Whatever time separates the GEMV from this kernel at the same launch
// shape is arithmetic, reduction and epilogue; whatever separates this kernel
// from the bytes at peak bandwidth is the memory system and the launch.
#include "glu_ceiling.h"
#include "glu_launch.h"
#include "glu_mfma_common.h"

namespace glu {

namespace {

typedef unsigned u32x4c __attribute__((ext_vector_type(4)));

constexpr uint32_t kSinkMagic = 0x7f3a5c91u;  // the store happens only if the XOR equals this

// Workgroup order.  The dispatcher deals consecutive workgroups to the 8 XCDs in
// turn, so by default the workgroups one XCD runs are spread over the whole row
// space.  With xcd_bands, workgroup b takes the logical index (b % 8) * (G / 8) +
// b / 8 (G a multiple of 8): each XCD streams one contiguous band of rows.
__device__ __forceinline__ int logical_block(bool xcd_bands)
{
    const int b = blockIdx.x, G = gridDim.x;
    return xcd_bands ? (b % kXcds) * (G / kXcds) + b / kXcds : b;
}

// rows of both matrices [rows, U * 1024 bytes], 16-byte aligned; sink: 64 words
template <int U, int R>
__global__ void __launch_bounds__(kValuMaxThreads)
read_ceiling_kernel(const u32x4c* __restrict__ a, const u32x4c* __restrict__ b, int rows, uint32_t* sink,
                    bool xcd_bands)
{
    constexpr int CPR = U * kWave;  // 16-byte chunks per row
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int wave_id = __builtin_amdgcn_readfirstlane(logical_block(xcd_bands) * wpb + threadIdx.x / kWave);
    const int nwaves = gridDim.x * wpb;
    const int ngroups = (rows + R - 1) / R;
    if (wave_id >= ngroups) return;
    const int nsteps = (ngroups - 1 - wave_id) / nwaves + 1;

    auto load = [&](int s, u32x4c (&x)[R][U], u32x4c (&y)[R][U]) {
        const int g = wave_id + s * nwaves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(g * R + r, rows - 1);
            const u32x4c* pa = a + (int64_t)row * CPR + lane;
            const u32x4c* pb = b + (int64_t)row * CPR + lane;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                x[r][i] = __builtin_nontemporal_load(pa + i * kWave);
                y[r][i] = __builtin_nontemporal_load(pb + i * kWave);
            }
        }
    };
    uint32_t acc = 0;
    auto consume = [&](const u32x4c (&x)[R][U], const u32x4c (&y)[R][U]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const u32x4c v = x[r][i] ^ y[r][i];
                acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
            }
        }
    };

    u32x4c xa[R][U], ya[R][U], xb[R][U], yb[R][U];
    load(0, xa, ya);
    int s = 0;
    while (true) {
        if (s + 1 >= nsteps) {
            consume(xa, ya);
            break;
        }
        load(s + 1, xb, yb);
        __builtin_amdgcn_sched_barrier(0);
        consume(xa, ya);
        ++s;
        if (s + 1 >= nsteps) {
            consume(xb, yb);
            break;
        }
        load(s + 1, xa, ya);
        __builtin_amdgcn_sched_barrier(0);
        consume(xb, yb);
        ++s;
    }
    if (acc == kSinkMagic) sink[lane] = acc;
}

// Unit ceilings: one workgroup of `waves` waves per compute unit repeats a body that
// exercises a single unit of the CU and nothing else, so that time per body is that
// unit's issue rate.  MFMA bodies keep 8 (16x16x32) or 4 (32x32x16) accumulators
// that no other instruction touches; operands are fixed registers holding finite
// bf16 values.  The LDS body reads 16 KiB per wave (16 ds_read_b128 of 1 KiB,
// lane l at byte 16 l of a 1 KiB row chosen from the iteration, conflict-free)
// from a 64 KiB array and folds the words by XOR.  Like the read ceiling, the
// single store happens only if the folded value equals kSinkMagic.
typedef float f32x16c __attribute__((ext_vector_type(16)));

template <int UNIT>
__global__ void __launch_bounds__(1024)
unit_ceiling_kernel(int64_t iters, uint32_t* sink)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    uint32_t acc = 0;
    if constexpr (UNIT == 1 || UNIT == 2) {
        const u32x4c a = u32x4c{0x3f803f80u ^ (uint32_t)lane, 0x3e003e00u, 0x3d803d80u, 0x3c003c00u + (uint32_t)wave};
        const u32x4c b = u32x4c{0x3c003c00u, 0x3f003f00u ^ (uint32_t)lane, 0x3e803e80u, 0x3b803b80u};
        const bf16x8_t ab = __builtin_bit_cast(bf16x8_t, a), bb = __builtin_bit_cast(bf16x8_t, b);
        if constexpr (UNIT == 1) {
            f32x4_t d[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) d[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
                for (int i = 0; i < 8; ++i) d[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, d[i], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc ^= __builtin_bit_cast(uint32_t, d[i][0] + d[i][3]);
        } else {
            f32x16c d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = f32x16c{};
            for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
                for (int i = 0; i < 4; ++i) d[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, d[i], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) acc ^= __builtin_bit_cast(uint32_t, d[i][0] + d[i][15]);
        }
    } else {
        __shared__ u32x4c L[4096];  // 64 KiB
        for (int i = threadIdx.x; i < 4096; i += blockDim.x) L[i] = u32x4c{(uint32_t)i, 1u, 2u, 3u};
        __syncthreads();
        u32x4c x = {0u, 0u, 0u, 0u};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x ^= L[lane + kWave * (((int)it + 5 * r + 3 * wave) & 63)];
        }
        acc = x[0] ^ x[1] ^ x[2] ^ x[3];
    }
    if (acc == kSinkMagic) sink[lane] = acc;
}

// Copy ceiling: the same streaming pattern reading a and b and writing them to ca and cb with
// nontemporal 16-byte stores, the read/write yardstick for the backward's one-pass kernels (which
// read both weight matrices once and write both weight gradients once).  Rows of groups the wave
// does not own are never touched; the padded rows of a last group re-read row rows-1 and skip
// their stores.
template <int U, int R>
__global__ void __launch_bounds__(kValuMaxThreads)
copy_ceiling_kernel(const u32x4c* __restrict__ a, const u32x4c* __restrict__ b, u32x4c* __restrict__ ca,
                    u32x4c* __restrict__ cb, int rows)
{
    constexpr int CPR = U * kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + threadIdx.x / kWave);
    const int nwaves = gridDim.x * wpb;
    const int ngroups = (rows + R - 1) / R;
    for (int g = wave_id; g < ngroups; g += nwaves) {
        u32x4c x[R][U], y[R][U];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(g * R + r, rows - 1);
#pragma unroll
            for (int i = 0; i < U; ++i) {
                x[r][i] = __builtin_nontemporal_load(a + (int64_t)row * CPR + lane + i * kWave);
                y[r][i] = __builtin_nontemporal_load(b + (int64_t)row * CPR + lane + i * kWave);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = g * R + r;
            if (row < rows) {
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    __builtin_nontemporal_store(x[r][i], ca + (int64_t)row * CPR + lane + i * kWave);
                    __builtin_nontemporal_store(y[r][i], cb + (int64_t)row * CPR + lane + i * kWave);
                }
            }
        }
    }
}

using CopyFn = void (*)(const u32x4c*, const u32x4c*, u32x4c*, u32x4c*, int);

template <int R>
CopyFn pick_copy_u(int U)
{
    switch (U) {
    case 1: return copy_ceiling_kernel<1, R>;
    case 2: return copy_ceiling_kernel<2, R>;
    case 3: return copy_ceiling_kernel<3, R>;
    case 4: return copy_ceiling_kernel<4, R>;
    case 5: return copy_ceiling_kernel<5, R>;
    case 6: return copy_ceiling_kernel<6, R>;
    case 7: return copy_ceiling_kernel<7, R>;
    case 8: return copy_ceiling_kernel<8, R>;
    default: return nullptr;
    }
}

CopyFn pick_copy(int U, int R)
{
    switch (R) {
    case 1: return pick_copy_u<1>(U);
    case 2: return pick_copy_u<2>(U);
    default: return nullptr;
    }
}

using CeilingFn = void (*)(const u32x4c*, const u32x4c*, int, uint32_t*, bool);

template <int R>
CeilingFn pick_u(int U)
{
    switch (U) {
    case 1: return read_ceiling_kernel<1, R>;
    case 2: return read_ceiling_kernel<2, R>;
    case 3: return read_ceiling_kernel<3, R>;
    case 4: return read_ceiling_kernel<4, R>;
    case 5: return read_ceiling_kernel<5, R>;
    case 6: return read_ceiling_kernel<6, R>;
    case 7: return read_ceiling_kernel<7, R>;
    case 8: return read_ceiling_kernel<8, R>;
    default: return nullptr;
    }
}

CeilingFn pick(int U, int R)
{
    switch (R) {
    case 1: return pick_u<1>(U);
    case 2: return pick_u<2>(U);
    case 4: return pick_u<4>(U);
    default: return nullptr;
    }
}

}  // namespace

bool read_ceiling_supported(int U, int R) { return pick(U, R) != nullptr; }

hipError_t read_ceiling_launch(const void* a, const void* b, int rows, int U, int R, int grid, int block,
                               bool xcd_bands, uint32_t* sink, hipStream_t stream)
{
    CeilingFn fn = pick(U, R);
    if (!fn || (xcd_bands && grid % kXcds != 0)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(block), 0, stream, static_cast<const u32x4c*>(a),
                       static_cast<const u32x4c*>(b), rows, sink, xcd_bands);
    return hipGetLastError();
}

bool copy_ceiling_supported(int U, int R) { return pick_copy(U, R) != nullptr; }

hipError_t copy_ceiling_launch(const void* a, const void* b, void* ca, void* cb, int rows, int U, int R, int grid,
                               int block, hipStream_t stream)
{
    CopyFn fn = pick_copy(U, R);
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(block), 0, stream, static_cast<const u32x4c*>(a),
                       static_cast<const u32x4c*>(b), static_cast<u32x4c*>(ca), static_cast<u32x4c*>(cb), rows);
    return hipGetLastError();
}

hipError_t unit_ceiling_launch(int unit, int cus, int waves, int64_t iters, uint32_t* sink, hipStream_t stream)
{
    void (*fn)(int64_t, uint32_t*) = unit == 1 ? unit_ceiling_kernel<1> : unit == 2 ? unit_ceiling_kernel<2>
                                   : unit == 3 ? unit_ceiling_kernel<3> : nullptr;
    if (!fn || cus < 1 || waves < 1 || waves * kWave > 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(cus), dim3(waves * kWave), 0, stream, iters, sink);
    return hipGetLastError();
}

}  // namespace glu
