// Fallback kernels: the dual GLU projection for inputs the fast paths do not
// take (pointers only 2-byte aligned, K or a row stride not a multiple of 8,
// strides above 2^25), and the K == 0 case.  Same arithmetic contract (fp32 sums, rounding epilogue), with
// 2-byte loads: correct for any layout, not tuned.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {

constexpr int kGenericMaxM = 8;
constexpr int kGenericWaves = 4;

// One wave per output row j; lane l sums k = l, l+64, ... for every hidden row.
template <int M>
__global__ void __launch_bounds__(kGenericWaves * kWave)
generic_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
               const uint16_t* __restrict__ up_w, uint16_t* __restrict__ out,
               int64_t N, int64_t K, RowStrides ld)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t j = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (j >= N) return;  // whole wave leaves together
    const uint16_t* grow = gate_w + j * ld.g;
    const uint16_t* urow = up_w + j * ld.u;
    float ag[M], au[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        ag[m] = 0.0f;
        au[m] = 0.0f;
    }
    for (int64_t k = lane; k < K; k += kWave) {
        const float wgk = bf16_to_f32(grow[k]);
        const float wuk = bf16_to_f32(urow[k]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float hk = bf16_to_f32(hidden[m * ld.h + k]);
            ag[m] = __builtin_fmaf(hk, wgk, ag[m]);
            au[m] = __builtin_fmaf(hk, wuk, au[m]);
        }
    }
    float G = 0.0f, U = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float gs = wave_sum(ag[m]);
        const float us = wave_sum(au[m]);
        if (lane == m) {
            G = gs;
            U = us;
        }
    }
    if (lane < M) {
        out[(int64_t)lane * ld.o + j] = glu_epilogue(G, U);
    }
}

__global__ void zero_kernel(uint16_t* __restrict__ out, int64_t count, int64_t N, int64_t ldo)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const int64_t m = i / N;
        out[m * ldo + (i - m * N)] = 0;
    }
}

hipError_t generic_launch(int M, const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                          uint16_t* out, int64_t N, int64_t K, RowStrides ld, hipStream_t stream)
{
    using Fn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int64_t, int64_t, RowStrides);
    static const Fn table[kGenericMaxM] = {
        generic_kernel<1>, generic_kernel<2>, generic_kernel<3>, generic_kernel<4>,
        generic_kernel<5>, generic_kernel<6>, generic_kernel<7>, generic_kernel<8>,
    };
    if (M < 1 || M > kGenericMaxM) return hipErrorInvalidValue;
    const int64_t grid = (N + kGenericWaves - 1) / kGenericWaves;
    hipLaunchKernelGGL(table[M - 1], dim3((unsigned)grid), dim3(kGenericWaves * kWave), 0, stream,
                       hidden, gate_w, up_w, out, N, K, ld);
    return hipGetLastError();
}

hipError_t zero_launch(uint16_t* out, int64_t M, int64_t N, int64_t ldo, hipStream_t stream)
{
    const int64_t count = M * N;
    int64_t grid = (count + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream, out, count, N, ldo);
    return hipGetLastError();
}

}  // namespace glu
