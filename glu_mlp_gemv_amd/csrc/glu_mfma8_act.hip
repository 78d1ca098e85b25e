// The backward's g and u step on the forward's slice-major 8-row kernel: the same walk over the
// weights and the same per-lane sums as the forward's M > 8 launches (mfma8_pass_body, so G and U
// are bitwise those of the forward and of the grouped GEMV's K-slice kernel), with the elementwise
// step (glu_act_grad) as the epilogue: one launch writes dg and du at the workspace head.  Its own
// translation unit so that these instantiations compile beside the forward's.
#include "glu_backward.h"
#include "glu_mfma8_pass.h"

namespace glu {

template <int MT8, int U, int JBMAX, bool RAGGED>
__global__ void __launch_bounds__(kMfmaMaxThreads)
mfma8_pass_act_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
                      const uint16_t* __restrict__ up_w, uint16_t* __restrict__ gu, int M, int N, int K,
                      RowStrides ld, int nsg, const uint16_t* __restrict__ dout)
{
    mfma8_pass_body<MT8, U, JBMAX, RAGGED, true>(hidden, gate_w, up_w, gu, M, N, K, ld, nsg, dout);
}

namespace {

using PassActFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int, RowStrides,
                           int, const uint16_t*);

// the forward's tilings: stages of 8 segments up to 32 rows, of 4 above
PassActFn pick_pass_act(int mt8, int U, bool ragged)
{
    if (U == 8) {
        switch (mt8) {
        case 2: return ragged ? mfma8_pass_act_kernel<2, 8, kPassBlocks, true> : mfma8_pass_act_kernel<2, 8, kPassBlocks, false>;
        case 3: return ragged ? mfma8_pass_act_kernel<3, 8, kPassBlocks, true> : mfma8_pass_act_kernel<3, 8, kPassBlocks, false>;
        case 4: return ragged ? mfma8_pass_act_kernel<4, 8, kPassBlocks, true> : mfma8_pass_act_kernel<4, 8, kPassBlocks, false>;
        default: return nullptr;
        }
    }
    if (U == 4) {
        switch (mt8) {
        case 5: return ragged ? mfma8_pass_act_kernel<5, 4, kPassBlocks, true> : mfma8_pass_act_kernel<5, 4, kPassBlocks, false>;
        case 6: return ragged ? mfma8_pass_act_kernel<6, 4, kPassBlocks, true> : mfma8_pass_act_kernel<6, 4, kPassBlocks, false>;
        case 7: return ragged ? mfma8_pass_act_kernel<7, 4, kPassBlocks, true> : mfma8_pass_act_kernel<7, 4, kPassBlocks, false>;
        case 8: return ragged ? mfma8_pass_act_kernel<8, 4, kPassBlocks, true> : mfma8_pass_act_kernel<8, 4, kPassBlocks, false>;
        default: return nullptr;
        }
    }
    return nullptr;
}

}  // namespace

hipError_t mfma8_act_launch(int M, int U, int nsg, bool ragged, int grid, const uint16_t* hidden,
                            const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* dout, uint16_t* gu,
                            int64_t N, int64_t K, hipStream_t stream)
{
    const int mt8 = pass_tiles(M, U);
    PassActFn fp = nullptr;
    if ((int64_t)grid * kPassBlocks >= mfma8_blocks(N)) fp = pick_pass_act(mt8, U, ragged);
    if (!fp || M < 1 || M > 8 * mt8 || N < 1 || K < 8 || (K & 7) != 0) return hipErrorInvalidValue;
    // dense operands: hidden [M][K], the weights [N][K], dout and both halves of gu [M][N]
    const RowStrides ld{K, K, K, N};
    hipLaunchKernelGGL(fp, dim3(grid), dim3(kMfmaMaxThreads), mfma8_slice_lds_bytes(mt8, U), stream, hidden, gate_w,
                       up_w, gu, M, (int)N, (int)K, ld, nsg, dout);
    return hipGetLastError();
}

}  // namespace glu
