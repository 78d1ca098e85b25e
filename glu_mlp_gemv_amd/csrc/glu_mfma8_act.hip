// The backward's g and u step on the forward's slice-major 8-row kernel: the same walk over the
// weights and the same per-lane sums as the forward's M > 8 launches (mfma8_pass_kernel, so G and U
// are bitwise those of the forward and of the grouped GEMV's K-slice kernel), with the elementwise
// step (glu_act_grad) as the epilogue: one launch writes dg and du at the workspace head.  Its own
// translation unit so that these instantiations compile beside the forward's.
#include "glu_backward.h"
#include "glu_mfma8_pass.h"

namespace glu {

hipError_t mfma8_act_launch(int M, int U, int nsg, bool ragged, int grid, const uint16_t* hidden,
                            const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* dout, uint16_t* gu,
                            int64_t N, int64_t K, hipStream_t stream)
{
    const int mt8 = pass_tiles(M, U);
    Mfma8PassFn fp = nullptr;
    if ((int64_t)grid * kPassBlocks >= mfma8_blocks(N)) fp = pick_pass<true>(mt8, U, ragged);
    if (!fp || M < 1 || M > 8 * mt8 || N < 1 || K < 8 || (K & 7) != 0) return hipErrorInvalidValue;
    // dense operands: hidden [M][K], the weights [N][K], dout and both halves of gu [M][N]
    const RowStrides ld{K, K, K, N};
    hipLaunchKernelGGL(fp, dim3(grid), dim3(kMfmaMaxThreads), mfma8_slice_lds_bytes(mt8, U), stream, hidden, gate_w,
                       up_w, gu, M, (int)N, (int)K, ld, nsg, dout);
    return hipGetLastError();
}

}  // namespace glu
