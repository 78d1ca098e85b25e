// The backward's g and u step for 2 <= M <= 16 on the forward's 4-row MFMA kernel with hidden in LDS:
// the same walk over the weights and the same per-lane sums as the forward's launch for (M, N, K)
// (mfma_body), with the elementwise step (glu_act_grad) as the epilogue: one launch writes dg and
// du at the workspace head.  Its own translation unit so that these instantiations compile beside
// the forward's.
#include "glu_backward.h"
#include "glu_mfma4.h"

namespace glu {

template <int MT4, int U, bool RAGGED>
__global__ void __launch_bounds__(kMfmaMaxThreads)
mfma_act_kernel(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ gate_w,
                const uint16_t* __restrict__ up_w, uint16_t* __restrict__ gu, int M, int N, int K, RowStrides ld,
                int nsg, const uint16_t* __restrict__ dout)
{
    mfma_body<MT4, U, true, RAGGED, true>(hidden, gate_w, up_w, gu, M, N, K, ld, nsg, dout);
}

namespace {

using MfmaActFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int, RowStrides,
                           int, const uint16_t*);

template <int MT4, bool RG>
MfmaActFn pick_act_u(int U)
{
    switch (U) {
    case 2: return mfma_act_kernel<MT4, 2, RG>;
    case 4: return mfma_act_kernel<MT4, 4, RG>;
    case 5: return mfma_act_kernel<MT4, 5, RG>;
    case 8: return mfma_act_kernel<MT4, 8, RG>;
    default: return nullptr;
    }
}

}  // namespace

bool mfma_act_supported(const MfmaConfig& c, int M)
{
    return c.rows == 4 && c.hidden == kHiddenLds && M >= 1 && M <= kMfmaActMaxM &&
           (c.U == 2 || c.U == 4 || c.U == 5 || c.U == 8);
}

hipError_t mfma_act_launch(const MfmaConfig& c, int M, const uint16_t* hidden, const uint16_t* gate_w,
                           const uint16_t* up_w, const uint16_t* dout, uint16_t* gu, int64_t N, int64_t K,
                           hipStream_t stream)
{
    if (!mfma_act_supported(c, M) || N < 1 || K < 8 || (K & 7) != 0 || c.grid < 1 || c.block < kWave ||
        c.block > kMfmaMaxThreads || c.block % kWave != 0) {
        return hipErrorInvalidValue;
    }
    MfmaActFn fn = nullptr;
    switch ((M + 3) / 4) {
    case 1: fn = c.ragged ? pick_act_u<1, true>(c.U) : pick_act_u<1, false>(c.U); break;
    case 2: fn = c.ragged ? pick_act_u<2, true>(c.U) : pick_act_u<2, false>(c.U); break;
    case 3: fn = c.ragged ? pick_act_u<3, true>(c.U) : pick_act_u<3, false>(c.U); break;
    case 4: fn = c.ragged ? pick_act_u<4, true>(c.U) : pick_act_u<4, false>(c.U); break;
    default: break;
    }
    if (!fn) return hipErrorInvalidValue;
    // dense operands: hidden [M][K], the weights [N][K], dout and both halves of gu [M][N]
    const RowStrides ld{K, K, K, N};
    hipLaunchKernelGGL(fn, dim3(c.grid), dim3(c.block), mfma_hidden_lds_bytes(M, K), stream, hidden, gate_w, up_w, gu,
                       M, (int)N, (int)K, ld, c.nsg, dout);
    return hipGetLastError();
}

}  // namespace glu
