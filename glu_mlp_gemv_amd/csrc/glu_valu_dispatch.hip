// Launch of the VALU GEMV: picks the instantiation for a configuration.
#include "glu_launch.h"

namespace glu {

namespace {

ValuFn pick(const ValuConfig& c)
{
    if (c.diag && c.M != 1) return nullptr;
    switch (c.M) {
    case 1: return valu_pick_1(c.R, c.U, c.NB, c.ragged, c.diag);
    case 2: return valu_pick_2(c.R, c.U, c.NB, c.ragged);
    case 3: return valu_pick_3(c.R, c.U, c.NB, c.ragged);
    case 4: return valu_pick_4(c.R, c.U, c.NB, c.ragged);
    case 5: return valu_pick_5(c.R, c.U, c.NB, c.ragged);
    case 6: return valu_pick_6(c.R, c.U, c.NB, c.ragged);
    case 7: return valu_pick_7(c.R, c.U, c.NB, c.ragged);
    case 8: return valu_pick_8(c.R, c.U, c.NB, c.ragged);
    default: return nullptr;
    }
}

}  // namespace

bool valu_supported(const ValuConfig& c)
{
    if (c.block < kWave || c.block > (c.diag ? kMfmaMaxThreads : kValuMaxThreads) || c.block % kWave != 0) return false;
    return pick(c) != nullptr;
}

hipError_t valu_launch(const ValuConfig& c, const uint16_t* hidden, const uint16_t* gate_w,
                       const uint16_t* up_w, uint16_t* out, int64_t N, int64_t K, RowStrides ld,
                       hipStream_t stream)
{
    ValuFn fn = pick(c);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = valu_hidden_in_lds(c.M, c.U, c.NB) ? (size_t)c.M * (size_t)K * sizeof(uint16_t) : 0;
    hipLaunchKernelGGL(fn, dim3(c.grid), dim3(c.block), lds, stream,
                       hidden, gate_w, up_w, out, (int)N, (int)K, ld);
    return hipGetLastError();
}

}  // namespace glu
