// Internal launch interface of the grouped GEMV (glu_grouped.hip).
#pragma once

#include "glu_launch.h"

namespace glu {

constexpr int kGroupMax = 8;            // projections in one call
constexpr int kGroupedGenericWaves = 4;

// The projections of one launch as a virtual row space: projection t owns
// rows [row0[t], row0[t] + N_t) (row0[0] = 0, row0[n] = rows); its weight row
// j is at w[t] + j*ldw[t] and its output row m at out[t] + m*ldo[t].  Passed
// by value as a kernel argument.
struct GroupDesc {
    const uint16_t* w[kGroupMax];
    uint16_t* out[kGroupMax];
    int64_t ldw[kGroupMax];
    int64_t ldo[kGroupMax];
    int row0[kGroupMax + 1];
    int n;
    int rows;
};

// out of virtual row `row`, hidden row m
__device__ __forceinline__ void group_store(const GroupDesc& d, int m, int row, uint16_t v)
{
    uint16_t* o = d.out[0];
    int64_t ldo = d.ldo[0];
    int local = row;
#pragma unroll
    for (int t = 1; t < kGroupMax; ++t) {
        const bool in = t < d.n && row >= d.row0[t];
        o = in ? d.out[t] : o;
        ldo = in ? d.ldo[t] : ldo;
        local = in ? row - d.row0[t] : local;
    }
    o[(int64_t)m * ldo + local] = v;
}

// VALU grouped GEMV (M <= 8 rows of hidden per launch; R is 1 or 2, and 1 above M = 4)
bool grouped_supported(const ValuConfig& c);
hipError_t grouped_launch(const ValuConfig& c, const uint16_t* hidden, int64_t ldh, int64_t K, const GroupDesc& d,
                          hipStream_t stream);
// any layout, M <= 8
hipError_t grouped_generic_launch(int M, const uint16_t* hidden, int64_t ldh, int64_t K, const GroupDesc& d,
                                  hipStream_t stream);
// block-diagonal MFMA grouped GEMV (glu_grouped_mfma.hip): every projection's
// row count a multiple of 4, M <= 32 per launch, hidden in LDS or read from L2
bool grouped_mfma_supported(const MfmaConfig& c);
hipError_t grouped_mfma_launch(const MfmaConfig& c, int M, const uint16_t* hidden, int64_t ldh, int64_t K,
                               const GroupDesc& d, hipStream_t stream);

}  // namespace glu
