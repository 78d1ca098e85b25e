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

// VALU grouped GEMV (M <= 8 rows of hidden per launch; R is 1 or 2, and 1 above M = 4)
bool grouped_supported(const ValuConfig& c);
hipError_t grouped_launch(const ValuConfig& c, const uint16_t* hidden, int64_t ldh, int64_t K, const GroupDesc& d,
                          hipStream_t stream);
// any layout, M <= 8
hipError_t grouped_generic_launch(int M, const uint16_t* hidden, int64_t ldh, int64_t K, const GroupDesc& d,
                                  hipStream_t stream);

}  // namespace glu
