// Unit ceilings (glu_ceiling.hip): issue-rate yardsticks of one unit of a compute unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glu {

// unit 1 = MFMA 16x16x32 bf16, 2 = MFMA 32x32x16 bf16, 3 = LDS ds_read_b128; `cus` workgroups
// of `waves` waves, each repeating its body `iters` times
hipError_t unit_ceiling_launch(int unit, int cus, int waves, int64_t iters, uint32_t* sink, hipStream_t stream);

}  // namespace glu
