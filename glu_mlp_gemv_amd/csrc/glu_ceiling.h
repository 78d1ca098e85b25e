// Yardsticks of glu_ceiling.hip beyond the read ceiling: unit issue rates and the read/write copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glu {

// unit 1 = MFMA 16x16x32 bf16, 2 = MFMA 32x32x16 bf16, 3 = LDS ds_read_b128; `cus` workgroups
// of `waves` waves, each repeating its body `iters` times
hipError_t unit_ceiling_launch(int unit, int cus, int waves, int64_t iters, uint32_t* sink, hipStream_t stream);

// copy ceiling: a -> ca and b -> cb, [rows][U KiB], in the read ceiling's launch shape (R rows per
// wave: 1 or 2)
bool copy_ceiling_supported(int U, int R);
hipError_t copy_ceiling_launch(const void* a, const void* b, void* ca, void* cb, int rows, int U, int R, int grid,
                               int block, hipStream_t stream);

}  // namespace glu
