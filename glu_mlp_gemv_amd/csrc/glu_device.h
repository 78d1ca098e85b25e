// Device helpers of the GLU kernels: bf16 widening and rounding, the
// rounding epilogue, and wave64 reductions.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glu_launch.h"

namespace glu {

// ---- bf16 <-> fp32 --------------------------------------------------------

// bf16 bits in the low or high half of a dword, widened exactly to fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest with ties to even; NaN stays a quiet NaN,
// magnitudes that round past the largest finite bf16 become infinity.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---- the rounding epilogue -------------------------------------------------
//
// DeepSpeed PR #9057 ("preserve HF precision boundaries in segKI kernels",
// section "Changes") keeps the bf16 roundings of a Hugging Face bf16 MLP:
// gate and up are bf16 tensors, the activation silu(gate) is a bf16 tensor,
// and the output is their product rounded to bf16.  silu is evaluated as
// g / (1 + exp(-g)) with each operation rounded to fp32.  Each fp32 step is
// computed here in fp64 and rounded once to fp32: for +, * and / of fp32
// operands this double rounding is innocuous (53 >= 2*24 + 2 bits), so the
// results are the IEEE fp32 results whatever the fp32 division and denormal
// modes are; exp is the fp64 library exp rounded to fp32 (the correctly
// rounded fp32 value except in vanishingly rare near-midpoint cases).
__device__ __forceinline__ uint16_t glu_epilogue(float gate_acc, float up_acc)
{
    const float g = bf16_to_f32(f32_to_bf16_rne(gate_acc));
    const float u = bf16_to_f32(f32_to_bf16_rne(up_acc));
    const float e = (float)exp(-(double)g);
    const float d = (float)(1.0 + (double)e);
    const float s32 = (float)((double)g / (double)d);
    const float s = bf16_to_f32(f32_to_bf16_rne(s32));
    const float p = (float)((double)s * (double)u);
    return f32_to_bf16_rne(p);
}

// ---- wave64 reduction --------------------------------------------------------
//
// Butterfly sum over the 64 lanes; every lane ends with the same value (each
// step adds a lane's value and its partner's, and fp32 addition commutes), so
// the result does not depend on which lane reads it.  Order of levels: lane
// bit 0, bit 1 (DPP quad permutations), bit 2 (row half mirror), bit 3 (row
// mirror), bit 4 (ds_swizzle swap of 16-lane groups), bit 5 (permlane32 swap).

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x)
{
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float x)
{
    x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
    x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
    x = dpp_add<0x141>(x);  // row_half_mirror: the other quad of 8
    x = dpp_add<0x140>(x);  // row_mirror: the other half of 16
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // lane ^ 16
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);  // lanes i and i^32, same order in all
}

}  // namespace glu
